// gfx950 (MI355X) kernels of the Longformer window + global attention forward.
//
// Three kernels, all launched on the caller's stream:
//   band_kernel        window keys of every non-global row, with the global keys
//                      outside the window folded into the same online softmax;
//   global_rows_kernel split-key partials (max, sum, unnormalised output) of the
//                      global rows over every unpadded key;
//   merge_kernel       log-sum-exp merge of those partials, global rows written.
//
// The key set of a query is the union of its dilated window and the global keys
// (page "基于自注意力机制的长文本建模算法：Longformer详解" §2 and §4); global rows see
// every key and every row sees the global keys (page "基于Block-Sparse Attention的
// Longformer" §2, §4).  The window band is a dense contraction per tile, so both
// products (S = K Q^T and O^T = V^T P^T) run on the matrix cores, bf16 inputs
// with fp32 accumulation (fp32 MFMA for fp32 inputs).  Softmax statistics are fp32.
//
// Dilation: rows i = r, r+dil, r+2*dil, ... of residue class r attend exactly to the
// keys of the same class within w steps, so each class is a plain band over a
// strided gather ("virtual" index i' with i = r + i'*dil).  Global keys ignore the
// lattice and are folded with an in-window test that keeps each key counted once.
//
// Register layout (v_mfma_f32_32x32x*): accumulator element i of lane l sits at
// row 8*(i/4) + 4*(l/32) + (i%4), column l%32.  Scores are computed transposed
// (rows = keys, columns = queries) so each lane owns one query: its row statistics
// need one exchange with the lane 32 away, and its 16 score values feed the P^T
// operand of the next product unchanged.  K rows are read in the order sigma(M) so
// that accumulator element i of lane-half h2 holds key 16*(i/8) + 8*h2 + (i%8); the
// output dimension is read in the order pi(M) so each lane ends up holding 16
// consecutive output columns.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lf_attn_internal.h"

namespace lf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// exp(x / sqrt(64)) = exp2(x * log2(e) / 8)
constexpr float kScaleLog2 = 1.4426950408889634f * 0.125f;
constexpr float kNegInf = -__builtin_inff();
constexpr int kStageKeys = kKeysPerTile;  // 64
constexpr int kNoPos = -(1 << 29);        // virtual position that is in no window

__device__ __forceinline__ int sigma(int M) {  // K row read by lane row M
    const int q = M >> 3, hh = (M >> 2) & 1, c = M & 3;
    return 16 * (q >> 1) + 8 * hh + 4 * (q & 1) + c;
}
__device__ __forceinline__ int pi_col(int M) {  // output column read by lane row M
    const int q = M >> 3, hh = (M >> 2) & 1, c = M & 3;
    return 16 * hh + 4 * q + c;
}
__device__ __forceinline__ int key_local(int i, int h2) { return 16 * (i >> 3) + 8 * h2 + (i & 7); }

// LDS swizzles of 16-byte chunks (bank-conflict-free 128-bit reads of the lane
// patterns above: every 8 consecutive lanes hit 8 distinct chunks).
__device__ __forceinline__ int swz_k(int row) { return (row & 3) | ((row >> 1) & 4); }
__device__ __forceinline__ int swz_v(int d) { return (d & 3) | ((d >> 2) & 4); }

// Lanes l and l^32 hold the two halves of one query's keys.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Work-groups are dispatched round-robin over the 8 XCDs; hand each XCD a
// contiguous range of logical ids so that neighbouring row tiles of one (b, h),
// which read overlapping K/V spans, share one L2.
__device__ __forceinline__ int xcd_remap(int pid, int n) {
    constexpr int X = 8;
    const int per = (n + X - 1) / X;
    int tall = n % X;
    if (tall == 0) tall = X;
    const int xcd = pid % X, local = pid / X;
    return xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
}

// ---------------------------------------------------------------------------
// Element-type traits: operand loads, K/V staging and the two products.
// A stage holds 64 keys: K row-major (64 x 64), and V row-major (fp32) or
// transposed V^T (bf16: the P^T.V contraction wants 8 consecutive keys per lane).

struct Bf16 {
    using Elem = uint16_t;
    static constexpr int kKBytes = kStageKeys * 128;   // 8 KiB
    static constexpr int kStageBytes = 2 * kKBytes;    // K + V^T
    struct QOp { bf16x8 v[4]; };
    struct Regs { u32x4 k[2]; u32x4 v[2]; };
    struct PFrag { bf16x8 v[2]; };

    // Round the weights to bf16 (the P^T operand) and return their sum as rounded,
    // so the normaliser matches the weights the product uses.
    __device__ static float make_p(const float* p, PFrag& pf) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        float sum = 0.f;
        for (int kb = 0; kb < 2; ++kb) {
            f32x8 t;
            for (int j = 0; j < 8; ++j) t[j] = p[8 * kb + j];
            const bf16x8 b = __builtin_convertvector(t, bf16x8);
            pf.v[kb] = b;
            // Sub-vectors by shuffle: hipcc mis-selects dot2 operands taken as words of
            // a bit-cast of the converted vector (every word reads as the first).
            sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 0, 1), one, sum, false);
            sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 2, 3), one, sum, false);
            sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 4, 5), one, sum, false);
            sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(b, b, 6, 7), one, sum, false);
        }
        return sum;
    }

    // B operand of S^T = K Q^T: lane (query, h2) holds d = 16*kb + 8*h2 + j.
    __device__ static void load_q(QOp& q, const Elem* row, int h2) {
        for (int kb = 0; kb < 4; ++kb) {
            u32x4 x = row ? *reinterpret_cast<const u32x4*>(row + 16 * kb + 8 * h2) : u32x4{0, 0, 0, 0};
            q.v[kb] = __builtin_bit_cast(bf16x8, x);
        }
    }

    // Global -> registers.  row_of(kk) gives the source row of stage key kk, or -1
    // (zero fill: padded, out of range or unused slot).
    template <class RowOf>
    __device__ static void load(Regs& r, const Elem* K, const Elem* V, RowOf row_of, int tid) {
        for (int u = 0; u < 2; ++u) {
            const int c = tid + kThreads * u, kk = c >> 3, col = c & 7;
            const int row = row_of(kk);
            r.k[u] = row >= 0 ? *reinterpret_cast<const u32x4*>(K + (size_t)row * 64 + col * 8) : u32x4{0, 0, 0, 0};
        }
        const int kk = tid & 63;
        const int row = row_of(kk);
        for (int u = 0; u < 2; ++u) {
            const int dc = (tid >> 6) + 4 * u;
            r.v[u] = row >= 0 ? *reinterpret_cast<const u32x4*>(V + (size_t)row * 64 + dc * 8) : u32x4{0, 0, 0, 0};
        }
    }

    __device__ static void store(char* stage, const Regs& r, int tid) {
        char* Ks = stage;
        char* Vt = stage + kKBytes;
        for (int u = 0; u < 2; ++u) {
            const int c = tid + kThreads * u, kk = c >> 3, col = c & 7;
            *reinterpret_cast<u32x4*>(Ks + kk * 128 + ((col ^ swz_k(kk)) << 4)) = r.k[u];
        }
        const int kk = tid & 63;
        for (int u = 0; u < 2; ++u) {
            const int dc = (tid >> 6) + 4 * u;
            for (int j = 0; j < 8; ++j) {
                const int d = 8 * dc + j;
                const uint32_t word = r.v[u][j >> 1];
                const uint16_t val = (j & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xffffu);
                *reinterpret_cast<uint16_t*>(Vt + d * 128 + (((kk >> 3) ^ swz_v(d)) << 4) + (kk & 7) * 2) = val;
            }
        }
    }

    // S^T (32 keys x 32 queries) of sub-tile `sub` (keys 32*sub .. 32*sub+31 of the stage).
    __device__ static f32x16 qk(const char* stage, int sub, int lane, const QOp& q) {
        const int row = 32 * sub + sigma(lane & 31), h2 = lane >> 5;
        const char* base = stage + row * 128;
        const int sw = swz_k(row);
        f32x16 acc = {};
        for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(base + (((2 * kb + h2) ^ sw) << 4));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q.v[kb], acc, 0, 0, 0);
        }
        return acc;
    }

    // O^T += V^T P^T over the 32 keys of sub-tile `sub`.
    __device__ static void pv(const char* stage, int sub, int lane, const PFrag& pf, f32x16* o) {
        const int M = lane & 31, h2 = lane >> 5;
        const char* Vt = stage + kKBytes;
        for (int db = 0; db < 2; ++db) {
            const int d = 32 * db + pi_col(M);
            const char* rowp = Vt + d * 128;
            const int sw = swz_v(d);
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(rowp + (((4 * sub + 2 * kb + h2) ^ sw) << 4));
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf.v[kb], o[db], 0, 0, 0);
            }
        }
    }

    // Lane (query, h2) holds output columns 32*db + 16*h2 + 0..15.
    __device__ static void store_row(Elem* row, int h2, const f32x16* o, float scale) {
        for (int db = 0; db < 2; ++db) {
            for (int half = 0; half < 2; ++half) {
                f32x8 t;
                for (int j = 0; j < 8; ++j) t[j] = o[db][8 * half + j] * scale;
                const bf16x8 b = __builtin_convertvector(t, bf16x8);
                *reinterpret_cast<u32x4*>(row + 32 * db + 16 * h2 + 8 * half) = __builtin_bit_cast(u32x4, b);
            }
        }
    }

    __device__ static Elem from_float(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
};

struct F32 {
    using Elem = float;
    static constexpr int kKBytes = kStageKeys * 256;   // 16 KiB
    static constexpr int kStageBytes = 2 * kKBytes;    // K + V, both row-major
    struct QOp { float v[32]; };
    struct Regs { u32x4 k[4]; u32x4 v[4]; };
    struct PFrag { float v[16]; };

    __device__ static float make_p(const float* p, PFrag& pf) {
        float sum = 0.f;
        for (int i = 0; i < 16; ++i) {
            pf.v[i] = p[i];
            sum += p[i];
        }
        return sum;
    }

    // B operand of S^T = K Q^T for the 32x32x2 product: step t, lane-half h2 -> d = 32*h2 + t.
    __device__ static void load_q(QOp& q, const Elem* row, int h2) {
        for (int t4 = 0; t4 < 8; ++t4) {
            f32x4 x = row ? *reinterpret_cast<const f32x4*>(row + 32 * h2 + 4 * t4) : f32x4{0, 0, 0, 0};
            for (int e = 0; e < 4; ++e) q.v[4 * t4 + e] = x[e];
        }
    }

    template <class RowOf>
    __device__ static void load(Regs& r, const Elem* K, const Elem* V, RowOf row_of, int tid) {
        for (int u = 0; u < 4; ++u) {
            const int c = tid + kThreads * u, kk = c >> 4, col = c & 15;
            const int row = row_of(kk);
            r.k[u] = row >= 0 ? *reinterpret_cast<const u32x4*>(K + (size_t)row * 64 + col * 4) : u32x4{0, 0, 0, 0};
            r.v[u] = row >= 0 ? *reinterpret_cast<const u32x4*>(V + (size_t)row * 64 + col * 4) : u32x4{0, 0, 0, 0};
        }
    }

    __device__ static void store(char* stage, const Regs& r, int tid) {
        char* Ks = stage;
        char* Vs = stage + kKBytes;
        for (int u = 0; u < 4; ++u) {
            const int c = tid + kThreads * u, kk = c >> 4, col = c & 15;
            *reinterpret_cast<u32x4*>(Ks + kk * 256 + ((col ^ swz_k(kk)) << 4)) = r.k[u];
            *reinterpret_cast<u32x4*>(Vs + kk * 256 + (col << 4)) = r.v[u];
        }
    }

    __device__ static f32x16 qk(const char* stage, int sub, int lane, const QOp& q) {
        const int row = 32 * sub + sigma(lane & 31), h2 = lane >> 5;
        const char* base = stage + row * 256;
        const int sw = swz_k(row);
        f32x16 acc = {};
        for (int t4 = 0; t4 < 8; ++t4) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(base + (((8 * h2 + t4) ^ sw) << 4));
            for (int e = 0; e < 4; ++e)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], q.v[4 * t4 + e], acc, 0, 0, 0);
        }
        return acc;
    }

    // Step u pairs lane-half h2 with key key_local(u, h2), matching the score layout.
    __device__ static void pv(const char* stage, int sub, int lane, const PFrag& pf, f32x16* o) {
        const int M = lane & 31, h2 = lane >> 5;
        const float* Vs = reinterpret_cast<const float*>(stage + kKBytes);
        for (int db = 0; db < 2; ++db) {
            const int d = 32 * db + pi_col(M);
            for (int u = 0; u < 16; ++u) {
                const float a = Vs[(32 * sub + key_local(u, h2)) * 64 + d];
                o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, pf.v[u], o[db], 0, 0, 0);
            }
        }
    }

    __device__ static void store_row(Elem* row, int h2, const f32x16* o, float scale) {
        for (int db = 0; db < 2; ++db)
            for (int c = 0; c < 4; ++c) {
                f32x4 t;
                for (int j = 0; j < 4; ++j) t[j] = o[db][4 * c + j] * scale;
                *reinterpret_cast<f32x4*>(row + 32 * db + 16 * h2 + 4 * c) = t;
            }
    }

    __device__ static Elem from_float(float x) { return x; }
};

// ---------------------------------------------------------------------------
// Online softmax state of one lane: running max m (raw score units), the lane's
// share of the running sum l, and 32 output accumulators (two 32x32 blocks).

struct State {
    float m;
    float l;
    f32x16 o[2];
};

__device__ __forceinline__ void state_init(State& st) {
    st.m = kNegInf;
    st.l = 0.f;
    st.o[0] = f32x16{};
    st.o[1] = f32x16{};
}

// Raise the running max only when a row's block max exceeds it by more than
// 2^8 in weight: weights may then reach 256 (exact in bf16 and fp32 alike), and
// the output/sum rescale runs only on the few blocks that raise a max.
constexpr float kRaiseRaw = 8.0f / kScaleLog2;

// Fold one 32-key score block into the state; the weights go to the P^T operand.
template <class T>
__device__ __forceinline__ void online_update(State& st, const f32x16& s, typename T::PFrag& pf) {
    float mx = s[0];
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = pair_max(mx);
    const bool raise = mx > st.m + kRaiseRaw;  // a first finite block always raises
    if (__any(raise)) {
        // Lanes that keep their max keep alpha = 1 (their max may still be -inf).
        const float mnew = raise ? mx : st.m;
        const float alpha = raise ? fast_exp2((st.m - mnew) * kScaleLog2) : 1.f;  // 0 from -inf
        st.l *= alpha;
        st.o[0] *= alpha;
        st.o[1] *= alpha;
        st.m = mnew;
    }
    const float mc = (st.m == kNegInf ? 0.f : st.m) * kScaleLog2;
    float p[16];
    for (int i = 0; i < 16; ++i) p[i] = fast_exp2(fmaf(s[i], kScaleLog2, -mc));
    st.l += T::make_p(p, pf);
}

__device__ __forceinline__ bool is_global_row(const Params& p, int row) {
    int lo = 0, hi = p.n_g;  // sorted, distinct
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const int g = p.g[mid];
        if (g == row) return true;
        if (g < row) lo = mid + 1; else hi = mid;
    }
    return false;
}

__device__ __forceinline__ uint64_t ballot64(bool x) { return __ballot(x); }

// ---------------------------------------------------------------------------
// (a)+(b): one work-group = 128 consecutive rows of one residue class of one
// (b, h); wave wv owns rows r0 + 32*wv .. +31.  Global keys outside each row's
// window are folded first; then the window band is streamed in 64-key stages
// (double-buffered in LDS), each wave skipping 32-key sub-tiles outside its rows'
// band and masking only sub-tiles that touch the band edge or hold invalid keys.

template <class T>
__global__ __launch_bounds__(kThreads) void band_kernel(const Params p) {
    using Elem = typename T::Elem;
    __shared__ __attribute__((aligned(16))) char smem[2 * T::kStageBytes + 64 * sizeof(int)];
    int* gpos = reinterpret_cast<int*>(smem + 2 * T::kStageBytes);

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, h2 = lane >> 5;
    const int pid = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = pid / p.tiles_per_head, t = pid - bh * p.tiles_per_head;
    const int h = bh % p.H, b = bh / p.H;
    const int L = p.L, w = p.w, dil = p.dil[h];
    const int tpr = ((L + dil - 1) / dil + kRowsPerBlock - 1) / kRowsPerBlock;  // tiles per residue
    const int r = t / tpr;
    if (r >= dil) return;
    const int Lr = (L - r + dil - 1) / dil;  // rows in residue class r
    const int r0 = (t - r * tpr) * kRowsPerBlock;
    if (r0 >= Lr) return;

    const size_t off = (size_t)bh * L * 64;
    const Elem* Q = reinterpret_cast<const Elem*>(p.q) + off;
    const Elem* K = reinterpret_cast<const Elem*>(p.k) + off;
    const Elem* V = reinterpret_cast<const Elem*>(p.v) + off;
    Elem* O = reinterpret_cast<Elem*>(p.out) + off;
    const uint8_t* pad = p.pad ? p.pad + (size_t)b * L : nullptr;

    const int qa = r0 + 32 * wv;           // first virtual row of this wave
    const int qv = qa + (lane & 31);       // this lane's virtual row
    const bool rows_live = qa < Lr;
    typename T::QOp qop;
    T::load_q(qop, qv < Lr ? Q + (size_t)(r + qv * dil) * 64 : nullptr, h2);
    State st;
    state_init(st);
    typename T::PFrag pw;
    typename T::Regs regs;

    // (b) global keys, up to 64 per stage.
    for (int g0 = 0; g0 < p.n_g; g0 += kStageKeys) {
        const int gi = g0 + lane;
        const int gphys = gi < p.n_g ? p.g[gi] : -1;
        const bool ok = gphys >= 0 && (!pad || pad[gphys] == 0);
        const uint64_t inv = ~ballot64(ok);
        if (inv == ~0ull) continue;
        T::load(regs, K, V, [&](int kk) { return ((inv >> kk) & 1) ? -1 : p.g[g0 + kk]; }, tid);
        T::store(smem, regs, tid);
        if (tid < 64) {  // same-class globals: virtual position, for the in-window test
            const bool same = ok && gphys >= r && (gphys - r) % dil == 0;
            gpos[tid] = same ? (gphys - r) / dil : kNoPos;
        }
        __syncthreads();
        if (rows_live) {
            for (int sub = 0; sub < 2; ++sub) {
                const uint32_t inv32 = (uint32_t)(inv >> (32 * sub));
                if (inv32 == ~0u) continue;
                f32x16 s = T::qk(smem, sub, lane, qop);
                for (int i = 0; i < 16; ++i) {
                    const int kl = key_local(i, h2);
                    const int gp = gpos[32 * sub + kl];
                    const bool in_window = (unsigned)(gp - qv + w) <= (unsigned)(2 * w);
                    if (((inv32 >> kl) & 1) || in_window) s[i] = kNegInf;
                }
                online_update<T>(st, s, pw);
                T::pv(smem, sub, lane, pw, st.o);
            }
        }
        __syncthreads();
    }

    // (a) window band of this tile's rows: keys [kb0, kend) of the class.
    const int kb0 = max(0, r0 - w);
    const int kend = min(Lr, r0 + kRowsPerBlock + w);
    const int n_st = (kend - kb0 + kStageKeys - 1) / kStageKeys;
    auto invalid_of = [&](int st_idx) -> uint64_t {
        const int key = kb0 + kStageKeys * st_idx + lane;
        bool ok = key < kend;
        if (ok && pad) ok = pad[r + key * dil] == 0;
        return ~ballot64(ok);
    };
    auto row_fn = [&](int ks, uint64_t inv) {
        return [=](int kk) { return ((inv >> kk) & 1) ? -1 : r + (ks + kk) * dil; };
    };

    uint64_t inv_cur = n_st > 0 ? invalid_of(0) : ~0ull;
    if (inv_cur != ~0ull) {
        T::load(regs, K, V, row_fn(kb0, inv_cur), tid);
        T::store(smem, regs, tid);
    }
    __syncthreads();
    for (int s_i = 0; s_i < n_st; ++s_i) {
        const int ks = kb0 + kStageKeys * s_i;
        const uint64_t inv_next = s_i + 1 < n_st ? invalid_of(s_i + 1) : ~0ull;
        if (inv_next != ~0ull) T::load(regs, K, V, row_fn(ks + kStageKeys, inv_next), tid);
        const char* cur = smem + (s_i & 1) * T::kStageBytes;
        if (rows_live && inv_cur != ~0ull) {
            for (int sub = 0; sub < 2; ++sub) {
                const int kss = ks + 32 * sub;
                const uint32_t inv32 = (uint32_t)(inv_cur >> (32 * sub));
                if (inv32 == ~0u) continue;
                if (kss > qa + 31 + w || kss + 31 < qa - w) continue;  // outside every row's band
                const bool interior = kss >= qa + 31 - w && kss + 31 <= qa + w;
                f32x16 s = T::qk(cur, sub, lane, qop);
                if (!interior || inv32 != 0u) {
                    for (int i = 0; i < 16; ++i) {
                        const int kl = key_local(i, h2);
                        const int kv = kss + kl;
                        const bool ok = (unsigned)(kv - qv + w) <= (unsigned)(2 * w) && !((inv32 >> kl) & 1);
                        if (!ok) s[i] = kNegInf;
                    }
                }
                online_update<T>(st, s, pw);
                T::pv(cur, sub, lane, pw, st.o);
            }
        }
        if (inv_next != ~0ull) T::store(smem + ((s_i + 1) & 1) * T::kStageBytes, regs, tid);
        __syncthreads();
        inv_cur = inv_next;
    }

    const float lt = pair_sum(st.l);
    const float scale = lt > 0.f ? 1.f / lt : 0.f;
    if (qv < Lr) {
        const int row = r + qv * dil;
        if (!is_global_row(p, row)) T::store_row(O + (size_t)row * 64, h2, st.o, scale);
    }
}

// ---------------------------------------------------------------------------
// (c): work-group (chunk, gblk, bh) runs up to 32 global queries over keys
// [chunk*C, chunk*C + C).  Each wave takes one 64-key stage of every 256 keys;
// the four wave states are merged in LDS and one partial (max, sum, 64 outputs)
// per query is written for the merge kernel.

template <class T>
__global__ __launch_bounds__(kThreads) void global_rows_kernel(const Params p) {
    using Elem = typename T::Elem;
    constexpr int kRedBytes = (4 * 32 + 4 * 32 + 4 * 32 * 64) * 4;
    constexpr int kBytes = 4 * T::kStageBytes > kRedBytes ? 4 * T::kStageBytes : kRedBytes;
    __shared__ __attribute__((aligned(16))) char smem[kBytes];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, h2 = lane >> 5;
    const int chunk = blockIdx.x, gblk = blockIdx.y, bh = blockIdx.z;
    const int b = bh / p.H;
    const int L = p.L;
    const size_t off = (size_t)bh * L * 64;
    const Elem* Q = reinterpret_cast<const Elem*>(p.q) + off;
    const Elem* K = reinterpret_cast<const Elem*>(p.k) + off;
    const Elem* V = reinterpret_cast<const Elem*>(p.v) + off;
    const uint8_t* pad = p.pad ? p.pad + (size_t)b * L : nullptr;

    const int gq = gblk * kGlobalQueriesPerBlock + (lane & 31);
    typename T::QOp qop;
    T::load_q(qop, gq < p.n_g ? Q + (size_t)p.g[gq] * 64 : nullptr, h2);
    State st;
    state_init(st);
    typename T::PFrag pw;
    typename T::Regs regs;
    const char* mybuf = smem + wv * T::kStageBytes;

    const int c0 = chunk * p.chunk;
    const int c1 = min(L, c0 + p.chunk);
    const int n_super = (c1 - c0 + 4 * kStageKeys - 1) / (4 * kStageKeys);
    for (int s_i = 0; s_i < n_super; ++s_i) {
        // Four 64-key stages per step, staged by all 256 threads; wave x computes stage x.
        uint64_t inv_mine = ~0ull;
        for (int x = 0; x < 4; ++x) {
            const int ks = c0 + 4 * kStageKeys * s_i + kStageKeys * x;
            const int key = ks + lane;
            bool ok = key < c1;
            if (ok && pad) ok = pad[key] == 0;
            const uint64_t inv = ~ballot64(ok);
            if (x == wv) inv_mine = inv;
            if (inv != ~0ull) {
                T::load(regs, K, V, [&](int kk) { return ((inv >> kk) & 1) ? -1 : ks + kk; }, tid);
                T::store(smem + x * T::kStageBytes, regs, tid);
            }
        }
        __syncthreads();
        if (inv_mine != ~0ull) {
            for (int sub = 0; sub < 2; ++sub) {
                const uint32_t inv32 = (uint32_t)(inv_mine >> (32 * sub));
                if (inv32 == ~0u) continue;
                f32x16 s = T::qk(mybuf, sub, lane, qop);
                if (inv32 != 0u)
                    for (int i = 0; i < 16; ++i)
                        if ((inv32 >> key_local(i, h2)) & 1) s[i] = kNegInf;
                online_update<T>(st, s, pw);
                T::pv(mybuf, sub, lane, pw, st.o);
            }
        }
        __syncthreads();
    }

    // Merge the four waves (each saw a disjoint quarter of the chunk).
    float* red_m = reinterpret_cast<float*>(smem);
    float* red_l = red_m + 4 * 32;
    float* red_o = red_l + 4 * 32;
    const float lsum = pair_sum(st.l);
    if (lane < 32) {
        red_m[wv * 32 + lane] = st.m;
        red_l[wv * 32 + lane] = lsum;
    }
    for (int db = 0; db < 2; ++db)
        for (int i = 0; i < 16; ++i) red_o[(wv * 32 + (lane & 31)) * 64 + 32 * db + 16 * h2 + i] = st.o[db][i];
    __syncthreads();

    const int q = tid >> 3, dc = tid & 7;
    const int gq2 = gblk * kGlobalQueriesPerBlock + q;
    if (gq2 < p.n_g) {
        float M = kNegInf;
        for (int x = 0; x < 4; ++x) M = fmaxf(M, red_m[x * 32 + q]);
        float e[4];
        for (int x = 0; x < 4; ++x) e[x] = M == kNegInf ? 0.f : fast_exp2((red_m[x * 32 + q] - M) * kScaleLog2);
        float l = 0.f;
        for (int x = 0; x < 4; ++x) l += red_l[x * 32 + q] * e[x];
        const size_t idx = ((size_t)bh * p.n_gblk * kGlobalQueriesPerBlock + gq2) * p.n_chunks + chunk;
        if (dc == 0) {
            p.ws_ml[2 * idx] = M;
            p.ws_ml[2 * idx + 1] = l;
        }
        for (int j = 0; j < 8; ++j) {
            const int d = 8 * dc + j;
            float o = 0.f;
            for (int x = 0; x < 4; ++x) o += red_o[(x * 32 + q) * 64 + d] * e[x];
            p.ws_acc[idx * 64 + d] = o;
        }
    }
}

// ---------------------------------------------------------------------------
// (d): one wave per (global query, bh); thread d merges the chunk partials of
// output column d in chunk order (deterministic) and writes the row.

template <class T>
__global__ __launch_bounds__(64) void merge_kernel(const Params p) {
    using Elem = typename T::Elem;
    const int gi = blockIdx.x, bh = blockIdx.y, d = threadIdx.x;
    const size_t base = ((size_t)bh * p.n_gblk * kGlobalQueriesPerBlock + gi) * p.n_chunks;
    float M = kNegInf;
    for (int c = 0; c < p.n_chunks; ++c) M = fmaxf(M, p.ws_ml[2 * (base + c)]);
    float l = 0.f, o = 0.f;
    if (M != kNegInf) {
        for (int c = 0; c < p.n_chunks; ++c) {
            const float e = fast_exp2((p.ws_ml[2 * (base + c)] - M) * kScaleLog2);
            l += p.ws_ml[2 * (base + c) + 1] * e;
            o += p.ws_acc[(base + c) * 64 + d] * e;
        }
    }
    const float res = l > 0.f ? o / l : 0.f;
    Elem* O = reinterpret_cast<Elem*>(p.out) + (size_t)bh * p.L * 64;
    O[(size_t)p.g[gi] * 64 + d] = T::from_float(res);
}

}  // namespace

hipError_t launch_band(const Params& p, int dtype, hipStream_t s) {
    const int blocks = p.B * p.H * p.tiles_per_head;
    if (blocks <= 0) return hipSuccess;
    if (dtype == LF_BF16)
        hipLaunchKernelGGL(band_kernel<Bf16>, dim3(blocks), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL(band_kernel<F32>, dim3(blocks), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_global_rows(const Params& p, int dtype, hipStream_t s) {
    if (p.n_g == 0) return hipSuccess;
    const dim3 grid(p.n_chunks, p.n_gblk, p.B * p.H);
    if (dtype == LF_BF16)
        hipLaunchKernelGGL(global_rows_kernel<Bf16>, grid, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL(global_rows_kernel<F32>, grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_merge(const Params& p, int dtype, hipStream_t s) {
    if (p.n_g == 0) return hipSuccess;
    const dim3 grid(p.n_g, p.B * p.H);
    if (dtype == LF_BF16)
        hipLaunchKernelGGL(merge_kernel<Bf16>, grid, dim3(64), 0, s, p);
    else
        hipLaunchKernelGGL(merge_kernel<F32>, grid, dim3(64), 0, s, p);
    return hipGetLastError();
}

}  // namespace lf
