// gfx950 (MI355X) kernels of the Longformer window + global attention backward
// (bf16 tensors with fp32 accumulation, or fp32 tensors: one set of kernels on
// element traits).
//
// For O = P V with P the row softmax of S = Q K^T / sqrt(d_h) over each row's key
// set (the forward's pattern: page "基于自注意力机制的长文本建模算法：Longformer详解"
// §2 and §4, page "基于Block-Sparse Attention的Longformer" §2 and §4), and an
// upstream gradient dO, the textbook derivatives of the product and the softmax
// (page "Reformer哈希" §"core principle" formula) are
//
//   D_i = dO_i . O_i,   dS_ij = P_ij (dO_i . V_j - D_i),
//   dQ_i = sum_j dS_ij K_j / sqrt(d_h),   dK_j = sum_i dS_ij Q_i / sqrt(d_h),
//   dV_j = sum_i P_ij dO_i,
//
// with P recomputed from the forward's per-row log-sum-exp (no softmax statistics
// are rebuilt).  The attended pairs (i, j) are split so that every gradient visits
// each pair exactly once:
//   A  i not global, j in the window of i (a global j included);
//   B  i not global, j global outside the window of i;
//   C  i global, every unpadded j.
//
// bwd_prep_kernel  D, and the log-sum-exp in base-2 units of the pre-scaled scores
//                  (lse2; lse2_band is +inf on global rows, which removes them from
//                  the window passes of the key-owned kernel).
// bwd_dq_kernel    row-owned, the forward's traversal (global key stages, then the
//                  window band): dQ of every non-global row over A and B; for the
//                  global rows (C), one partial per (tile, global query) over the
//                  tile's 128 home keys.
// bwd_dkv_kernel   key-owned, the same traversal with the roles of rows and keys
//                  exchanged (global query stages, then the band of window queries):
//                  dK, dV of every key over A and C; for global keys, one partial per
//                  (tile, global key) over the tile's home queries in B.
// bwd_merge_kernel sums the partials of each global row and key in tile order and
//                  writes dQ of the global rows and dK, dV of the global keys.
//
// Every product is a 32 x 32 tile on the matrix cores (v_mfma_f32_32x32x16_bf16 for
// bf16, v_mfma_f32_32x32x2_f32 for fp32).
// Row-owned: S^T = K Q^T and dP^T = V dO^T with one query per lane, dQ^T += K^T dS^T.
// Key-owned: S = Q K^T and dP = dO V^T with one key per lane, dV^T += dO^T P and
// dK^T += Q^T dS.  The staged tiles (K and V, or Q and dO) are row-major in LDS with
// the 16-byte-chunk XOR swizzle and are read both ways: 128-bit row reads for the
// first operand of the score products and transposed reads (ds_read_b64_tr_b16) for
// the first operand of the gradient products.

#include <type_traits>

#include "lf_attn_device.h"

namespace lf {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPosInf = __builtin_inff();
constexpr int kBwdMaskWindow = 64;
constexpr int kBwdMaskRing = 2 * kBwdMaskWindow;
constexpr int kBwdMaxGlobalStages = LF_MAX_GLOBALS / kStageKeys;

// 4 bytes per lane from global memory into LDS at lds_base + 4 * lane (see dma16).
__device__ __forceinline__ void dma4(const void* src, char* lds_base) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(lds_base));
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(base) : "memory", "m0");
}

// Element traits of the backward kernels.  One stage holds tile A (64 rows), tile B
// (64 rows), 64 floats of lse2 and 64 of D; tile rows are row-major with the K
// swizzle of 16-byte chunks and are read both ways: by rows for the first operand of
// the score products (prod) and by columns for the first operand of the gradient
// products (load_t / acc_t).  Accumulator element i of lane-half h2 of a score product
// belongs to tile row 32*sub + key_local(i, h2) in both.

// bf16 tensors: v_mfma_f32_32x32x16_bf16, transposed reads with ds_read_b64_tr_b16.
struct BBf16 {
    using Elem = uint16_t;
    static constexpr int kRowB = 128;
    static constexpr int kTileB = kStageKeys * kRowB;  // 8 KiB
    static constexpr int kLseOff = 2 * kTileB;
    static constexpr int kDOff = kLseOff + 256;
    static constexpr int kStageB = kDOff + 256;
    static constexpr int kWavesPerEU = 3;

    struct Op { bf16x8 v[4]; };      // B operand of a score product: lane (n, h2) holds d = 16*kb + 8*h2 + j
    struct Frag { bf16x8 v[2]; };    // B operand of a gradient product (weights or dS)
    struct TOp { bf16x8 v[2][2]; };  // transposed A operand [db][kb]

    __device__ __forceinline__ static void load_op(Op& o, const Elem* row, int h2) {
        if (!row) row = reinterpret_cast<const Elem*>(g_zero_row);
        for (int kb = 0; kb < 4; ++kb)
            o.v[kb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 16 * kb + 8 * h2));
    }
    __device__ __forceinline__ static void scale_op(Op& o) {
        for (int kb = 0; kb < 4; ++kb) {
            const f32x8 f = __builtin_convertvector(o.v[kb], f32x8);
            o.v[kb] = __builtin_convertvector(f * kScaleLog2, bf16x8);
        }
    }

    // Rows of two tensors into tiles A and B of a stage: wave wv copies 1-KiB blocks
    // 2*wv, 2*wv+1 (8 rows each).  row_of(kk) is the source row of stage row kk, or -1
    // for a zero row.
    template <class RowOf>
    __device__ __forceinline__ static void dma_tiles(char* slot, const Elem* A, const Elem* Bt, RowOf row_of, int wv,
                                                     int lane) {
        const Elem* zero = reinterpret_cast<const Elem*>(g_zero_row);
        for (int u = 0; u < 2; ++u) {
            const int blk = 2 * wv + u;
            const int row = 8 * blk + (lane >> 3), cl = lane & 7;
            const int src = row_of(row);
            const int c = 8 * (cl ^ swz_k(row));
            dma16((src >= 0 ? A + (size_t)src * 64 : zero) + c, slot + blk * 1024);
            dma16((src >= 0 ? Bt + (size_t)src * 64 : zero) + c, slot + kTileB + blk * 1024);
        }
    }

    // Per-lane LDS byte offsets.  nk: 128-bit row reads (row sigma(M), chunk
    // (2*kb + h2) ^ swz_k(row)).  tr: transposed reads; within each 16-lane group, lane i
    // addresses row 8*h2 + i/4 (+ 4*t + 16*kb + 32*sub), columns 32*db + 16*g1 + 4*(i%4)
    // .. +3, and receives one column of four consecutive rows.  Rows 8*h2 + i/4 have bit
    // 2 clear, so adding 4 (t = 1) keeps swz_k; multiples of 16 keep it as well.
    struct Lanes { int nk[4]; int tr[2]; };
    __device__ __forceinline__ static void lane_setup(Lanes& lo, int lane) {
        const int row = sigma(lane & 31), h2 = lane >> 5;
        for (int kb = 0; kb < 4; ++kb) lo.nk[kb] = row * kRowB + (((2 * kb + h2) ^ swz_k(row)) << 4);
        const int g1 = (lane >> 4) & 1, i = lane & 15;
        const int vrow = 8 * h2 + (i >> 2);
        for (int db = 0; db < 2; ++db) {
            const int chunk = 4 * db + 2 * g1 + ((i & 3) >> 1);
            lo.tr[db] = vrow * kRowB + ((chunk ^ swz_k(vrow)) << 4) + 8 * (i & 1);
        }
    }

    // seed + (rows 32*sub .. +31 of the tile) x (lane operand).
    __device__ __forceinline__ static f32x16 prod(const char* tile, int sub, const Lanes& lo, const Op& b,
                                                  const f32x16& seed) {
        const char* base = tile + sub * 32 * kRowB;
        f32x16 acc = seed;
        for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(base + lo.nk[kb]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b.v[kb], acc, 0, 0, 0);
        }
        return acc;
    }

    __device__ __forceinline__ static void to_frag(const float* x, Frag& f) {
        for (int kb = 0; kb < 2; ++kb) {
            f32x8 t;
            for (int j = 0; j < 8; ++j) t[j] = x[8 * kb + j];
            f.v[kb] = __builtin_convertvector(t, bf16x8);
        }
    }

    // Transposed operand of rows 32*sub .. +31 of a tile: lane l holds column 32*db + l%32
    // of rows 16*kb + 8*h2 + 0..7.
    __device__ __forceinline__ static void load_t(TOp& t, const char* tile, int sub, const Lanes& lo) {
        const char* base = tile + sub * 32 * kRowB;
        for (int db = 0; db < 2; ++db)
            for (int kb = 0; kb < 2; ++kb) {
                const char* a = base + lo.tr[db] + 16 * kb * kRowB;
                const s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LF_LDS(s16x4, a));
                const s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LF_LDS(s16x4, a + 4 * kRowB));
                t.v[db][kb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7));
            }
    }
    __device__ __forceinline__ static void acc_t(const TOp& t, const Frag& f, f32x16* acc) {
        for (int kb = 0; kb < 2; ++kb)
            for (int db = 0; db < 2; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t.v[db][kb], f.v[kb], acc[db], 0, 0, 0);
    }

    __device__ __forceinline__ static uint32_t pack_bf16(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
    }
    // Accumulator element (db, i) of lane-half h2 is column 32*db + 8*(i/4) + 4*h2 + i%4.
    __device__ __forceinline__ static void store_row(Elem* row, int h2, const f32x16* o, float scale) {
        for (int db = 0; db < 2; ++db)
            for (int q = 0; q < 4; ++q) {
                const float a = o[db][4 * q] * scale, b = o[db][4 * q + 1] * scale;
                const float c = o[db][4 * q + 2] * scale, d = o[db][4 * q + 3] * scale;
                const u32x2 w = {pack_bf16(a, b), pack_bf16(c, d)};
                *reinterpret_cast<u32x2*>(row + 32 * db + 8 * q + 4 * h2) = w;
            }
    }
    __device__ __forceinline__ static Elem from_float(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
};

// fp32 tensors: v_mfma_f32_32x32x2_f32 (step t of a score product pairs lane-half h2
// with d = 32*h2 + t; step u of a gradient product with tile row key_local(u, h2)),
// single-float column reads for the transposed operand.
struct BF32 {
    using Elem = float;
    static constexpr int kRowB = 256;
    static constexpr int kTileB = kStageKeys * kRowB;  // 16 KiB
    static constexpr int kLseOff = 2 * kTileB;
    static constexpr int kDOff = kLseOff + 256;
    static constexpr int kStageB = kDOff + 256;
    static constexpr int kWavesPerEU = 2;

    struct Op { float v[32]; };
    struct Frag { float v[16]; };
    struct TOp { const char* base; };  // rows 32*sub .. of the tile, read inside acc_t
    struct Lanes { int nk; int sw; int h2; int col; };

    __device__ __forceinline__ static void load_op(Op& o, const Elem* row, int h2) {
        if (!row) row = reinterpret_cast<const Elem*>(g_zero_row);
        for (int t4 = 0; t4 < 8; ++t4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(row + 32 * h2 + 4 * t4);
            for (int e = 0; e < 4; ++e) o.v[4 * t4 + e] = x[e];
        }
    }
    __device__ __forceinline__ static void scale_op(Op& o) {
        for (int i = 0; i < 32; ++i) o.v[i] *= kScaleLog2;
    }

    // Wave wv copies 1-KiB blocks 4*wv .. 4*wv+3 of each tile (4 rows each).
    template <class RowOf>
    __device__ __forceinline__ static void dma_tiles(char* slot, const Elem* A, const Elem* Bt, RowOf row_of, int wv,
                                                     int lane) {
        const Elem* zero = reinterpret_cast<const Elem*>(g_zero_row);
        for (int u = 0; u < 4; ++u) {
            const int blk = 4 * wv + u;
            const int row = 4 * blk + (lane >> 4), cl = lane & 15;
            const int src = row_of(row);
            const int c = 4 * (cl ^ swz_k(row));
            dma16((src >= 0 ? A + (size_t)src * 64 : zero) + c, slot + blk * 1024);
            dma16((src >= 0 ? Bt + (size_t)src * 64 : zero) + c, slot + kTileB + blk * 1024);
        }
    }

    __device__ __forceinline__ static void lane_setup(Lanes& lo, int lane) {
        const int row = sigma(lane & 31);
        lo.nk = row * kRowB;
        lo.sw = swz_k(row);
        lo.h2 = lane >> 5;
        lo.col = lane & 31;
    }

    __device__ __forceinline__ static f32x16 prod(const char* tile, int sub, const Lanes& lo, const Op& b,
                                                  const f32x16& seed) {
        const char* base = tile + sub * 32 * kRowB + lo.nk;
        f32x16 acc = seed;
        for (int t4 = 0; t4 < 8; ++t4) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(base + (((8 * lo.h2 + t4) ^ lo.sw) << 4));
            for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b.v[4 * t4 + e], acc, 0, 0, 0);
        }
        return acc;
    }

    __device__ __forceinline__ static void to_frag(const float* x, Frag& f) {
        for (int i = 0; i < 16; ++i) f.v[i] = x[i];
    }

    __device__ __forceinline__ static void load_t(TOp& t, const char* tile, int sub, const Lanes&) {
        t.base = tile + sub * 32 * kRowB;
    }
    // acc[db] (column 32*db + l%32 of the tile, lane's column of f) += sum over the 32
    // rows of the sub-tile: step u takes row key_local(u, h2) for lane-half h2.
    __device__ __forceinline__ static void acc_t(const TOp& t, const Frag& f, f32x16* acc, const Lanes& lo) {
        for (int u = 0; u < 16; ++u) {
            const int row = key_local(u, lo.h2);
            const char* rb = t.base + row * kRowB + 4 * (lo.col & 3);
            for (int db = 0; db < 2; ++db) {
                const int c = 32 * db + lo.col;
                const float a = *reinterpret_cast<const float*>(rb + (((c >> 2) ^ swz_k(row)) << 4));
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, f.v[u], acc[db], 0, 0, 0);
            }
        }
    }

    __device__ __forceinline__ static void store_row(Elem* row, int h2, const f32x16* o, float scale) {
        for (int db = 0; db < 2; ++db)
            for (int q = 0; q < 4; ++q) {
                f32x4 t;
                for (int j = 0; j < 4; ++j) t[j] = o[db][4 * q + j] * scale;
                *reinterpret_cast<f32x4*>(row + 32 * db + 8 * q + 4 * h2) = t;
            }
    }
    __device__ __forceinline__ static Elem from_float(float x) { return x; }
};

// Gradient product through the traits (the fp32 form also needs the lane layout).
template <class T>
__device__ __forceinline__ void acc_t(const typename T::TOp& t, const typename T::Frag& f, f32x16* acc,
                                      const typename T::Lanes& lo) {
    if constexpr (std::is_same_v<T, BF32>)
        T::acc_t(t, f, acc, lo);
    else
        T::acc_t(t, f, acc);
}

// lse2 and D of the 64 stage rows (one wave; zero for row -1).
template <class T, class RowOf>
__device__ __forceinline__ void dma_floats(char* slot, const float* lse2, const float* dsum, RowOf row_of, int lane) {
    const int src = row_of(lane);
    const float* zero = reinterpret_cast<const float*>(g_zero_row);
    dma4(src >= 0 ? lse2 + src : zero, slot + T::kLseOff);
    dma4(src >= 0 ? dsum + src : zero, slot + T::kDOff);
}

__device__ __forceinline__ void store_row_f32(float* row, int h2, const f32x16* o, float scale) {
    for (int db = 0; db < 2; ++db)
        for (int q = 0; q < 4; ++q) {
            f32x4 t;
            for (int j = 0; j < 4; ++j) t[j] = o[db][4 * q + j] * scale;
            *reinterpret_cast<f32x4*>(row + 32 * db + 8 * q + 4 * h2) = t;
        }
}

// Per-element seeds of a key-owned product: minus the staged floats of the 16 rows
// the lane's elements belong to (rows 32*sub + key_local(i, h2)).
__device__ __forceinline__ f32x16 row_seed(const char* arr, int sub, int h2) {
    const f32x4* a = reinterpret_cast<const f32x4*>(arr) + 8 * sub + 2 * h2;
    const f32x4 x0 = a[0], x1 = a[1], x2 = a[4], x3 = a[5];
    f32x16 s;
    for (int j = 0; j < 4; ++j) {
        s[j] = -x0[j];
        s[4 + j] = -x1[j];
        s[8 + j] = -x2[j];
        s[12 + j] = -x3[j];
    }
    return s;
}

// Bits lo..31 of a word (lo may lie outside 0..31).
__device__ __forceinline__ uint32_t bits_from(int lo) {
    return lo <= 0 ? ~0u : (lo >= 32 ? 0u : (~0u << lo));
}
// Bits 0..hi-1 of a word (hi may lie outside 0..32).
__device__ __forceinline__ uint32_t bits_below(int hi) {
    return hi <= 0 ? 0u : (hi >= 32 ? ~0u : ((1u << hi) - 1u));
}

// Relative position bias table of head h in LDS, base 2, with kBiasPad zeros on both
// ends: entry kBiasPad + w + m holds offset m (reversed: offset -m).
__device__ __forceinline__ void fill_bias(float* lds, const BwdParams& p, int h, int w, int tid, bool reversed) {
    const float* tab = p.bias + (size_t)h * (2 * p.bias_w + 1) + p.bias_w;  // entry of offset 0
    for (int t = tid; t < 2 * w + 1 + 2 * kBiasPad; t += kThreads) {
        const int m = (reversed ? -1 : 1) * (t - kBiasPad - w);
        lds[t] = (m >= -w && m <= w) ? tab[m] * kLog2eF : 0.f;
    }
}
__device__ __forceinline__ void add_bias(f32x16& s, const float* brow) {
    for (int i = 0; i < 16; ++i) s[i] += brow[kc_of(i)];
}

__device__ __forceinline__ f32x16 splat(float x) {
    f32x16 s;
    for (int i = 0; i < 16; ++i) s[i] = x;
    return s;
}

// Cross-wave sum of a 32 x 64 block per wave (lane-half h2 of lane (q, h2) holds
// accumulator columns as in store_row), written as fp32 rows dst + q*64 for q < nq.
// Uses red (32 KiB of LDS); the caller brackets it with barriers.
__device__ __forceinline__ void wave_sum_store(float* red, const f32x16* a, int wv, int lane, int tid, float* dst,
                                               int nq) {
    // Four columns 4c .. 4c+3 of row q (a 16-byte chunk c) sit at chunk c ^ (q % 16) of
    // row q: one 16-byte store per accumulator group, two 16-byte loads per column block.
    const int q0 = lane & 31, h2 = lane >> 5;
    for (int db = 0; db < 2; ++db)
        for (int m = 0; m < 4; ++m) {
            const int c = 8 * db + 2 * m + h2;  // columns 32 db + 8 m + 4 h2 .. + 3
            *reinterpret_cast<f32x4*>(red + (wv * 32 + q0) * 64 + 4 * (c ^ (q0 & 15))) =
                f32x4{a[db][4 * m], a[db][4 * m + 1], a[db][4 * m + 2], a[db][4 * m + 3]};
        }
    __syncthreads();
    const int q = tid >> 3, dc = tid & 7;  // 32 rows x 8 column chunks
    if (q < nq) {
        f32x4 o4[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        for (int x = 0; x < kWaves; ++x)
            for (int u = 0; u < 2; ++u)
                o4[u] += *reinterpret_cast<const f32x4*>(red + (x * 32 + q) * 64 + 4 * ((2 * dc + u) ^ (q & 15)));
        *reinterpret_cast<f32x4*>(dst + (size_t)q * 64 + 8 * dc) = o4[0];
        *reinterpret_cast<f32x4*>(dst + (size_t)q * 64 + 8 * dc + 4) = o4[1];
    }
    __syncthreads();
}

// The work-group's tile: 128 own rows [r0, r0 + 128) of residue class r of one
// (b, h), and the other side's rows [kb0, kend) of the same class (every row whose
// offset from an own row, other - own, lies in [-A, B]) in 64-row stages on a grid
// aligned to r0: nb stages before the own rows, the two "home" stages
// [r0, r0 + 128), na stages after, processed in the order before, after, home.
struct Tile {
    int bh, b, h, t_in, r, dil, Lr, r0, kb0, kend, nb, na, n_band, gbase;
    __device__ int stage_row(int u) const {
        const int bs = u < nb ? u : (u < nb + na ? u + 2 : u - na);
        return gbase + kStageKeys * bs;
    }
};
// The tile of this work-group from the grid size, tiles per head, heads, length and
// shared dilation (the kernels' leading arguments, preloaded into scalar registers);
// false when the slot holds no tile.  tile_extent adds the other side's rows.
__device__ __forceinline__ bool tile_of(Tile& t, const BwdParams& p, int nblk, int tph, int H, int L, int dil_u) {
    const int pid = xcd_remap(blockIdx.x, nblk);
    t.bh = pid / tph;
    t.t_in = pid - t.bh * tph;
    t.h = t.bh % H;
    t.b = t.bh / H;
    t.dil = head_dil(dil_u, p.dil, t.h);
    return decode_tile(t.t_in, L, t.dil, t.r, t.Lr, t.r0);
}
__device__ __forceinline__ void tile_extent(Tile& t, int A, int B) {
    t.kb0 = max(0, t.r0 - A);
    t.kend = min(t.Lr, t.r0 + kRowsPerBlock + B);
    t.nb = (t.r0 - t.kb0 + kStageKeys - 1) / kStageKeys;
    t.gbase = t.r0 - kStageKeys * t.nb;
    t.na = max(0, (t.kend - (t.r0 + 2 * kStageKeys) + kStageKeys - 1) / kStageKeys);
    t.n_band = t.nb + 2 + t.na;
}

// ---------------------------------------------------------------------------
// Row statistics: D, lse2, lse2_band.  One work-group per 128 rows of one (b, h): eight
// lanes per row, each reading 16 bytes of O and of dO (a wave reads eight whole rows of
// each per load); a lane group takes kPrepRowsPerGroup rows with all their loads in
// flight together, adds the partial dot products across its eight lanes, and lane k of
// the group finishes row k (log-sum-exp conversion, global test, stores).

constexpr int kPrepRowsPerGroup = 4;
constexpr int kPrepGroups = kThreads / 8;
constexpr int kPrepRowsPerBlock = kPrepGroups * kPrepRowsPerGroup;
template <class T>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(const BwdParams p) {
    using Elem = typename T::Elem;
    __shared__ int gpos[LF_MAX_GLOBALS];  // this sequence's global positions, sorted
    const int L = p.L;
    const int nblk = (L + kPrepRowsPerBlock - 1) / kPrepRowsPerBlock;
    const int bh = blockIdx.x / nblk, blk = blockIdx.x - bh * nblk;
    const int bseq = bh / p.H, gofs = bseq * p.gstride;
    const int ng = p.gstride ? p.gcnt[bseq] : p.n_g;
    const int c = threadIdx.x & 7;  // eighth of a row
    const int pos0 = blk * kPrepRowsPerBlock + (threadIdx.x >> 3);
    const size_t off = (size_t)bh * L;
    // a lane's eighth of a row: 16 bytes (bf16) or 32 bytes (fp32)
    constexpr int kV = sizeof(Elem) == 2 ? 1 : 2;
    u32x4 o[kPrepRowsPerGroup][kV], g[kPrepRowsPerGroup][kV];
    for (int k = 0; k < kPrepRowsPerGroup; ++k) {
        const int pos = pos0 + k * kPrepGroups;
        const size_t row = off + (pos < L ? pos : 0);
        for (int v = 0; v < kV; ++v) {
            o[k][v] = reinterpret_cast<const u32x4*>(reinterpret_cast<const Elem*>(p.o) + row * 64)[kV * c + v];
            g[k][v] = reinterpret_cast<const u32x4*>(reinterpret_cast<const Elem*>(p.dout) + row * 64)[kV * c + v];
        }
    }
    for (int t = threadIdx.x; t < ng; t += kThreads) gpos[t] = p.g[gofs + t];
    __syncthreads();
    float mine = 0.f;  // the dot product of row c of this group (c < kPrepRowsPerGroup)
    for (int k = 0; k < kPrepRowsPerGroup; ++k) {
        float acc = 0.f;
        if constexpr (kV == 1) {
            const f32x8 a = __builtin_convertvector(__builtin_bit_cast(bf16x8, o[k][0]), f32x8);
            const f32x8 b = __builtin_convertvector(__builtin_bit_cast(bf16x8, g[k][0]), f32x8);
            for (int j = 0; j < 8; ++j) acc += a[j] * b[j];
        } else {
            for (int v = 0; v < kV; ++v) {
                const f32x4 a = __builtin_bit_cast(f32x4, o[k][v]), b = __builtin_bit_cast(f32x4, g[k][v]);
                for (int j = 0; j < 4; ++j) acc += a[j] * b[j];
            }
        }
        for (int m = 1; m < 8; m <<= 1) acc += __shfl_xor(acc, m);  // the row's eight lanes
        mine = c == k ? acc : mine;
    }
    const int pos = pos0 + c * kPrepGroups;
    if (c >= kPrepRowsPerGroup || pos >= L) return;
    const size_t i = off + pos;
    const float lse = p.lse[i];
    const float l2 = lse == kNegInf ? kPosInf : lse * kLog2e;
    const int cnt = count_le(gpos, ng, pos);
    const bool is_g = cnt > 0 && gpos[cnt - 1] == pos;
    p.dsum[i] = mine;
    p.lse2[i] = l2;
    p.lse2_band[i] = is_g ? kPosInf : l2;
}

// ---------------------------------------------------------------------------
// dQ: one work-group per 128 rows of one residue class of one (b, h); wave wv owns
// rows r0 + 32*wv .. +31, one per lane (both lane halves).  Stages: the global keys
// (with the in-window test, so each key counts once), the random key blocks of the
// tile's two query blocks (kRandom, as in the forward), then the window band.

// With kBiasGrad (and kBias) each wave also sums dS of its window pairs per offset
// m = key - query (class steps) into an LDS accumulator of its own (dynamic LDS,
// 2w + 1 + 2*kBiasPad floats per wave); per 32-key sub-tile and score element, the 32
// lanes of one lane half hit 32 distinct offsets, so the adds are free of conflicts and
// their order is fixed.  The work-group's sum over its waves goes to ws_db.
template <class T, bool kCausal, bool kBias, bool kRandom, bool kBiasGrad = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(T::kWavesPerEU)))
void bwd_dq_kernel(const int nblk, const int tph, const int H, const int L, const int dil_u, const void* const q_arg,
                   const void* const dout_arg, const float* const lse2_arg, const float* const dsum_arg,
                   const BwdParams p) {
    static_assert(!kBiasGrad || kBias, "the table gradient needs the table");
    using Elem = typename T::Elem;
    constexpr int kStageB = T::kStageB, kTileB = T::kTileB;
    extern __shared__ float db_lds[];
    __shared__ __attribute__((aligned(16))) char ring[2 * kStageB];
    __shared__ uint64_t band_mask[kBwdMaskRing];
    __shared__ uint64_t glob_mask[kBwdMaxGlobalStages];
    __shared__ int glob_src[LF_MAX_GLOBALS];
    __shared__ __attribute__((aligned(16))) int glob_pos[LF_MAX_GLOBALS];
    __shared__ int glob_abs[LF_MAX_GLOBALS];
    __shared__ int glob_row[LF_MAX_GLOBALS];
    __shared__ uint32_t row_glob[kRowsPerBlock / 32];
    __shared__ float bias_lds[kBias ? kBiasLds : 1];  // offset m at kBiasPad + m + w, base 2
    __shared__ uint64_t rnd_inv[kRandom ? 2 * LF_MAX_RANDOM_DRAWS : 1];  // invalid keys of random stages

    // Keys of a row: w class steps before it and wr after (wr = 0 one-sided).
    constexpr bool causal = kCausal;
    // The leading arguments (grid size, p.tiles_per_head, p.H, p.L, p.dil_u and the
    // pointers of the row loads) are preloaded into scalar registers by the build: the
    // tile decode and the first loads wait for no memory.  The shared global set's
    // positions are loaded first (the slot set-up then waits for them alone), and the
    // other arguments are read in one batch after the row loads are issued.
    Tile tl;
    if (!tile_of(tl, p, nblk, tph, H, L, dil_u)) return;
    const int tid = threadIdx.x, lane = tid & 63, h2 = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int dil = tl.dil, r = tl.r, r0 = tl.r0, Lr = tl.Lr;
    const size_t off = (size_t)tl.bh * L * 64;
    static_assert(kThreads <= LF_MAX_GLOBALS && kBwdMaxGlobalStages * kStageKeys <= kThreads,
                  "one slot per thread covers every global stage");
    const int g_shared = p.g[tid];
    const Elem* Q = reinterpret_cast<const Elem*>(q_arg) + off;
    const Elem* dO = reinterpret_cast<const Elem*>(dout_arg) + off;
    const float* lse2 = lse2_arg + (size_t)tl.bh * L;
    const float* dsum = dsum_arg + (size_t)tl.bh * L;
    const int qa = r0 + 32 * wv, qv = qa + (lane & 31);
    const bool rows_live = qa < Lr;
    const int row = r + qv * dil;
    typename T::Op qop, dop;
    T::load_op(qop, qv < Lr ? Q + (size_t)row * 64 : nullptr, h2);
    T::load_op(dop, qv < Lr ? dO + (size_t)row * 64 : nullptr, h2);
    const float my_l2 = qv < Lr ? lse2[row] : kPosInf;
    const float my_d = qv < Lr ? dsum[row] : 0.f;

    asm volatile("" ::"s"(p.w), "s"(p.gstride), "s"(p.n_g), "s"(p.k), "s"(p.v), "s"(p.pad), "s"(p.dq));
    const int w = p.w;
    const int wr = causal ? 0 : w, span = w + wr;
    tile_extent(tl, w, wr);
    const Elem* K = reinterpret_cast<const Elem*>(p.k) + off;
    const Elem* V = reinterpret_cast<const Elem*>(p.v) + off;
    Elem* dQ = reinterpret_cast<Elem*>(p.dq) + off;
    const uint8_t* pad = p.pad ? p.pad + (size_t)tl.b * L : nullptr;
    const int gstride = p.gstride;
    const int gofs = tl.b * gstride;  // this sequence's global set
    const int ng = seq_globals(gstride, p.n_g, p.gcnt, tl.b);

    const int n_gst = (ng + kStageKeys - 1) / kStageKeys;
    // Random stages (every head undilated): draws of query block r0/64, then r0/64 + 1.
    const int* rnd_a = nullptr;
    const int* rnd_b = nullptr;
    int na_r = 0, nb_r = 0;
    if (kRandom) {
        const int qb0 = r0 / kRandomBlock;
        rnd_a = p.rnd + ((size_t)tl.h * p.rnd_nq + qb0) * p.rnd_r;
        rnd_b = rnd_a + p.rnd_r;
        while (na_r < p.rnd_r && rnd_a[na_r] >= 0) ++na_r;
        if (qb0 + 1 < p.rnd_nq)
            while (nb_r < p.rnd_r && rnd_b[nb_r] >= 0) ++nb_r;
    }
    auto rnd_block = [&](int j) { return j < na_r ? rnd_a[j] : rnd_b[j - na_r]; };
    const int n_rst = na_r + nb_r;
    const int n_lst = n_gst + n_rst;
    const int n_st = n_lst + tl.n_band;
    auto band_invalid = [&](int u) -> uint64_t {
        if (pad) return band_mask[u % kBwdMaskRing];
        const int ks = tl.stage_row(u);
        const int lo = tl.kb0 - ks, hi = tl.kend - ks;
        uint64_t m = 0;
        if (lo > 0) m |= lo >= 64 ? ~0ull : ((1ull << lo) - 1);
        if (hi < 64) m |= hi <= 0 ? ~0ull : (~0ull << hi);
        return m;
    };
    // A band stage's first key and invalid-key bits, computed when its copy is issued
    // (one iteration before it is computed) and reused there.
    int ks_next = 0;
    auto issue = [&](int s) -> uint64_t {
        char* slot = ring + (s & 1) * kStageB;
        if (s < n_gst) {
            const int* src = glob_src + kStageKeys * s;
            T::dma_tiles(slot, K, V, [&](int kk) { return src[kk]; }, wv, lane);
        } else if (kRandom && s < n_lst) {
            const int j = s - n_gst, kb0 = kRandomBlock * rnd_block(j);
            const uint64_t inv = uniform64(rnd_inv[j]);
            T::dma_tiles(slot, K, V, [&](int kk) { return ((inv >> kk) & 1) ? -1 : kb0 + kk; }, wv, lane);
        } else {
            const int u = s - n_lst;
            const uint64_t inv = uniform64(band_invalid(u));
            const int ks = tl.stage_row(u);
            ks_next = ks;
            T::dma_tiles(slot, K, V, [&](int kk) { return ((inv >> kk) & 1) ? -1 : r + (ks + kk) * dil; }, wv, lane);
            return inv;
        }
        return 0ull;
    };
    // Invalid-key bits (outside [kb0, kend) or padded) of band stages
    // [64*W, 64*W + 64): wave wv builds words wv, wv + 4, ... (all loads first).
    auto fill_band_masks = [&](int W) {
        constexpr int kPer = kBwdMaskWindow / kWaves;
        uint32_t flag[kPer];
        for (int j = 0; j < kPer; ++j) {
            const int u = W * kBwdMaskWindow + wv + kWaves * j;
            const int key = u < tl.n_band ? tl.stage_row(u) + lane : -1;
            flag[j] = (key >= tl.kb0 && key < tl.kend) ? pad[r + key * dil] : 1u;
        }
        for (int j = 0; j < kPer; ++j) {
            const int u = W * kBwdMaskWindow + wv + kWaves * j;
            const uint64_t inv = ballot64(flag[j] != 0);
            if (lane == 0 && u < tl.n_band) band_mask[u % kBwdMaskRing] = inv;
        }
    };

    if (const int gi = tid; gi < n_gst * kStageKeys) {  // slot gi is thread gi's
        int g = gi < ng ? g_shared : -1;
        if (gstride) {
            g = gi < ng ? p.g[gofs + gi] : -1;
            asm volatile("" ::"v"(g));  // awaited here: a wait after the branch would wait for the row loads too
        }
        const bool ok = g >= 0 && (!pad || pad[g] == 0);
        const int vpos = (g >= r && (g - r) % dil == 0) ? (g - r) / dil : kNoPos;
        glob_src[gi] = ok ? g : -1;
        glob_pos[gi] = ok ? vpos : kNoPos;
        glob_abs[gi] = g;
        glob_row[gi] = vpos;
    }
    if (tid < kRowsPerBlock / 32) row_glob[tid] = 0u;
    if (pad) fill_band_masks(0);
    if (kBias) fill_bias(bias_lds, p, tl.h, w, tid, false);
    barrier_lds();  // the row loads stay in flight
    if (wv == 0)
        for (int s = 0; s < n_gst; ++s) {
            const uint64_t inv = ~ballot64(glob_src[kStageKeys * s + lane] >= 0);
            if (lane == 0) glob_mask[s] = inv;
        }
    for (int gi = tid; gi < ng; gi += kThreads) {
        const int vr = glob_row[gi] - r0;
        if (vr >= 0 && vr < kRowsPerBlock) atomicOr(&row_glob[vr >> 5], 1u << (vr & 31));
    }
    if (kRandom)  // invalid keys of random stage j: past the end, padded or global
        for (int j = wv; j < n_rst; j += kWaves) {
            const int key = kRandomBlock * rnd_block(j) + lane;
            bool ok = key < L && (!pad || pad[key] == 0);
            if (ok && ng > 0) {
                const int c = count_le(glob_abs, ng, key);
                ok = !(c > 0 && glob_abs[c - 1] == key);
            }
            const uint64_t inv = ~ballot64(ok);
            if (lane == 0) rnd_inv[j] = inv;
        }
    barrier_lds();

    // One-sided variant: the global slots at or before this lane's row.
    const int gcnt = causal ? count_le(glob_abs, ng, row) : 0;
    typename T::Lanes lo;
    T::lane_setup(lo, lane);
    // Per-wave sums of dS per window offset (kBiasGrad): offset m at db_acc[m + w], with
    // kBiasPad slack entries on both sides for the offsets of masked pairs.
    const int db_len = 2 * w + 1 + 2 * kBiasPad;
    float* db_acc = db_lds + wv * db_len + kBiasPad;
    bool row_is_global = false;
    if (kBiasGrad) {
        for (int i = lane; i < db_len; i += 64) db_lds[wv * db_len + i] = 0.f;
        const int vr = qv - r0;
        row_is_global = qv < Lr && ((row_glob[vr >> 5] >> (vr & 31)) & 1u);
    }
    uint64_t inv_next = 0ull;
    if (n_st > 0) inv_next = issue(0);
    wait_vmcnt<0>();
    T::scale_op(qop);
    // The score product is seeded with -lse2 (its exponentials are the weights); D is
    // subtracted after the dP product instead of seeding it, which keeps one fewer
    // 16-register vector live across the loop.
    const f32x16 seed_s = splat(-my_l2);
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    for (int t = 0; t < n_st; ++t) {
        const uint64_t inv_cur = inv_next;
        const int ks_cur = ks_next;
        wait_vmcnt<0>();
        barrier_nofence();
        if (t + 1 < n_st) {
            const int bn = t + 1 - n_lst;
            if (pad && bn > 0 && bn % kBwdMaskWindow == 0) {
                fill_band_masks(bn / kBwdMaskWindow);
                __syncthreads();
            }
            inv_next = issue(t + 1);
        }
        const bool gstage = t < n_gst;
        const bool rstage = kRandom && !gstage && t < n_lst;
        const int j = t - n_gst;  // random stage index when rstage
        const int ks = gstage ? 0 : (rstage ? kRandomBlock * rnd_block(j) : ks_cur);
        const uint64_t inv = uniform64(gstage ? glob_mask[t] : (rstage ? rnd_inv[j] : inv_cur));
        const char* slot = ring + (t & 1) * kStageB;
        if (!rows_live || inv == ~0ull) continue;
        if (rstage && (wv >> 1) != (j < na_r ? 0 : 1)) continue;  // another query block's draw
        for (int sub = 0; sub < 2; ++sub) {
            const uint32_t inv32 = (uint32_t)(inv >> (32 * sub));
            const int kss = ks + 32 * sub;
            if (inv32 == ~0u) continue;
            if (rstage) {
                if (kss >= qa + 31 - w && kss + 31 <= qa + wr) continue;  // inside every row's window
                if (causal && kss > qa + 31) continue;                    // after every row
            } else if (!gstage && (kss > qa + 31 + wr || kss + 31 < qa - w)) {
                continue;
            }
            const bool interior = !gstage && !rstage && inv32 == 0u && kss >= qa + 31 - w && kss + 31 <= qa + wr;
            const int mode = rstage ? 3 : (gstage ? 2 : (interior ? 0 : 1));
            f32x16 s = T::prod(slot, sub, lo, qop, seed_s);  // scores - lse, base 2
            const int bbase = kss + 8 * h2 - qv + w;
            if (kBias && !gstage && !rstage) add_bias(s, bias_lds + kBiasPad + bbase);
            const int goff = kStageKeys * t + 32 * sub + 8 * h2;
            mask_scores<kRandom>(s, mode, inv32, h2, bbase, span, glob_pos + goff, w - qv,
                                 !causal ? 1 << 30 : (rstage ? w - bbase + 1 : gcnt - goff));
            const f32x16 dp = T::prod(slot + kTileB, sub, lo, dop, f32x16{});  // dO.V
            float ds[16];
            for (int i = 0; i < 16; ++i) ds[i] = fast_exp2(s[i]) * (dp[i] - my_d);
            if (kBiasGrad && !gstage && !rstage) {
                // element i of this lane: offset m = bbase - w + kc_of(i), at db_acc[m + w];
                // global rows get no bias
#pragma unroll
                for (int half = 0; half < 2; ++half)
                    if (h2 == half)
                        for (int i = 0; i < 16; ++i)
                            __hip_atomic_fetch_add(db_acc + bbase + kc_of(i), row_is_global ? 0.f : ds[i],
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            typename T::Frag f;
            T::to_frag(ds, f);
            typename T::TOp tk;
            T::load_t(tk, slot, sub, lo);
            acc_t<T>(tk, f, acc, lo);
        }
    }
    if (kBiasGrad) {  // this tile's sums per offset, waves added in order
        __syncthreads();
        float* dst = p.ws_db + ((size_t)tl.bh * p.tiles_per_head + tl.t_in) * (2 * w + 1);
        for (int m = tid; m < 2 * w + 1; m += kThreads) {
            float sum = 0.f;
            for (int x = 0; x < kWaves; ++x) sum += db_lds[x * db_len + kBiasPad + m];
            dst[m] = sum;
        }
    }
    if (qv < Lr) {
        const int vr = qv - r0;  // global rows: the merge
        if (!((row_glob[vr >> 5] >> (vr & 31)) & 1u)) {
            T::store_row(dQ + (size_t)row * 64, h2, acc, 0.125f);
            if (p.sep) T::store_row(reinterpret_cast<Elem*>(p.dqg) + off + (size_t)row * 64, h2, acc, 0.f);
        }
    }
    if (ng == 0) return;

    // Global rows (C): each wave takes one 32-key sub-tile of the home keys
    // [r0, r0 + 128) (the last two band stages, still in the ring for the first 32
    // global queries; copied again for the others, and from k_g, v_g with separate
    // projections, whose global queries are q_g).
    const bool sep = p.sep != 0;
    const Elem* QG = sep ? reinterpret_cast<const Elem*>(p.qg) + off : Q;
    const Elem* KG = sep ? reinterpret_cast<const Elem*>(p.kg) + off : K;
    const Elem* VG = sep ? reinterpret_cast<const Elem*>(p.vg) + off : V;
    const int ngq = p.n_gblk * kGlobalQueriesPerBlock;
    const size_t part0 = ((size_t)tl.bh * p.tiles_per_head + tl.t_in) * ngq;
    const int hs = wv >> 1, hsub = wv & 1;
    const int home_end = min(Lr, r0 + kRowsPerBlock);
    const int n_gblk_b = (ng + kGlobalQueriesPerBlock - 1) / kGlobalQueriesPerBlock;  // this sequence's blocks
    for (int gb = 0; gb < n_gblk_b; ++gb) {
        const int gq = gb * kGlobalQueriesPerBlock + (lane & 31);
        const int g = gq < ng ? p.g[gofs + gq] : -1;
        typename T::Op gop, gdo;
        T::load_op(gop, g >= 0 ? QG + (size_t)g * 64 : nullptr, h2);
        T::load_op(gdo, g >= 0 ? dO + (size_t)g * 64 : nullptr, h2);
        const float gl = g >= 0 ? lse2[g] : kPosInf;
        const float gd = g >= 0 ? dsum[g] : 0.f;
        const char* hslot;
        uint32_t inv32;
        if (gb == 0 && !sep) {
            const int u = tl.n_band - 2 + hs;
            hslot = ring + ((n_lst + u) & 1) * kStageB;
            inv32 = (uint32_t)(band_invalid(u) >> (32 * hsub));
            wait_vmcnt<0>();
        } else {
            uint64_t hinv[2];
            for (int j = 0; j < 2; ++j) {
                const int key = r0 + kStageKeys * j + lane;
                bool ok = key < home_end;
                if (ok && pad) ok = pad[r + key * dil] == 0;
                hinv[j] = uniform64(~ballot64(ok));
            }
            __syncthreads();  // the ring is free
            for (int j = 0; j < 2; ++j) {
                const uint64_t iv = hinv[j];
                const int ks = r0 + kStageKeys * j;
                T::dma_tiles(ring + j * kStageB, KG, VG,
                          [&](int kk) { return ((iv >> kk) & 1) ? -1 : r + (ks + kk) * dil; }, wv, lane);
            }
            wait_vmcnt<0>();
            __syncthreads();
            hslot = ring + hs * kStageB;
            inv32 = (uint32_t)((hs ? hinv[1] : hinv[0]) >> (32 * hsub));
        }
        T::scale_op(gop);
        f32x16 gacc[2] = {f32x16{}, f32x16{}};
        if (inv32 != ~0u) {
            f32x16 s = T::prod(hslot, hsub, lo, gop, splat(-gl));
            if (causal) {  // keys of this class at or before the global row
                const int vlim = g >= r ? (g - r) / dil : -1;
                const int kss = r0 + kStageKeys * hs + 32 * hsub;
                mask_scores(s, 1, inv32, h2, kss + 8 * h2 - vlim + kLargeW, kLargeW, nullptr, 0);
            } else {
                mask_scores(s, inv32 != 0u ? 1 : 0, inv32, h2, 0, 2 * kLargeW, nullptr, 0);
            }
            const f32x16 dp = T::prod(hslot + kTileB, hsub, lo, gdo, splat(-gd));
            float ds[16];
            for (int i = 0; i < 16; ++i) ds[i] = fast_exp2(s[i]) * dp[i];
            typename T::Frag f;
            T::to_frag(ds, f);
            typename T::TOp tk;
            T::load_t(tk, hslot, hsub, lo);
            acc_t<T>(tk, f, gacc, lo);
        }
        __syncthreads();  // done with the staged keys: the ring holds the reduction
        const int nq = min(kGlobalQueriesPerBlock, ng - gb * kGlobalQueriesPerBlock);
        wave_sum_store(reinterpret_cast<float*>(ring), gacc, wv, lane, tid,
                       p.ws_dq + (part0 + (size_t)gb * kGlobalQueriesPerBlock) * 64, nq);
    }
}

// ---------------------------------------------------------------------------
// dK, dV: one work-group per 128 keys of one residue class of one (b, h); wave wv
// owns keys r0 + 32*wv .. +31, one per lane.  Stages: the global queries (every
// unpadded key is theirs), then the window band of queries (global queries are
// removed there by lse2_band = +inf: their weights are 0).  With random blocks
// (kRandom, every head undilated) the query blocks that drew the tile's first key
// block (for waves 0-1), then those that drew its second (waves 2-3), come between
// the global queries and the band, one 64-query stage each; pairs that the window
// already holds, global own keys (their pairs are folded by the global-key pass) and
// queries past the end are masked.
//
// With separate projections of the global rows the global-query stages are left out
// here (their pairs use q_g, k_g, v_g), and kGlobalProj instantiates the kernel that
// computes them: own keys from k_g, v_g, the global queries from q_g as its only
// stages, every key's dK_g, dV_g written directly.

template <class T, bool kCausal, bool kBias, bool kRandom, bool kGlobalProj = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(T::kWavesPerEU)))
void bwd_dkv_kernel(const int nblk, const int tph, const int H, const int L, const int dil_u, const void* const k_arg,
                    const void* const v_arg, const uint8_t* const pad_arg, const BwdParams p) {
    using Elem = typename T::Elem;
    constexpr int kStageB = T::kStageB, kTileB = T::kTileB, kLseOff = T::kLseOff, kDOff = T::kDOff;
    __shared__ __attribute__((aligned(16))) char ring[2 * kStageB];
    __shared__ int own_gidx[kRowsPerBlock];  // index in g of each own key, or -1
    __shared__ int gq_pos[LF_MAX_GLOBALS];  // position of each global slot (sorted)
    __shared__ float bias_lds[kBias ? kBiasLds : 1];  // reversed: offset m at kBiasPad + w - m, base 2

    // Queries of a key: query - key in [-wl, w] class steps (wl = 0 one-sided: no query
    // before its key).
    constexpr bool causal = kCausal;
    // The leading arguments (grid size, p.tiles_per_head, p.H, p.L, p.dil_u, the own
    // key and value rows' tensors and p.pad) are preloaded into scalar registers by the
    // build, as in the dQ kernel; the shared global positions are loaded first and the
    // other arguments in one batch after the row loads are issued.
    Tile tl;
    if (!tile_of(tl, p, nblk, tph, H, L, dil_u)) return;
    const int tid = threadIdx.x, lane = tid & 63, h2 = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int dil = tl.dil, r = tl.r, r0 = tl.r0, Lr = tl.Lr;
    const size_t off = (size_t)tl.bh * L * 64;
    static_assert(kThreads == LF_MAX_GLOBALS, "one global slot per thread");
    const int g_shared = p.g[tid];
    const Elem* K = reinterpret_cast<const Elem*>(k_arg) + off;
    const Elem* V = reinterpret_cast<const Elem*>(v_arg) + off;
    const uint8_t* pad = pad_arg ? pad_arg + (size_t)tl.b * L : nullptr;
    const int qa = r0 + 32 * wv, qv = qa + (lane & 31);  // own keys (virtual index)
    const bool rows_live = qa < Lr;
    const int krow = r + qv * dil;
    const bool kvalid = qv < Lr && (!pad || pad[krow] == 0);
    typename T::Op kop, vop;
    T::load_op(kop, kvalid ? K + (size_t)krow * 64 : nullptr, h2);
    T::load_op(vop, kvalid ? V + (size_t)krow * 64 : nullptr, h2);

    asm volatile("" ::"s"(p.w), "s"(p.gstride), "s"(p.n_g), "s"(p.sep), "s"(kGlobalProj ? p.qg : p.q), "s"(p.dout),
                 "s"(p.lse2), "s"(p.lse2_band), "s"(p.dsum));
    const int w = p.w;
    const int wl = causal ? 0 : w, span = wl + w;
    tile_extent(tl, wl, w);
    const Elem* Q = reinterpret_cast<const Elem*>(kGlobalProj ? p.qg : p.q) + off;
    const Elem* dO = reinterpret_cast<const Elem*>(p.dout) + off;
    Elem* dK = reinterpret_cast<Elem*>(kGlobalProj ? p.dkg : p.dk) + off;
    Elem* dV = reinterpret_cast<Elem*>(kGlobalProj ? p.dvg : p.dv) + off;
    const float* lse2 = p.lse2 + (size_t)tl.bh * L;
    const float* lse2b = p.lse2_band + (size_t)tl.bh * L;
    const float* dsum = p.dsum + (size_t)tl.bh * L;
    const int gstride = p.gstride;
    const int gofs = tl.b * gstride;  // this sequence's global set
    const int ng = seq_globals(gstride, p.n_g, p.gcnt, tl.b);

    // global-query stages: none here with separate projections (their own launch)
    const int n_gst = (!kGlobalProj && p.sep) ? 0 : (ng + kStageKeys - 1) / kStageKeys;
    // Random stages: the query blocks that drew key block r0/64, then r0/64 + 1.
    const int* inv_a = nullptr;
    const int* inv_b = nullptr;
    int na_r = 0, nb_r = 0;
    if (kRandom) {
        const int kb0 = r0 / kRandomBlock;
        inv_a = p.rnd_inv + ((size_t)tl.h * p.rnd_nq + kb0) * p.rnd_inv_r;
        inv_b = inv_a + p.rnd_inv_r;
        while (na_r < p.rnd_inv_r && inv_a[na_r] >= 0) ++na_r;
        if (kb0 + 1 < p.rnd_nq)
            while (nb_r < p.rnd_inv_r && inv_b[nb_r] >= 0) ++nb_r;
    }
    auto rnd_qblock = [&](int j) { return j < na_r ? inv_a[j] : inv_b[j - na_r]; };
    const int n_lst = n_gst + na_r + nb_r;
    const int n_st = n_lst + (kGlobalProj ? 0 : tl.n_band);
    int ks_next = 0;  // first query of the band stage copied last, reused when it is computed
    auto issue = [&](int s) {
        char* slot = ring + (s & 1) * kStageB;
        if (s < n_gst) {
            auto row_of = [&](int kk) {
                const int gi = kStageKeys * s + kk;
                return gi < ng ? gq_pos[gi] : -1;
            };
            T::dma_tiles(slot, Q, dO, row_of, wv, lane);
            if (wv == 0) dma_floats<T>(slot, lse2, dsum, row_of, lane);
        } else if (kRandom && s < n_lst) {
            const int x0 = kRandomBlock * rnd_qblock(s - n_gst);
            auto row_of = [&](int kk) { return x0 + kk < L ? x0 + kk : -1; };
            T::dma_tiles(slot, Q, dO, row_of, wv, lane);
            if (wv == 0) dma_floats<T>(slot, lse2b, dsum, row_of, lane);
        } else {
            const int ks = tl.stage_row(s - n_lst);
            ks_next = ks;
            auto row_of = [&](int kk) {
                const int x = ks + kk;
                return (x >= tl.kb0 && x < tl.kend) ? r + x * dil : -1;
            };
            T::dma_tiles(slot, Q, dO, row_of, wv, lane);
            if (wv == 0) dma_floats<T>(slot, lse2b, dsum, row_of, lane);
        }
    };

    if (tid < kRowsPerBlock) own_gidx[tid] = -1;
    if (const int gi = tid; gi < ng) {  // slot gi is thread gi's (ng <= LF_MAX_GLOBALS)
        int g = g_shared;
        if (gstride) {
            g = p.g[gofs + gi];
            asm volatile("" ::"v"(g));  // awaited here: a wait after the branch would wait for the row loads too
        }
        gq_pos[gi] = g;
    }
    if (kBias) fill_bias(bias_lds, p, tl.h, w, tid, true);
    barrier_lds();  // the row loads stay in flight
    for (int gi = tid; gi < ng; gi += kThreads) {
        const int g = gq_pos[gi];
        if (g >= r && (g - r) % dil == 0) {
            const int vr = (g - r) / dil - r0;
            if (vr >= 0 && vr < kRowsPerBlock) own_gidx[vr] = gi;
        }
    }
    barrier_lds();

    // One-sided variant: the first global slot at or after this lane's key (the
    // global queries that see it; slots are sorted by position).
    const int gfirst = causal ? count_le(gq_pos, ng, krow - 1) : 0;
    typename T::Lanes lo;
    T::lane_setup(lo, lane);
    if (n_st > 0) issue(0);
    wait_vmcnt<0>();
    T::scale_op(kop);
    f32x16 dk[2] = {f32x16{}, f32x16{}}, dv[2] = {f32x16{}, f32x16{}};
    // Random stages: an own key that is global takes its random pairs from the
    // global-key pass instead.
    const bool own_global = kRandom && qv < Lr && own_gidx[qv - r0] >= 0;
    for (int t = 0; t < n_st; ++t) {
        const int ks_cur = ks_next;
        wait_vmcnt<0>();
        barrier_nofence();
        if (t + 1 < n_st) issue(t + 1);
        const bool gstage = t < n_gst;
        const bool rstage = kRandom && !gstage && t < n_lst;
        const int j = t - n_gst;  // random stage index when rstage
        const int ks = gstage ? 0 : (rstage ? kRandomBlock * rnd_qblock(j) : ks_cur);
        const char* slot = ring + (t & 1) * kStageB;
        if (!rows_live) continue;
        if (rstage && (wv >> 1) != (j < na_r ? 0 : 1)) continue;  // a draw of the other key block
        for (int sub = 0; sub < 2; ++sub) {
            const int kss = ks + 32 * sub;
            if (gstage) {
                if (kss >= ng) continue;
            } else if (rstage) {
                if (kss >= L) continue;                                    // no valid query
                if (kss >= qa + 31 - wl && kss + 31 <= qa + w) continue;  // every pair in the window
                if (causal && kss + 31 < qa) continue;                     // every query before every key
            } else {
                if (kss > qa + 31 + w || kss + 31 < qa - wl) continue;  // outside every own key's window
                if (kss >= tl.kend || kss + 31 < tl.kb0) continue;      // no valid query
            }
            const bool interior = !gstage && !rstage && kss >= qa + 31 - wl && kss + 31 <= qa + w;
            const int mode = rstage ? 3 : ((gstage || interior) ? 0 : 1);
            f32x16 s = T::prod(slot, sub, lo, kop, row_seed(slot + kLseOff, sub, h2));  // scores - lse, base 2
            // element i: query kss + 8*h2 + kc, key qv, offset m = qv - query: reversed table
            if (kBias && !gstage && !rstage) add_bias(s, bias_lds + kBiasPad + kss + 8 * h2 - qv + w);
            // Random stage: invalid queries are those past the end.
            const uint32_t rinv = rstage ? ~bits_below(L - kss) : 0u;
            mask_scores<kRandom>(s, mode, rinv, h2, kss + 8 * h2 - qv + wl, span, nullptr, 0);
            if (rstage) {  // one-sided: no query before the key; global own keys: none
                uint32_t keep = own_global ? 0u : ~0u;
                if (causal) keep &= bits_from(qv - (kss + 8 * h2));
                for (int i = 0; i < 16; ++i)
                    if (!((keep >> kc_of(i)) & 1u)) s[i] = kNegInf;
            }
            if (gstage && causal) {  // a global query sees no key after it: slots from gfirst on
                const uint32_t keep = bits_from(gfirst - (kStageKeys * t + 32 * sub + 8 * h2));
                for (int i = 0; i < 16; ++i)
                    if (!((keep >> kc_of(i)) & 1u)) s[i] = kNegInf;
            }
            const f32x16 dp = T::prod(slot + kTileB, sub, lo, vop, row_seed(slot + kDOff, sub, h2));  // dO.V - D
            float pr[16], ds[16];
            for (int i = 0; i < 16; ++i) {
                pr[i] = fast_exp2(s[i]);
                ds[i] = pr[i] * dp[i];
            }
            typename T::Frag fp, fs;
            T::to_frag(pr, fp);
            T::to_frag(ds, fs);
            typename T::TOp tt;
            T::load_t(tt, slot + kTileB, sub, lo);
            acc_t<T>(tt, fp, dv, lo);
            T::load_t(tt, slot, sub, lo);
            acc_t<T>(tt, fs, dk, lo);
        }
    }
    const int ngq = p.n_gblk * kGlobalQueriesPerBlock;
    if (qv < Lr) {
        const int gi = kGlobalProj ? -1 : own_gidx[qv - r0];
        const float sk = kvalid ? 0.125f : 0.f, sv = kvalid ? 1.f : 0.f;
        if (gi < 0) {
            T::store_row(dK + (size_t)krow * 64, h2, dk, sk);
            T::store_row(dV + (size_t)krow * 64, h2, dv, sv);
        } else {  // global key: completed by the merge (unscaled fp32)
            store_row_f32(p.ws_dkg + ((size_t)tl.bh * ngq + gi) * 64, h2, dk, kvalid ? 1.f : 0.f);
            store_row_f32(p.ws_dvg + ((size_t)tl.bh * ngq + gi) * 64, h2, dv, sv);
        }
    }
    if (kGlobalProj || ng == 0) return;

    // Global keys (B): lane = global key, elements = the home queries of one 32-row
    // sub-tile per wave, minus the queries whose window holds the key (those pairs
    // are in the key's own tile) and minus global queries (lse2_band = +inf).
    const size_t part0 = ((size_t)tl.bh * p.tiles_per_head + tl.t_in) * ngq;
    const int hs = wv >> 1, hsub = wv & 1;
    const int hq = r0 + kStageKeys * hs + 32 * hsub;  // first home query of this wave
    const int n_gblk_b = (ng + kGlobalQueriesPerBlock - 1) / kGlobalQueriesPerBlock;  // this sequence's blocks
    for (int gb = 0; gb < n_gblk_b; ++gb) {
        const int gk = gb * kGlobalQueriesPerBlock + (lane & 31);
        const int g = gk < ng ? p.g[gofs + gk] : -1;
        const bool gvalid = g >= 0 && (!pad || pad[g] == 0);
        typename T::Op kg, vg;
        T::load_op(kg, gvalid ? K + (size_t)g * 64 : nullptr, h2);
        T::load_op(vg, gvalid ? V + (size_t)g * 64 : nullptr, h2);
        const int vpos = (g >= r && (g - r) % dil == 0) ? (g - r) / dil : kNoPos;
        const char* hslot;
        if (gb == 0) {
            const int u = tl.n_band - 2 + hs;
            hslot = ring + ((n_lst + u) & 1) * kStageB;
            wait_vmcnt<0>();
        } else {
            __syncthreads();  // the ring is free
            for (int j = 0; j < 2; ++j) {
                const int ks = r0 + kStageKeys * j;
                auto row_of = [&](int kk) {
                    const int x = ks + kk;
                    return x < Lr ? r + x * dil : -1;
                };
                T::dma_tiles(ring + j * kStageB, Q, dO, row_of, wv, lane);
                if (wv == 0) dma_floats<T>(ring + j * kStageB, lse2b, dsum, row_of, lane);
            }
            wait_vmcnt<0>();
            __syncthreads();
            hslot = ring + hs * kStageB;
        }
        T::scale_op(kg);
        f32x16 gk_acc[2] = {f32x16{}, f32x16{}}, gv_acc[2] = {f32x16{}, f32x16{}};
        if (hq < Lr) {
            f32x16 s = T::prod(hslot, hsub, lo, kg, row_seed(hslot + kLseOff, hsub, h2));
            // Queries kept, one bit per kc (element i holds query base + kc_of(i)): below
            // Lr, not in the window that holds the key (those pairs are in the key's own
            // tile), and, one-sided, not before the key.  Built as bit ranges so that the
            // selection stays branch-free.
            const int base = hq + 8 * h2;
            uint32_t keep = gvalid ? bits_below(Lr - base) : 0u;
            keep &= ~(bits_from(vpos - wl - base) & bits_below(vpos + p.w + 1 - base));
            if (causal) keep &= bits_from((g > r ? (g - r + dil - 1) / dil : 0) - base);
            for (int i = 0; i < 16; ++i)
                if (!((keep >> kc_of(i)) & 1u)) s[i] = kNegInf;
            const f32x16 dp = T::prod(hslot + kTileB, hsub, lo, vg, row_seed(hslot + kDOff, hsub, h2));
            float pr[16], ds[16];
            for (int i = 0; i < 16; ++i) {
                pr[i] = fast_exp2(s[i]);
                ds[i] = pr[i] * dp[i];
            }
            typename T::Frag fp, fs;
            T::to_frag(pr, fp);
            T::to_frag(ds, fs);
            typename T::TOp tt;
            T::load_t(tt, hslot + kTileB, hsub, lo);
            acc_t<T>(tt, fp, gv_acc, lo);
            T::load_t(tt, hslot, hsub, lo);
            acc_t<T>(tt, fs, gk_acc, lo);
        }
        __syncthreads();  // done with the staged queries: the ring holds the reductions
        const int nq = min(kGlobalQueriesPerBlock, ng - gb * kGlobalQueriesPerBlock);
        const size_t dst = (part0 + (size_t)gb * kGlobalQueriesPerBlock) * 64;
        wave_sum_store(reinterpret_cast<float*>(ring), gk_acc, wv, lane, tid, p.ws_dk + dst, nq);
        wave_sum_store(reinterpret_cast<float*>(ring), gv_acc, wv, lane, tid, p.ws_dv + dst, nq);
    }
}

// ---------------------------------------------------------------------------
// Global rows and keys: one work-group of W <= kBwdMergeWaves waves per (global index,
// h, b) (grid x, y, z), lane = column (W = blockDim / 64, chosen by the host).  Wave x sums tiles
// x, x + W, ... (the loads of kBwdMergeChunk tiles issued together, absent tiles read
// tile 0 and are dropped), then the wave sums are added in wave order.

constexpr int kBwdMergeWaves = 16;
constexpr int kBwdMergeChunk = 8;
//
// The leading arguments (p.tiles_per_head, the partial rows per tile n_gblk * 32, p.H,
// p.L, p.dil_u and the three partial arrays) are preloaded into scalar registers by the
// build, so the partial loads wait for no argument; the others are read while those
// loads are in flight.  kDilU: every head has dilation dil_u (no read of p.dil).
template <class T, bool kDilU>
__global__ __launch_bounds__(64 * kBwdMergeWaves) void bwd_merge_kernel(const int tph, const int ngq, const int H,
                                                                        const int L, const int dil_u,
                                                                        const float* const ws_dq,
                                                                        const float* const ws_dk,
                                                                        const float* const ws_dv, const BwdParams p) {
    using Elem = typename T::Elem;
    __shared__ float red[kBwdMergeWaves][3][64];
    const int gi = blockIdx.x, h = blockIdx.y, bseq = blockIdx.z, d = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int bh = bseq * H + h, dil = kDilU ? dil_u : p.dil[h];
    const int W = merge_waves(tph, kBwdMergeChunk, kBwdMergeWaves);  // = blockDim.x / 64
    const int tpr = dil == 1 ? 0 : ((L + dil - 1) / dil + kRowsPerBlock - 1) / kRowsPerBlock;  // unused when dil == 1
    // gi < n_g <= ngq: the loads below stay in bounds even for a sequence with fewer
    // globals, whose work-groups drop what they loaded and return after the loop.
    const size_t base = (size_t)bh * tph * ngq * 64 + (size_t)gi * 64 + d;
    const int n_g = p.n_g, gstride = p.gstride, cnt = p.gcnt[bseq], g_shared = p.g[gi];
    // the global key's own-tile dK and dV (wave 0 adds them), loaded with the first chunk
    const size_t own = ((size_t)bh * ngq + gi) * 64 + d;
    const float own_k = wv == 0 ? p.ws_dkg[own] : 0.f, own_v = wv == 0 ? p.ws_dvg[own] : 0.f;
    float sq = 0.f, sk = 0.f, sv = 0.f;
    for (int c0 = 0; c0 * W < tph; c0 += kBwdMergeChunk) {
        float a[kBwdMergeChunk], b[kBwdMergeChunk], c[kBwdMergeChunk];
        bool ex[kBwdMergeChunk];
#pragma unroll
        for (int j = 0; j < kBwdMergeChunk; ++j) {
            const int t = (c0 + j) * W + wv;
            ex[j] = t < tph && tile_exists(t, tpr, dil, L, kRowsPerBlock);
        }
        __builtin_amdgcn_sched_barrier(0);  // every test before the first load
#pragma unroll
        for (int j = 0; j < kBwdMergeChunk; ++j) {
            const size_t idx = base + (ex[j] ? (size_t)((c0 + j) * W + wv) * ngq * 64 : 0);
            a[j] = ws_dq[idx];
            b[j] = ws_dk[idx];
            c[j] = ws_dv[idx];
        }
#pragma unroll
        for (int j = 0; j < kBwdMergeChunk; ++j) {
            sq += ex[j] ? a[j] : 0.f;
            sk += ex[j] ? b[j] : 0.f;
            sv += ex[j] ? c[j] : 0.f;
        }
    }
    if (gi >= (gstride ? cnt : n_g)) return;  // this sequence has fewer globals
    const int g = gstride ? p.g[bseq * gstride + gi] : g_shared;  // position of this global row
    red[wv][0][d] = sq;
    red[wv][1][d] = sk;
    red[wv][2][d] = sv;
    __syncthreads();
    if (wv != 0) return;
    sq = 0.f;
    sk = own_k;
    sv = own_v;
    for (int x = 0; x < W; ++x) {
        sq += red[x][0][d];
        sk += red[x][1][d];
        sv += red[x][2][d];
    }
    const size_t o = (size_t)bh * L * 64 + (size_t)g * 64 + d;
    // with separate projections a global row's dQ goes to dq_g and its dq is zero
    if (p.sep) reinterpret_cast<Elem*>(p.dqg)[o] = T::from_float(sq * 0.125f);
    reinterpret_cast<Elem*>(p.dq)[o] = T::from_float(p.sep ? 0.f : sq * 0.125f);
    reinterpret_cast<Elem*>(p.dk)[o] = T::from_float(sk * 0.125f);
    reinterpret_cast<Elem*>(p.dv)[o] = T::from_float(sv);
}

}  // namespace

namespace {

template <class T>
hipError_t bwd_prep_t(const BwdParams& p, hipStream_t s) {
    const long long blocks = (long long)p.B * p.H * ((p.L + kPrepRowsPerBlock - 1) / kPrepRowsPerBlock);
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    launch_kernel(bwd_prep_kernel<T>, dim3((unsigned)blocks), dim3(kThreads), s, p);
    return hipGetLastError();
}

template <class T>
hipError_t bwd_dq_t(const BwdParams& p, hipStream_t s) {
    const int blocks = p.B * p.H * p.tiles_per_head;
    if (blocks <= 0) return hipSuccess;
    // leading arguments, preloaded into scalar registers (see the kernel)
#define LF_DQ_ARGS blocks, p.tiles_per_head, p.H, p.L, p.dil_u, p.q, p.dout, (const float*)p.lse2, (const float*)p.dsum, p
    if (p.dbias) {  // position-bias table gradient: per-wave offset sums in dynamic LDS
        const unsigned shm = kWaves * (2 * p.w + 1 + 2 * kBiasPad) * sizeof(float);
        if (p.rnd) {
            if (p.causal)
                return launch_kernel_shm(bwd_dq_kernel<T, true, true, true, true>, dim3(blocks), dim3(kThreads), shm, s, LF_DQ_ARGS);
            return launch_kernel_shm(bwd_dq_kernel<T, false, true, true, true>, dim3(blocks), dim3(kThreads), shm, s, LF_DQ_ARGS);
        }
        if (p.causal)
            return launch_kernel_shm(bwd_dq_kernel<T, true, true, false, true>, dim3(blocks), dim3(kThreads), shm, s, LF_DQ_ARGS);
        return launch_kernel_shm(bwd_dq_kernel<T, false, true, false, true>, dim3(blocks), dim3(kThreads), shm, s, LF_DQ_ARGS);
    }
#define LF_DQ(C, Bi, R) launch_kernel(bwd_dq_kernel<T, C, Bi, R>, dim3(blocks), dim3(kThreads), s, LF_DQ_ARGS)
#define LF_DQ_R(C, Bi) \
    if (p.rnd) LF_DQ(C, Bi, true); else LF_DQ(C, Bi, false)
    if (p.causal) {
        if (p.bias) { LF_DQ_R(true, true); } else { LF_DQ_R(true, false); }
    } else {
        if (p.bias) { LF_DQ_R(false, true); } else { LF_DQ_R(false, false); }
    }
#undef LF_DQ_R
#undef LF_DQ
#undef LF_DQ_ARGS
    return hipGetLastError();
}

template <class T>
hipError_t bwd_dkv_t(const BwdParams& p, hipStream_t s) {
    const int blocks = p.B * p.H * p.tiles_per_head;
    if (blocks <= 0) return hipSuccess;
#define LF_DKV(C, Bi, R)                                                                                   \
    launch_kernel(bwd_dkv_kernel<T, C, Bi, R>, dim3(blocks), dim3(kThreads), s, blocks, p.tiles_per_head, p.H, p.L, \
                  p.dil_u, p.k, p.v, p.pad, p)
#define LF_DKV_R(C, Bi) \
    if (p.rnd) LF_DKV(C, Bi, true); else LF_DKV(C, Bi, false)
    if (p.causal) {
        if (p.bias) { LF_DKV_R(true, true); } else { LF_DKV_R(true, false); }
    } else {
        if (p.bias) { LF_DKV_R(false, true); } else { LF_DKV_R(false, false); }
    }
#undef LF_DKV_R
#undef LF_DKV
    return hipGetLastError();
}

template <class T>
hipError_t bwd_dkv_global_proj_t(const BwdParams& p, hipStream_t s) {
    const int blocks = p.B * p.H * p.tiles_per_head;
    if (blocks <= 0) return hipSuccess;
    if (p.causal)
        launch_kernel(bwd_dkv_kernel<T, true, false, false, true>, dim3(blocks), dim3(kThreads), s, blocks,
                      p.tiles_per_head, p.H, p.L, p.dil_u, p.kg, p.vg, p.pad, p);
    else
        launch_kernel(bwd_dkv_kernel<T, false, false, false, true>, dim3(blocks), dim3(kThreads), s, blocks,
                      p.tiles_per_head, p.H, p.L, p.dil_u, p.kg, p.vg, p.pad, p);
    return hipGetLastError();
}

template <class T>
hipError_t bwd_merge_t(const BwdParams& p, hipStream_t s) {
    if (p.n_g == 0 || p.B == 0) return hipSuccess;
    if (p.B > 65535) return hipErrorInvalidConfiguration;  // grid z
    const int waves = merge_waves(p.tiles_per_head, kBwdMergeChunk, kBwdMergeWaves);
    const int ngq = p.n_gblk * kGlobalQueriesPerBlock;
    if (p.dil_u)
        launch_kernel(bwd_merge_kernel<T, true>, dim3(p.n_g, p.H, p.B), dim3(64 * waves), s, p.tiles_per_head, ngq, p.H,
                      p.L, p.dil_u, (const float*)p.ws_dq, (const float*)p.ws_dk, (const float*)p.ws_dv, p);
    else
        launch_kernel(bwd_merge_kernel<T, false>, dim3(p.n_g, p.H, p.B), dim3(64 * waves), s, p.tiles_per_head, ngq,
                      p.H, p.L, p.dil_u, (const float*)p.ws_dq, (const float*)p.ws_dk, (const float*)p.ws_dv, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep(const BwdParams& p, hipStream_t s) {
    return p.dtype == LF_F32 ? bwd_prep_t<BF32>(p, s) : bwd_prep_t<BBf16>(p, s);
}
hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t s) {
    return p.dtype == LF_F32 ? bwd_dq_t<BF32>(p, s) : bwd_dq_t<BBf16>(p, s);
}
hipError_t launch_bwd_dkv(const BwdParams& p, hipStream_t s) {
    return p.dtype == LF_F32 ? bwd_dkv_t<BF32>(p, s) : bwd_dkv_t<BBf16>(p, s);
}
hipError_t launch_bwd_dkv_global_proj(const BwdParams& p, hipStream_t s) {
    return p.dtype == LF_F32 ? bwd_dkv_global_proj_t<BF32>(p, s) : bwd_dkv_global_proj_t<BBf16>(p, s);
}

// dbias[h][m] = sum over sequences b and the existing tiles t of head h (in that order)
// of ws_db[b*H + h][t][m]: one thread per (h, m).  The table has 2*bias_w + 1 entries;
// the kernels ran with w = min(bias_w, L), and the offsets beyond that (no pair has
// them) get 0.
__global__ __launch_bounds__(256) void bwd_dbias_kernel(const BwdParams p) {
    const int h = blockIdx.y, n = 2 * p.w + 1;
    const int m = blockIdx.x * 256 + threadIdx.x;
    if (m >= 2 * p.bias_w + 1) return;
    const int mm = m - (p.bias_w - p.w);  // entry in the per-tile sums
    float sum = 0.f;
    if (mm >= 0 && mm < n) {
        const int dil = p.dil[h], L = p.L;
        const int tpr = ((L + dil - 1) / dil + kRowsPerBlock - 1) / kRowsPerBlock;
        for (int b = 0; b < p.B; ++b) {
            const float* src = p.ws_db + (size_t)(b * p.H + h) * p.tiles_per_head * n + mm;
            for (int t = 0; t < p.tiles_per_head; ++t)
                if (tile_exists(t, tpr, dil, L, kRowsPerBlock)) sum += src[(size_t)t * n];
        }
    }
    p.dbias[(size_t)h * (2 * p.bias_w + 1) + m] = sum;
}

hipError_t launch_bwd_dbias(const BwdParams& p, hipStream_t s) {
    if (!p.dbias || p.H <= 0) return hipSuccess;
    const int n = 2 * p.bias_w + 1;
    return launch_kernel(bwd_dbias_kernel, dim3((n + 255) / 256, p.H), dim3(256), s, p);
}

hipError_t launch_bwd_merge(const BwdParams& p, hipStream_t s) {
    return p.dtype == LF_F32 ? bwd_merge_t<BF32>(p, s) : bwd_merge_t<BBf16>(p, s);
}

}  // namespace lf
