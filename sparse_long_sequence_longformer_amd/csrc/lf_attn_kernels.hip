// gfx950 (MI355X) kernels of the Longformer window + global attention forward.
//
// band_kernel: one work-group per 128 rows of one residue class of one (b, h):
//   (a) window band: the window keys of every row of the tile, streamed through
//       LDS in 64-key stages;
//   (b) global columns: the global keys outside each row's window, folded into the
//       same online softmax before the band;
//   (c) global rows: each work-group folds the global queries over its own 128
//       "home" keys and writes one partial (max, sum, unnormalised output) per query.
// merge_kernel:
//   (d) log-sum-exp merge of those partials in tile order; writes the global rows.
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
// Data movement: K and V stages of 64 keys go from HBM/L2 straight into LDS with
// global_load_lds_dwordx4 (no VGPR round trip), into a ring of stages so that the
// loads of the next stages are in flight while the current one is computed.  Keys
// that are padded, out of range or unused read a static zero row, so their LDS rows
// are zero and their contents never reach the output.  V stays row-major in LDS
// and the P.V product reads it transposed with ds_read_b64_tr_b16.
//
// Softmax: Q is pre-multiplied by log2(e)/sqrt(d_h), so the score product yields
// base-2 exponents, and the product is seeded with minus the query's running max,
// so the weights are exp2 of the accumulators as they come out.  The running max
// is raised lazily: a tile goes through the fast path (no max reduction) when its
// weight sum, taken by a small matrix product, stays at most 2^8; only tiles above
// that bound (or a query's first valid tile) compute a max and rescale.
//
// Register layout (v_mfma_f32_32x32x*): accumulator element i of lane l sits at
// row 8*(i/4) + 4*(l/32) + (i%4), column l%32.  Scores are computed transposed
// (rows = keys, columns = queries) so each lane owns one query: its row statistics
// need one exchange with the lane 32 away, and its 16 score values feed the P^T
// operand of the next product unchanged.  K rows are read in the order sigma(M) so
// that accumulator element i of lane-half h2 holds key 16*(i/8) + 8*h2 + (i%8).

#include <mutex>
#include <type_traits>

#include "lf_attn_device.h"

namespace lf {
namespace {

constexpr int kMaskWindow = 64;           // band stages whose pad masks are built at once
constexpr int kMergeWaves = 16;           // merge_kernel: most waves per work-group
constexpr int kMergeChunk = 8;            // merge_kernel: tiles whose loads a wave issues together
constexpr int kMaskRing = 2 * kMaskWindow;
constexpr int kMaxGlobalStages = LF_MAX_GLOBALS / kStageKeys;
constexpr int kAllParts = -1;     // dma_stage: every block of the wave

#ifndef LF_BF16_WAVES_PER_EU
#define LF_BF16_WAVES_PER_EU 3
#endif
#ifndef LF_BF16_NS
#define LF_BF16_NS 2
#endif

// ---------------------------------------------------------------------------
// Element-type traits: operand loads, stage DMA, the two products, output store.
// A stage holds 64 keys: K (64 x 64) then V (64 x 64), both row-major.  Output
// column d of lane (query, h2) accumulator element i is 32*db + 8*(i/4) + 4*h2 + i%4.

struct Bf16 {
    using Elem = uint16_t;
    static constexpr int kRowBytes = 128;
    static constexpr int kTileBytes = kStageKeys * kRowBytes;  // 8 KiB
    static constexpr int kStageBytes = 2 * kTileBytes;        // K + V
    static constexpr int kNS = LF_BF16_NS;                    // stages in the LDS ring
    static constexpr int kDmaPerStage = 4;                    // per wave: 2 for K, 2 for V
    static constexpr int kWavesPerEU = LF_BF16_WAVES_PER_EU;
    struct QOp { bf16x8 v[4]; };
    struct PFrag { bf16x8 v[2]; };

    // B operand of S^T = K Q^T: lane (query, h2) holds d = 16*kb + 8*h2 + j.  The raw
    // load and the scaling by log2(e)/sqrt(d_h) (rounded back to bf16) are separate, so
    // the loads can stay in flight while other set-up work is issued.
    // row == nullptr reads the static zero row (no branch around the loads).
    __device__ __forceinline__ static void load_q(QOp& q, const Elem* row, int h2) {
        if (!row) row = reinterpret_cast<const Elem*>(g_zero_row);
        for (int kb = 0; kb < 4; ++kb)
            q.v[kb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + 16 * kb + 8 * h2));
    }
    __device__ __forceinline__ static void scale_q(QOp& q) {
        for (int kb = 0; kb < 4; ++kb) {
            const f32x8 f = __builtin_convertvector(q.v[kb], f32x8);
            q.v[kb] = __builtin_convertvector(f * kScaleLog2, bf16x8);
        }
    }

    // Stage DMA by all four waves: wave wv fills 1-KiB blocks 2*wv and 2*wv+1 of K
    // and of V (8 rows each), block 2*wv + part for part = 0, 1 (kAllParts: both).
    // row_of(kk) is the source row of stage key kk or -1; rs the row stride of K and
    // V in elements.
    template <class RowOf>
    __device__ __forceinline__ static void dma_stage(char* slot, const Elem* K, const Elem* V, int rs, RowOf row_of, int wv,
                                                     int lane, int part = kAllParts) {
        const Elem* zero = reinterpret_cast<const Elem*>(g_zero_row);
        for (int u = 0; u < 2; ++u) {
            if (part != kAllParts && u != part) continue;
            const int blk = 2 * wv + u;
            const int row = 8 * blk + (lane >> 3), cl = lane & 7;
            const int src = row_of(row);
            const Elem* kr = src >= 0 ? K + (size_t)src * rs : zero;
            const Elem* vr = src >= 0 ? V + (size_t)src * rs : zero;
            dma16(kr + 8 * (cl ^ swz_k(row)), slot + blk * 1024);
            dma16(vr + 8 * (cl ^ swz_v(row)), slot + kTileBytes + blk * 1024);
        }
    }

    // 32 rows copied to dst (row-major, 128 B each): wave wv copies rows 8*wv .. +7.
    template <class RowPtr>
    __device__ __forceinline__ static void dma_rows(char* dst, RowPtr row_ptr, int wv, int lane) {
        const int row = 8 * wv + (lane >> 3);
        dma16(row_ptr(row) + 8 * (lane & 7), dst + wv * 1024);
    }

    // Byte offsets of this lane's stage copies (block 2*wv) relative to the stage's
    // first source row, for stages whose 64 keys are all valid (consecutive class
    // rows `step` elements apart: dil times the row stride).  Block 2*wv+1 lies 8 rows
    // further (scalar base advanced by 8 steps); its rows differ from block 2*wv's in
    // bit 3 only, so swz_v is the same and swz_k differs by 4 (chunk bit 2: byte offset
    // bit 6).
    struct DmaLane { uint32_t k, v; int step; };
    __device__ __forceinline__ static void dma_lane(DmaLane& dl, int wv, int lane, int step) {
        const int row = 16 * wv + (lane >> 3), cl = lane & 7;
        const uint32_t r0b = (uint32_t)row * (uint32_t)step * (uint32_t)sizeof(Elem);
        dl.k = r0b + 16u * (uint32_t)(cl ^ swz_k(row));
        dl.v = r0b + 16u * (uint32_t)(cl ^ swz_v(row));
        dl.step = step;
    }
    __device__ __forceinline__ static void dma_stage_direct(char* slot, const Elem* K0, const Elem* V0, const DmaLane& dl, int wv) {
        for (int u = 0; u < 2; ++u) {
            const int blk = 2 * wv + u;
            const size_t adv = (size_t)u * 8 * dl.step;
            dma16s(K0 + adv, u ? dl.k ^ 64u : dl.k, slot + blk * 1024);
            dma16s(V0 + adv, dl.v, slot + kTileBytes + blk * 1024);
        }
    }

    // Per-lane LDS byte offsets of the operand reads, independent of the stage slot
    // and of the sub-tile (the swizzles only depend on the row modulo 8).
    struct Lane {
        int k[4];  // K operand: row sigma(M), chunk (2*kb + h2) ^ swz_k(row)
        int v[2];  // V^T operand: row 8*h2 + i/4 (+ 4*t + 16*kb + 32*sub), per column block db
        bf16x8 sel;  // A operand of the weight-sum product (see tile_sum)
    };
    __device__ __forceinline__ static void lane_offsets(Lane& lo, int lane) {
        const int row = sigma(lane & 31), h2 = lane >> 5;
        {
            const int m = lane & 15, g = lane >> 4;
            const __bf16 one = (m & 3) == 0 && ((m >> 2) & 1) == (g & 1) ? (__bf16)1.0f : (__bf16)0.0f;
            for (int j = 0; j < 8; ++j) lo.sel[j] = one;
        }
        for (int kb = 0; kb < 4; ++kb) lo.k[kb] = row * kRowBytes + (((2 * kb + h2) ^ swz_k(row)) << 4);
        const int g1 = (lane >> 4) & 1, i = lane & 15;
        const int vrow = 8 * h2 + (i >> 2);
        for (int db = 0; db < 2; ++db) {
            const int chunk = 4 * db + 2 * g1 + ((i & 3) >> 1);
            lo.v[db] = kTileBytes + vrow * kRowBytes + ((chunk ^ swz_v(vrow)) << 4) + 8 * (i & 1);
        }
    }
    // Operand reads of sub-tile `sub` with sub = 0 arguments (a wave that only ever
    // reads one sub-tile of each stage; the swizzles repeat every 8 rows).
    __device__ __forceinline__ static void shift_lane(Lane& lo, int sub) {
        for (int kb = 0; kb < 4; ++kb) lo.k[kb] += sub * 32 * kRowBytes;
        for (int db = 0; db < 2; ++db) lo.v[db] += sub * 32 * kRowBytes;
    }

    // seed + S^T (32 keys x 32 queries) of sub-tile `sub` (keys 32*sub .. 32*sub+31 of
    // the stage).  The four K operand reads go out before the first product (left to
    // itself the scheduler reuses one register quad and waits for each read in turn).
    __device__ __forceinline__ static f32x16 qk(const char* slot, int sub, const Lane& lo, const QOp& q, const f32x16& seed) {
        const char* base = slot + sub * 32 * kRowBytes;
        bf16x8 a[4];
        for (int kb = 0; kb < 4; ++kb) a[kb] = *reinterpret_cast<const bf16x8*>(base + lo.k[kb]);
        f32x16 acc = seed;
        for (int kb = 0; kb < 4; ++kb) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], q.v[kb], acc, 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        return acc;
    }

    // Round the weights to bf16: the P^T operand.
    __device__ __forceinline__ static void to_p(const float* p, PFrag& pf) {
        for (int kb = 0; kb < 2; ++kb) {
            f32x8 t;
            for (int j = 0; j < 8; ++j) t[j] = p[8 * kb + j];
            pf.v[kb] = __builtin_convertvector(t, bf16x8);
        }
    }

    // Sum of the 32 rounded weights of the lane's query (both halves), in both lanes
    // of the pair, from two 16x16x32 products with P^T as the B operand.  In that
    // shape lane l holds B rows 8*(l/16) .. +7 of column l%16, i.e. query l%16 +
    // 16*((l/16)&1), key half (l/16)>>1; and result element 0 of lane l is row
    // 4*(l/16), column l%16.  A rows 0 and 8 select the B row groups of query n =
    // column, rows 4 and 12 those of query n + 16; so element 0 of lane l is the sum
    // of query l%32, the lane's own query.  The bf16 vector units share the matrix
    // cores' datapath, which makes this cheaper than a dot-product chain.
    __device__ __forceinline__ static float tile_sum(const PFrag& pf, const float*, const Lane& lo) {
        f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo.sel, pf.v[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo.sel, pf.v[1], acc, 0, 0, 0);
        return acc[0];
    }

    // O^T += V^T P^T over the 32 keys of sub-tile `sub`.  The V^T operand (lane l:
    // column 32*db + l%32, keys 16*kb + 8*h2 + 0..7) comes from two transposed
    // reads: within each 16-lane group, input lane i addresses row base + i/4,
    // columns 4*(i%4)..+3, and output lane o receives column o of rows base..base+3.
    // Rows base = 32*sub + 16*kb + 8*h2 + 4*t are multiples of 4, so the V swizzle
    // (row modulo 4) is the same for all of them.
    struct VOp { bf16x8 v[2][2]; };  // [db][kb]
    __device__ __forceinline__ static void load_v(VOp& vo, const char* slot, int sub, const Lane& lo) {
        const char* base = slot + sub * 32 * kRowBytes;
        for (int db = 0; db < 2; ++db)
            for (int kb = 0; kb < 2; ++kb) {
                const char* a = base + lo.v[db] + 16 * kb * kRowBytes;
                const s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LF_LDS(s16x4, a));
                const s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LF_LDS(s16x4, a + 4 * kRowBytes));
                vo.v[db][kb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7));
            }
    }
    __device__ __forceinline__ static void pv(const VOp& vo, const PFrag& pf, f32x16* o) {
        for (int kb = 0; kb < 2; ++kb)
            for (int db = 0; db < 2; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vo.v[db][kb], pf.v[kb], o[db], 0, 0, 0);
    }

    __device__ __forceinline__ static uint32_t pack_bf16(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
    }

    // Output row of the lane's query: accumulator group (db, q) of lane-half h2 holds
    // columns 32*db + 8*q + 4*h2 .. +3.  For each pair of groups q = 2m, 2m+1 the two
    // lanes of a query swap one group (lane-half 0 keeps q = 2m and takes the other
    // half's, lane-half 1 keeps q = 2m+1 and takes the other half's), so each lane holds
    // 8 consecutive columns 32*db + 16*m + 8*h2 .. +7: four 16-byte stores per lane, 32
    // contiguous bytes per row and instruction.  Every lane takes part in the swaps.
    struct RowOut { u32x4 c[2][2]; };  // [db][m]
    __device__ __forceinline__ static void pack_row(RowOut& ro, const f32x16* o, float scale) {
        for (int db = 0; db < 2; ++db)
            for (int m = 0; m < 2; ++m) {
                const int qe = 2 * m, qo = 2 * m + 1;
                const uint32_t e0 = pack_bf16(o[db][4 * qe] * scale, o[db][4 * qe + 1] * scale);
                const uint32_t e1 = pack_bf16(o[db][4 * qe + 2] * scale, o[db][4 * qe + 3] * scale);
                const uint32_t d0 = pack_bf16(o[db][4 * qo] * scale, o[db][4 * qo + 1] * scale);
                const uint32_t d1 = pack_bf16(o[db][4 * qo + 2] * scale, o[db][4 * qo + 3] * scale);
                // lanes 32-63 of the first operand swap with lanes 0-31 of the second
                const auto x0 = __builtin_amdgcn_permlane32_swap(e0, d0, false, false);
                const auto x1 = __builtin_amdgcn_permlane32_swap(e1, d1, false, false);
                ro.c[db][m] = u32x4{x0[0], x1[0], x0[1], x1[1]};
            }
    }
    __device__ __forceinline__ static void store_row(Elem* row, int h2, const RowOut& ro) {
        for (int db = 0; db < 2; ++db)
            for (int m = 0; m < 2; ++m) *reinterpret_cast<u32x4*>(row + 32 * db + 16 * m + 8 * h2) = ro.c[db][m];
    }

    __device__ __forceinline__ static Elem from_float(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
};

struct F32 {
    using Elem = float;
    static constexpr int kRowBytes = 256;
    static constexpr int kTileBytes = kStageKeys * kRowBytes;  // 16 KiB
    static constexpr int kStageBytes = 2 * kTileBytes;        // K + V
    static constexpr int kNS = 2;
    static constexpr int kDmaPerStage = 8;                    // per wave: 4 for K, 4 for V (kNS = 2: unused)
    static constexpr int kWavesPerEU = 1;
    struct QOp { float v[32]; };
    struct PFrag { float v[16]; };

    // B operand of S^T = K Q^T for the 32x32x2 product: step t, lane-half h2 -> d = 32*h2 + t;
    // scale_q multiplies by log2(e)/sqrt(d_h).
    __device__ __forceinline__ static void load_q(QOp& q, const Elem* row, int h2) {
        if (!row) row = reinterpret_cast<const Elem*>(g_zero_row);
        for (int t4 = 0; t4 < 8; ++t4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(row + 32 * h2 + 4 * t4);
            for (int e = 0; e < 4; ++e) q.v[4 * t4 + e] = x[e];
        }
    }
    __device__ __forceinline__ static void scale_q(QOp& q) {
        for (int i = 0; i < 32; ++i) q.v[i] *= kScaleLog2;
    }

    // Wave wv fills 1-KiB blocks 4*wv .. 4*wv+3 of K and of V (4 rows each); part
    // p = 0, 1 fills blocks 4*wv + 2*p and 4*wv + 2*p + 1 (kAllParts: all four).
    template <class RowOf>
    __device__ __forceinline__ static void dma_stage(char* slot, const Elem* K, const Elem* V, int rs, RowOf row_of, int wv,
                                                     int lane, int part = kAllParts) {
        const Elem* zero = reinterpret_cast<const Elem*>(g_zero_row);
        for (int u = 0; u < 4; ++u) {
            if (part != kAllParts && (u >> 1) != part) continue;
            const int blk = 4 * wv + u;
            const int row = 4 * blk + (lane >> 4), cl = lane & 15;
            const int src = row_of(row);
            const Elem* kr = src >= 0 ? K + (size_t)src * rs : zero;
            const Elem* vr = src >= 0 ? V + (size_t)src * rs : zero;
            dma16(kr + 4 * (cl ^ swz_k(row)), slot + blk * 1024);
            dma16(vr + 4 * cl, slot + kTileBytes + blk * 1024);
        }
    }

    // 32 rows copied to dst (row-major, 256 B each): wave wv copies rows 8*wv .. +7.
    template <class RowPtr>
    __device__ __forceinline__ static void dma_rows(char* dst, RowPtr row_ptr, int wv, int lane) {
        for (int u = 0; u < 2; ++u) {
            const int row = 8 * wv + 4 * u + (lane >> 4);
            dma16(row_ptr(row) + 4 * (lane & 15), dst + (2 * wv + u) * 1024);
        }
    }

    struct DmaLane { uint32_t k[4], v[4]; };
    __device__ __forceinline__ static void dma_lane(DmaLane& dl, int wv, int lane, int step) {
        for (int u = 0; u < 4; ++u) {
            const int row = 4 * (4 * wv + u) + (lane >> 4), cl = lane & 15;
            const uint32_t r0b = (uint32_t)row * (uint32_t)step * (uint32_t)sizeof(Elem);
            dl.k[u] = r0b + 16u * (uint32_t)(cl ^ swz_k(row));
            dl.v[u] = r0b + 16u * (uint32_t)cl;
        }
    }
    __device__ __forceinline__ static void dma_stage_direct(char* slot, const Elem* K0, const Elem* V0, const DmaLane& dl, int wv) {
        for (int u = 0; u < 4; ++u) {
            const int blk = 4 * wv + u;
            dma16s(K0, dl.k[u], slot + blk * 1024);
            dma16s(V0, dl.v[u], slot + kTileBytes + blk * 1024);
        }
    }

    struct Lane {
        int k;  // K operand row sigma(M) (chunks swizzled by swz_k)
        int sw;
        int h2;
        int v;  // V operand column 32*db + M of key key_local(u, h2): base of column M
    };
    __device__ __forceinline__ static void lane_offsets(Lane& lo, int lane) {
        const int row = sigma(lane & 31);
        lo.k = row * kRowBytes;
        lo.sw = swz_k(row);
        lo.h2 = lane >> 5;
        lo.v = kTileBytes + 4 * (lane & 31);
    }
    __device__ __forceinline__ static void shift_lane(Lane& lo, int sub) {
        lo.k += sub * 32 * kRowBytes;
        lo.v += sub * 32 * kRowBytes;
    }

    __device__ __forceinline__ static f32x16 qk(const char* slot, int sub, const Lane& lo, const QOp& q, const f32x16& seed) {
        const char* base = slot + sub * 32 * kRowBytes + lo.k;
        f32x16 acc = seed;
        for (int t4 = 0; t4 < 8; ++t4) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(base + (((8 * lo.h2 + t4) ^ lo.sw) << 4));
            for (int e = 0; e < 4; ++e)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], q.v[4 * t4 + e], acc, 0, 0, 0);
        }
        return acc;
    }

    __device__ __forceinline__ static void to_p(const float* p, PFrag& pf) {
        for (int i = 0; i < 16; ++i) pf.v[i] = p[i];
    }
    // Sum of the query's 32 weights, in both lanes of the pair.
    __device__ __forceinline__ static float tile_sum(const PFrag&, const float* p, const Lane&) {
        float sum[2] = {0.f, 0.f};
        for (int i = 0; i < 16; ++i) sum[i & 1] += p[i];
        return pair_sum(sum[0] + sum[1]);
    }

    // Step u pairs lane-half h2 with key key_local(u, h2), matching the score layout.
    struct VOp { const char* base; int h2; };
    __device__ __forceinline__ static void load_v(VOp& vo, const char* slot, int sub, const Lane& lo) {
        vo.base = slot + sub * 32 * kRowBytes + lo.v;
        vo.h2 = lo.h2;
    }
    __device__ __forceinline__ static void pv(const VOp& vo, const PFrag& pf, f32x16* o) {
        for (int db = 0; db < 2; ++db)
            for (int u = 0; u < 16; ++u) {
                const float a = *reinterpret_cast<const float*>(vo.base + key_local(u, vo.h2) * kRowBytes + 128 * db);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, pf.v[u], o[db], 0, 0, 0);
            }
    }

    struct RowOut { f32x16 o[2]; };
    __device__ __forceinline__ static void pack_row(RowOut& ro, const f32x16* o, float scale) {
        for (int db = 0; db < 2; ++db)
            for (int i = 0; i < 16; ++i) ro.o[db][i] = o[db][i] * scale;
    }
    __device__ __forceinline__ static void store_row(Elem* row, int h2, const RowOut& ro) {
        for (int db = 0; db < 2; ++db)
            for (int q = 0; q < 4; ++q) {
                f32x4 t;
                for (int j = 0; j < 4; ++j) t[j] = ro.o[db][4 * q + j];
                *reinterpret_cast<f32x4*>(row + 32 * db + 8 * q + 4 * h2) = t;
            }
    }

    __device__ __forceinline__ static Elem from_float(float x) { return x; }
};

// Wait until this wave's loads of the oldest outstanding stage have landed, given
// that `ahead` later stages have been issued since.
template <class T>
__device__ __forceinline__ void wait_stage(int ahead) {
    if constexpr (T::kNS > 2) {
        if (ahead >= 1) {
            wait_vmcnt<T::kDmaPerStage>();
            return;
        }
    }
    wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// Online softmax state of one lane.  Exponents are base 2 (scores come out of the
// product already multiplied by log2(e)/sqrt(d_h)).

struct State {
    float cofs;    // offset seeded into the score product (base 2): 0 until the query's
                   // first tile with a valid key, then that tile's largest score or more
    float l;       // running weight sum of the query (both lane halves), relative to cofs
    f32x16 seed;   // -cofs in every element
    f32x16 o[2];   // unnormalised output, relative to cofs
};

__device__ __forceinline__ void state_init(State& st) {
    st.cofs = 0.f;
    st.l = 0.f;
    st.seed = f32x16{};
    st.o[0] = f32x16{};
    st.o[1] = f32x16{};
}

// Natural-log sum of a row's exp(scores) from its base-2 offset and the weight sum
// relative to it; -inf for a row with no key.
__device__ __forceinline__ float lse_of(float ofs2, float l) {
    return l > 0.f ? (ofs2 + __builtin_log2f(l)) * 0.69314718055994531f : kNegInf;
}

// A tile whose weights (relative to cofs) sum to at most 2^8 has every weight at
// most 2^8: exact in bf16 and fp32 alike, so it is folded as it is.
constexpr float kTileSumBound = 256.0f;

// Offset of a partial result for a log-sum-exp merge: -inf when it holds no weight.
__device__ __forceinline__ float state_offset(const State& st) { return st.l > 0.f ? st.cofs : kNegInf; }

__device__ __forceinline__ bool pair_or(bool x) {
    auto r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    return (r[0] | r[1]) != 0u;
}

// Rare path of a tile fold: the triggering queries (weights that may exceed 2^8) raise
// their offset to the tile's largest score (both lanes of a pair take the same
// decision) and recompute their weights against it; every lane refreshes its seed and
// the tile sum.
template <class T>
__device__ __forceinline__ void fold_slow(State& st, const f32x16& x, float* p, typename T::PFrag& pf, float& ts,
                                          bool trig, const typename T::Lane& lo) {
    float m4[4];
    for (int j = 0; j < 4; ++j) m4[j] = fmaxf(fmaxf(x[4 * j], x[4 * j + 1]), fmaxf(x[4 * j + 2], x[4 * j + 3]));
    const float tmax = pair_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))) + st.cofs;
    if (pair_or(trig) && tmax != kNegInf) {
        // The state so far is relative to cofs; without weight it is zero.
        const float alpha = st.l > 0.f ? fast_exp2(st.cofs - tmax) : 0.f;
        st.l *= alpha;
        st.o[0] *= alpha;
        st.o[1] *= alpha;
        const float sh = tmax - st.cofs;
        for (int i = 0; i < 16; ++i) p[i] = fast_exp2(x[i] - sh);
        st.cofs = tmax;
    }
    for (int i = 0; i < 16; ++i) st.seed[i] = -st.cofs;
    T::to_p(p, pf);
    ts = T::tile_sum(pf, p, lo);  // with the whole wave active
}

// Fast path unless the weights may exceed the bound (a non-finite sum included).
__device__ __forceinline__ bool fold_trigger(const State&, float ts) { return !(ts <= kTileSumBound); }

// A query's first tile with a valid key sets its offset to the tile's largest score
// before the exponentials (queries that already hold weight keep theirs): its largest
// weight is then exactly 1 and no weight overflows or underflows.
__device__ __forceinline__ void first_offset(State& st, f32x16& x) {
    float m4[4];
    for (int j = 0; j < 4; ++j) m4[j] = fmaxf(fmaxf(x[4 * j], x[4 * j + 1]), fmaxf(x[4 * j + 2], x[4 * j + 3]));
    const float tm = pair_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));  // relative to cofs
    const bool set = st.l == 0.f && tm != kNegInf;
    const float sh = set ? tm : 0.f;
    for (int i = 0; i < 16; ++i) x[i] -= sh;
    st.cofs += sh;
    for (int i = 0; i < 16; ++i) st.seed[i] = -st.cofs;
}

// Fold one 32-key tile of exponents x (score - cofs; -inf for masked keys) into the
// state; the weights go to the P^T operand.  The rare path recomputes the exponents
// with `scores()` (the staged keys are still in LDS) instead of keeping x alive across
// the fast path.
template <class T, class Scores>
__device__ __forceinline__ void fold_tile(State& st, f32x16 x, typename T::PFrag& pf,
                                          const typename T::Lane& lo, Scores scores) {
    if (__any(st.l == 0.f)) first_offset(st, x);
    float p[16];
    for (int i = 0; i < 16; ++i) p[i] = fast_exp2(x[i]);
    T::to_p(p, pf);
    float ts = T::tile_sum(pf, p, lo);
    const bool trig = fold_trigger(st, ts);
    if (__any(trig)) {
        asm volatile("" ::: "memory");  // re-read the staged keys: nothing stays alive for this path
        const f32x16 x2 = scores();
        for (int i = 0; i < 16; ++i) p[i] = fast_exp2(x2[i]);
        fold_slow<T>(st, x2, p, pf, ts, trig, lo);
    }
    st.l += ts;
}


// Relative position bias of a window sub-tile: element i of the lane holds the key at
// offset base + kc_of(i) in the (padded, base-2) table row starting at brow.
__device__ __forceinline__ void add_bias_run(f32x16& s, const float* brow) {
    for (int i = 0; i < 16; ++i) s[i] += brow[kc_of(i)];
}

// One 32-key sub-tile of a stage: scores, masks, softmax update, P.V product.
template <class T, bool kRand = false>
__device__ __forceinline__ void sub_step(State& st, const char* slot, int sub, const typename T::Lane& lo,
                                         const typename T::QOp& q, int mode, uint32_t inv32, int h2, int base,
                                         int span, const int* gp, int wq, int climit = 1 << 30,
                                         const float* brow = nullptr) {
    // exponents: scores - cofs, masked
    auto scores = [&]() __attribute__((always_inline)) {
        f32x16 s = T::qk(slot, sub, lo, q, st.seed);
        if (brow) add_bias_run(s, brow);
        mask_scores<kRand>(s, mode, inv32, h2, base, span, gp, wq, climit);
        return s;
    };
    const f32x16 s = scores();
    typename T::VOp vo;
    T::load_v(vo, slot, sub, lo);  // in flight during the softmax
    typename T::PFrag pf;
    fold_tile<T>(st, s, pf, lo, scores);
    T::pv(vo, pf, st.o);
}

// ---------------------------------------------------------------------------
// (a)+(b): one work-group = 128 consecutive rows of one residue class of one
// (b, h); wave wv owns rows r0 + 32*wv .. +31.  The stage sequence is the global
// keys (up to 64 per stage, with an in-window test so each key counts once)
// followed by the window band [kb0, kend) of the class in 64-key stages.  The band
// stages lie on a grid aligned to r0: nb stages before the tile's own rows, the two
// "home" stages [r0, r0 + 128), na stages after; they are processed in the order
// before, after, home (the softmax fold does not depend on the order), so that the
// home keys are still in LDS when the band ends, for (c).  Each wave skips 32-key
// sub-tiles outside its rows' band and masks only sub-tiles that touch the band
// edge or hold invalid keys.
//
// Random blocks (kRandom; every head undilated, so the tile's rows are positions
// r0 .. r0+127, i.e. query blocks r0/64 and r0/64 + 1): after the global stages come
// the key blocks drawn by the first query block (for waves 0-1), then those drawn by
// the second (waves 2-3), one 64-key stage each.  Their keys that lie in a row's
// window, are global, padded or past the end are masked, so each key counts once.

// Dilation of head h from the band kernel's dilation code (dil_code below): the value
// every head shares (> 0), two bits per head (< 0), or else the head's own entry.
__device__ __forceinline__ int head_dil_code(int code, const int* dil, int h) {
    if (code > 0) return code;
    if (code < 0) return (((-code - 1) >> (2 * h)) & 3) + 1;
    asm volatile("");
    return dil[h];
}

// Global-row partials of tile slot t_in of slice bh that hold no weight (no tile, or
// no valid home key): the merge reads every slot of a head.
__device__ __forceinline__ void empty_partials(const Params& p, int bh, int tph, int t_in, int tid) {
    const int n = p.n_gblk * kGlobalQueriesPerBlock;
    const size_t part0 = ((size_t)bh * tph + t_in) * n;
    for (int i = tid; i < n; i += kThreads) {
        p.ws_ml[2 * (part0 + i)] = kNegInf;
        p.ws_ml[2 * (part0 + i) + 1] = 0.f;
    }
    for (int i = tid; i < n * 16; i += kThreads)
        reinterpret_cast<f32x4*>(p.ws_acc + part0 * 64)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <class T, bool kCausal, bool kBias, bool kRandom, bool kStrided = false, bool kSplit = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(T::kWavesPerEU)))
void band_kernel(const int nblk, const int tph, const int H, const int L, const int dil_u, const void* const q_arg,
                 const int nseq, const Params p) {
    using Elem = typename T::Elem;
    // kSplit: 64-row tiles; waves 2 rb and 2 rb + 1 share row block rb and take the
    // even and the odd 32-key sub-tiles of every stage, then merge their states.
    static_assert(!(kSplit && (kRandom || kStrided)), "the split tiling has no random-block or strided form");
    constexpr int kRows = kSplit ? kSplitRows : kRowsPerBlock;  // rows of the tile
    constexpr int kHome = kRows / kStageKeys;                   // stages of its own rows as keys
    __shared__ __attribute__((aligned(16))) char ring[T::kNS * T::kStageBytes];
    __shared__ uint64_t band_mask[kMaskRing];        // invalid-key bits of band stages
    __shared__ uint64_t glob_mask[kMaxGlobalStages];  // invalid-key bits of global stages
    __shared__ int glob_src[LF_MAX_GLOBALS];          // source row of each global slot or -1
    __shared__ __attribute__((aligned(16))) int glob_pos[LF_MAX_GLOBALS];  // same-class virtual position or kNoPos
    __shared__ int glob_abs[LF_MAX_GLOBALS];          // position of each global slot (sorted)
    __shared__ int glob_row[LF_MAX_GLOBALS];          // same as glob_pos, padded or not
    __shared__ int glob_g[kGlobalQueriesPerBlock];    // first 32 global positions (or -1)
    // Relative position bias of this head, base 2, offset m at kBiasPad + m + w (zero padding
    // around it covers every lane's reads of a processed sub-tile).
    __shared__ float bias_lds[kBias ? kBiasLds : 1];
    __shared__ uint32_t row_glob[kRowsPerBlock / 32]; // tile rows that are global queries
    __shared__ uint64_t rnd_inv[kRandom ? 2 * LF_MAX_RANDOM_DRAWS : 1];  // invalid-key bits of random stages
    __shared__ __attribute__((aligned(16))) char gq_rows[kGlobalQueriesPerBlock * T::kRowBytes];  // first 32 global Q rows

    const int tid = threadIdx.x, lane = tid & 63, h2 = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int rb = kSplit ? wv >> 1 : wv;  // the wave's 32-row block of the tile
    const int kh = kSplit ? wv & 1 : 0;    // kSplit: the sub-tile of each stage it takes
    // The leading arguments (the grid size, p.tiles_per_head, p.H, p.L, p.dil_u, p.q,
    // p.B) are the tile decode's and the Q load's; the build preloads them into scalar
    // registers, so neither waits for memory.  The other arguments of the set-up are read
    // in one batch after the Q load is issued: left alone, the compiler waits for each
    // argument load at its first use, one memory round trip after another across the
    // set-up's branches.
    if constexpr (kStrided) asm volatile("" ::"s"(p.s_b), "s"(p.s_h), "s"(p.s_r), "s"(p.o_b), "s"(p.o_h), "s"(p.o_r));
    const int pid = xcd_remap(blockIdx.x, nblk);
    // Slice j = pid / tph holds sequence j % nseq, head j / nseq: one XCD's contiguous
    // range of slices then takes every sequence in turn, so sequences of different
    // true lengths (padding) load the XCDs evenly.
    const int j_bh = pid / tph, t_in = pid - j_bh * tph;
    const int h = j_bh / nseq, b = j_bh - h * nseq;
    const int bh = b * H + h;
    const int dil = head_dil_code(dil_u, p.dil, h);
    int r, Lr, r0;  // residue class, its length, the tile's first class row
    if (!decode_tile<kRows>(t_in, L, dil, r, Lr, r0)) {
        // A slot without a tile (a head or residue class with fewer tiles than the
        // grid's per-head count): its global-row partials say "no weight", so the merge
        // reads every slot without working out which hold tiles.
        if (p.n_g > 0) empty_partials(p, bh, tph, t_in, tid);
        return;
    }

    // q, k, v (and q_g, k_g, v_g): row i of (b, h) at b*s_b + h*s_h + i*rs elements,
    // out at b*o_b + h*o_h + i*o_r (kStrided); else [B][H][L][64] with constant strides.
    const int rs = kStrided ? p.s_r : 64, ors = kStrided ? p.o_r : 64;
    const size_t off = kStrided ? (size_t)b * p.s_b + (size_t)h * p.s_h : (size_t)bh * L * 64;
    const size_t ooff = kStrided ? (size_t)b * p.o_b + (size_t)h * p.o_h : (size_t)bh * L * 64;
    const Elem* Q = reinterpret_cast<const Elem*>(q_arg) + off;
    // Position of global slot tid of a shared set, loaded ahead of the Q rows so that the
    // slot set-up waits for this load alone (a per-sequence set is read there).
    static_assert(kThreads <= LF_MAX_GLOBALS && kMaxGlobalStages * kStageKeys <= kThreads,
                  "one slot per thread covers every global stage");
    const int g_shared = p.g[tid];
    const int qa = r0 + 32 * rb;      // first virtual row of this wave
    const int qv = qa + (lane & 31);  // this lane's virtual row
    const bool rows_live = qa < Lr;
    typename T::QOp qop;
    T::load_q(qop, qv < Lr ? Q + (size_t)(r + qv * dil) * rs : nullptr, h2);

    const int w = p.w, gstride = p.gstride, n_g = p.n_g;
    const void* const k_arg = p.k;
    const void* const v_arg = p.v;
    const void* const kg_arg = p.kg;
    const uint8_t* const pad_arg = p.pad;
    asm volatile("" ::"s"(w), "s"(gstride), "s"(n_g), "s"(k_arg), "s"(v_arg), "s"(kg_arg), "s"(pad_arg));
    const Elem* K = reinterpret_cast<const Elem*>(k_arg) + off;
    const Elem* V = reinterpret_cast<const Elem*>(v_arg) + off;
    Elem* O = reinterpret_cast<Elem*>(p.out) + ooff;
    const uint8_t* pad = pad_arg ? pad_arg + (size_t)b * L : nullptr;
    // Global set of this sequence: one shared set (gstride 0) or one row per sequence.
    const int gofs = b * gstride;
    const int ng = seq_globals(gstride, n_g, p.gcnt, b);
    // Tensors of the global rows' own attention (c): the separate projections if given.
    const bool sep = kg_arg != nullptr;
    const Elem* QG = sep ? reinterpret_cast<const Elem*>(p.qg) + off : Q;
    const Elem* KG = sep ? reinterpret_cast<const Elem*>(kg_arg) + off : K;
    const Elem* VG = sep ? reinterpret_cast<const Elem*>(p.vg) + off : V;

    // Window of a row: keys w steps before it and wr after (wr = 0 in the one-sided
    // variant, which also drops global keys after the row and, for a global row,
    // every key after it).
    constexpr bool causal = kCausal;
    const int wr = causal ? 0 : w, span = w + wr;
    const int kb0 = max(0, r0 - w);
    const int kend = min(Lr, r0 + kRows + wr);
    const int nb = (r0 - kb0 + kStageKeys - 1) / kStageKeys;  // stages before the home keys
    const int gbase = r0 - kStageKeys * nb;                    // first key of the grid (<= kb0)
    const int na = max(0, (kend - (r0 + kHome * kStageKeys) + kStageKeys - 1) / kStageKeys);
    const int n_band = nb + kHome + na;
    const int n_gst = (ng + kStageKeys - 1) / kStageKeys;
    // Random stages: the draws of query block r0/64 (rnd_a, na_r of them), then those
    // of the next query block (rnd_b, nb_r); rows are sorted with -1 after the draws.
    const int* rnd_a = nullptr;
    const int* rnd_b = nullptr;
    int na_r = 0, nb_r = 0;
    if (kRandom) {
        const int qb0 = r0 / kRandomBlock;
        rnd_a = p.rnd + ((size_t)h * p.rnd_nq + qb0) * p.rnd_r;
        rnd_b = rnd_a + p.rnd_r;
        while (na_r < p.rnd_r && rnd_a[na_r] >= 0) ++na_r;
        if (qb0 + 1 < p.rnd_nq)
            while (nb_r < p.rnd_r && rnd_b[nb_r] >= 0) ++nb_r;
    }
    const int n_rst = na_r + nb_r;
    const int n_lst = n_gst + n_rst;  // stages of listed keys (global, then random)
    const int n_st = n_lst + n_band;
    // Stage order: the global and random stages (listed keys), then the band stages.
    auto is_glob = [&](int t) __attribute__((always_inline)) { return t < n_lst; };  // a listed-key stage
    auto band_u = [&](int t) __attribute__((always_inline)) { return t - n_lst; };
    auto rnd_block = [&](int j) __attribute__((always_inline)) { return j < na_r ? rnd_a[j] : rnd_b[j - na_r]; };  // key block of random stage j
    // Processing order of the band stages: the two home stages last (the global-row pass
    // reuses them).  A tile with the full band of P = ceil(w/64) + 2 + ceil(wr/64) grid
    // stages takes its other stages in ascending order of their 64-key block index
    // modulo P: each block of the class is then read at about the same step by every
    // tile whose band holds it, so a head's K/V comes from HBM a few blocks per step
    // instead of all of it in the first two steps.  Tiles whose band is cut by the
    // sequence ends take before, after, home.
    const int P = ((w + kStageKeys - 1) / kStageKeys) + kHome + ((wr + kStageKeys - 1) / kStageKeys);
    const bool rot = n_band == P && P > kHome;
    int bs0 = 0, hlo = 0, hhi = 0;
    if (rot) {
        const int a0 = (gbase / kStageKeys) % P;  // gbase >= 0 here (a multiple of 64)
        bs0 = a0 == 0 ? 0 : P - a0;                 // grid stage of the first block = 0 mod P
        const int h0 = nb >= bs0 ? nb - bs0 : nb - bs0 + P;  // rotated positions of the home stages
        const int h1 = h0 + 1 == P ? 0 : h0 + 1;
        hlo = kHome == 2 ? min(h0, h1) : h0;
        hhi = kHome == 2 ? max(h0, h1) : P;  // one home stage: no second position to skip
    }
    // Grid stage of the u-th band stage in processing order.
    auto band_bs = [&](int u) __attribute__((always_inline)) {
        if (!rot) return u < nb ? u : (u < nb + na ? u + kHome : u - na);
        if (u >= P - kHome) return nb + u - (P - kHome);
        int k = u;
        if (k >= hlo) ++k;
        if (k >= hhi) ++k;
        const int b = bs0 + k;
        return b >= P ? b - P : b;
    };
    // First key of the u-th band stage.
    auto stage_key = [&](int u) __attribute__((always_inline)) { return gbase + kStageKeys * band_bs(u); };

    // Invalid-key bits of band stage u: keys outside [kb0, kend), or padded.
    auto band_invalid = [&](int bs) __attribute__((always_inline)) -> uint64_t {
        if (pad) return band_mask[bs % kMaskRing];
        const int ks = stage_key(bs);
        const int lo = kb0 - ks, hi = kend - ks;  // valid keys: lo <= kk < hi
        uint64_t m = 0;
        if (lo > 0) m |= lo >= 64 ? ~0ull : ((1ull << lo) - 1);
        if (hi < 64) m |= hi <= 0 ? ~0ull : (~0ull << hi);
        return m;
    };
    typename T::DmaLane dl;
    T::dma_lane(dl, wv, lane, dil * rs);
    // The scalar-base copies use 32-bit per-lane offsets of up to 64 rows dil apart.
    const bool direct_ok = (uint64_t)dil * rs * kStageKeys * sizeof(Elem) < (1ull << 31);
    // Copies of stage s into its ring slot: part 0 or 1 of this wave's share, or all.
    int ks_next = 0;  // first key of the band stage copied last (see the stage loop)
    auto issue = [&](int s, int part) __attribute__((always_inline)) -> uint64_t {
        char* slot = ring + (s % T::kNS) * T::kStageBytes;
        if (kRandom && is_glob(s) && s >= n_gst) {
            const int j = s - n_gst;
            const int kb0 = kRandomBlock * rnd_block(j);
            const uint64_t inv = uniform64(rnd_inv[j]);
            if (inv == 0ull && part == kAllParts && direct_ok) {
                T::dma_stage_direct(slot, K + (size_t)kb0 * rs, V + (size_t)kb0 * rs, dl, wv);
            } else {
                T::dma_stage(slot, K, V, rs, [&](int kk) __attribute__((always_inline)) { return ((inv >> kk) & 1) ? -1 : kb0 + kk; }, wv, lane, part);
            }
            return 0ull;
        } else if (is_glob(s)) {
            const int* src = glob_src + kStageKeys * s;
            T::dma_stage(slot, K, V, rs, [&](int kk) __attribute__((always_inline)) { return src[kk]; }, wv, lane, part);
            return 0ull;
        } else {
            const int bs = band_u(s);
            const uint64_t inv = uniform64(band_invalid(bs));
            const int ks = stage_key(bs);
            ks_next = ks;
            if (inv == 0ull && part == kAllParts && direct_ok) {
                const size_t row0 = (size_t)(r + ks * dil) * rs;
                T::dma_stage_direct(slot, K + row0, V + row0, dl, wv);
            } else {
                T::dma_stage(slot, K, V, rs, [&](int kk) __attribute__((always_inline)) { return ((inv >> kk) & 1) ? -1 : r + (ks + kk) * dil; },
                             wv, lane, part);
            }
            return inv;
        }
    };

    // Without padding a band stage needs nothing from LDS: its copy goes out before
    // the set-up below, together with the Q operand loads.
    const bool early = !pad && n_st > 0 && !is_glob(0);
    uint64_t inv_next = 0ull;  // invalid-key bits of the next band stage, from its copy
    if (early) inv_next = issue(0, kAllParts);

    // Pad masks of band stages [64*W, 64*W + 64): wave wv builds words wv, wv+4, ... of
    // the stages that exist; every pad load of a window is issued before the first is
    // used (the ballots), and those of window 0 before the global slots' own loads.
    constexpr int kPadWords = kMaskWindow / kWaves;
    auto load_band_pad = [&](int W, uint32_t* flag) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kPadWords; ++j) {
            const int bs = W * kMaskWindow + wv + kWaves * j;
            flag[j] = 1u;
            if (bs < n_band) {
                const int key = stage_key(bs) + lane;
                if (key >= kb0 && key < kend) flag[j] = pad[r + key * dil];
            }
        }
    };
    // Also whether any of this wave's words has a valid key (a band longer than one
    // window counts as live).
    __shared__ uint32_t band_live[kWaves];
    auto store_band_masks = [&](int W, const uint32_t* flag) __attribute__((always_inline)) {
        bool live = n_band > kMaskWindow;
#pragma unroll
        for (int j = 0; j < kPadWords; ++j) {
            const int bs = W * kMaskWindow + wv + kWaves * j;
            if (bs < n_band) {
                const uint64_t inv = ballot64(flag[j] != 0);
                if (lane == 0) band_mask[bs % kMaskRing] = inv;
                live |= inv != ~0ull;
            }
        }
        if (lane == 0) band_live[wv] = live;
    };
    uint32_t pflag[kPadWords];
    if (pad) load_band_pad(0, pflag);

    // Global slots: source row (or -1 if unused/padded) and in-window position; slot gi
    // is thread gi's.
    if (const int gi = tid; gi < n_gst * kStageKeys) {
        int g = gi < ng ? g_shared : -1;
        if (gstride) {
            g = gi < ng ? p.g[gofs + gi] : -1;
            asm volatile("" ::"v"(g));  // awaited here: a wait after the branch would wait for the Q rows too
        }
        const bool ok = g >= 0 && (!pad || pad[g] == 0);
        const int vpos = (g >= r && (g - r) % dil == 0) ? (g - r) / dil : kNoPos;
        glob_src[gi] = ok ? g : -1;
        glob_pos[gi] = ok ? vpos : kNoPos;
        glob_abs[gi] = g;
        glob_row[gi] = vpos;
        if (gi < kGlobalQueriesPerBlock) glob_g[gi] = g;
    }
    if (tid < kRows / 32) row_glob[tid] = 0u;
    // Windows after the first (a band of more than 64 stages), from inside the stage
    // loop: four words at a time, which keeps the registers of the loads few.
    auto fill_band_masks = [&](int W) __attribute__((always_inline)) {
        constexpr int kGroup = 4;
        for (int j0 = 0; j0 < kPadWords; j0 += kGroup) {
            if (W * kMaskWindow + wv + kWaves * j0 >= n_band) break;
            uint32_t flag[kGroup];
            for (int j = 0; j < kGroup; ++j) {
                const int bs = W * kMaskWindow + wv + kWaves * (j0 + j);
                const int key = stage_key(bs) + lane;
                flag[j] = (bs < n_band && key >= kb0 && key < kend) ? pad[r + key * dil] : 1u;
            }
            for (int j = 0; j < kGroup; ++j) {
                const int bs = W * kMaskWindow + wv + kWaves * (j0 + j);
                const uint64_t inv = ballot64(flag[j] != 0);
                if (lane == 0 && bs < n_band) band_mask[bs % kMaskRing] = inv;
            }
        }
    };
    if (pad) store_band_masks(0, pflag);
    if (kBias) {
        const float* tab = p.bias + (size_t)h * (2 * p.bias_w + 1) + p.bias_w;  // entry of offset 0
        for (int t = tid; t < 2 * w + 1 + 2 * kBiasPad; t += kThreads) {
            const int m = t - kBiasPad - w;
            bias_lds[t] = (m >= -w && m <= w) ? tab[m] * kLog2eF : 0.f;
        }
    }
    barrier_lds();  // the Q rows and the first stage stay in flight
    if (wv == 0)
        for (int s = 0; s < n_gst; ++s) {
            const uint64_t inv = ~ballot64(glob_src[kStageKeys * s + lane] >= 0);
            if (lane == 0) glob_mask[s] = inv;
        }
    for (int gi = tid; gi < ng; gi += kThreads) {
        const int vr = glob_row[gi] - r0;
        if (vr >= 0 && vr < kRows) atomicOr(&row_glob[vr >> 5], 1u << (vr & 31));
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
    const int gcnt = causal ? count_le(glob_abs, ng, r + qv * dil) : 0;
    // A band whose keys are all padded (rows past a sequence's end by more than w) is
    // neither copied nor visited: stages [0, n_run) are the ones run.  Its home keys
    // are padded too, so the global-row pass below has nothing to fold either.
    const bool band_dead = pad && !(band_live[0] | band_live[1] | band_live[2] | band_live[3]);
    const int n_run = band_dead ? n_lst : n_st;

    State st;
    state_init(st);
    typename T::Lane lo;
    T::lane_offsets(lo, lane);
    // kSplit: the wave reads only sub-tile kh of each stage, addressed as sub-tile 0.
    if (kSplit) T::shift_lane(lo, kh);

    // The first stages are copied while the Q operand loads are still in flight;
    // every register load (Q operand, masks) completes at the wait below, so the
    // compiler's own waits inside the loop have nothing left to wait for (an
    // in-loop vmcnt wait would also drain the stage copies in flight).
    for (int s = early ? 1 : 0; s < T::kNS - 1; ++s)
        if (s < n_run) {
            const uint64_t x = issue(s, kAllParts);
            if (s == 0) inv_next = x;
        }
    wait_vmcnt<0>();
    T::scale_q(qop);
    // Stages [0, n_gen): the listed-key stages (global, random), in the general body
    // below; stages [n_gen, n_st): band stages only, in the lean loop after it.
    const int n_gen = n_lst;
    static_assert(T::kNS == 2, "stage t + 1 is issued while stage t is computed");
    for (int t = 0; t < n_gen; ++t) {
        wait_stage<T>(0);
        barrier_nofence();
        // The next stage: listed, or band stage 0 (whose pad masks are already built).
        if (t + 1 < n_run) inv_next = issue(t + 1, kAllParts);
        if (t == 0 && ng > 0) {  // Q rows of the first 32 global queries, for (c)
            const Elem* zero = reinterpret_cast<const Elem*>(g_zero_row);
            T::dma_rows(gq_rows, [&](int j) __attribute__((always_inline)) { const int g = glob_g[j]; return g >= 0 ? QG + (size_t)g * rs : zero; },
                        wv, lane);
        }
        const char* slot = ring + (t % T::kNS) * T::kStageBytes;
        // Stage kind: random (kRandom: key block rnd_block(j), for the waves of its
        // query block) or global (listed slots).
        const bool rstage = kRandom && t >= n_gst;
        const int j = t - n_gst;  // random stage index when rstage
        const int ks = rstage ? kRandomBlock * rnd_block(j) : 0;
        const uint64_t inv = uniform64(rstage ? rnd_inv[j] : glob_mask[t]);
        const bool wave_on = !rstage || (wv >> 1) == (j < na_r ? 0 : 1);
        if (kSplit) {
            const int sub = kh;
            const uint32_t inv32 = (uint32_t)(inv >> (32 * sub));
            if (rows_live && inv32 != ~0u) {
                const int goff = kStageKeys * t + 32 * sub + 8 * h2;
                const int bbase = 32 * sub + 8 * h2 - qv + w;
                const int climit = !causal ? 1 << 30 : gcnt - goff;
                sub_step<T>(st, slot, 0, lo, qop, 2, inv32, h2, bbase, span, glob_pos + goff, w - qv, climit, nullptr);
            }
        } else if (rows_live && wave_on && inv != ~0ull) {
            // Both sub-tiles in straight-line code: the second one's operand reads and
            // products can be scheduled against the first one's softmax.
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                const uint32_t inv32 = (uint32_t)(inv >> (32 * sub));
                const int kss = ks + 32 * sub;
                if (inv32 == ~0u) continue;
                if (rstage) {
                    if (kss >= qa + 31 - w && kss + 31 <= qa + wr) continue;  // inside every row's window
                    if (causal && kss > qa + 31) continue;                    // after every row
                }
                const int mode = rstage ? 3 : 2;
                const int goff = kStageKeys * t + 32 * sub + 8 * h2;
                const int bbase = kss + 8 * h2 - qv + w;
                const int climit = !causal ? 1 << 30 : (rstage ? w - bbase + 1 : gcnt - goff);
                sub_step<T, kRandom>(st, slot, sub, lo, qop, mode, inv32, h2, bbase, span, glob_pos + goff, w - qv,
                                     climit, nullptr);
            }
        }
    }

    // Band stages.  Sub-tile j of the band grid holds keys gbase + 32 j .. + 31; the
    // wave's first row is grid position 32 ja.  Some row of the wave has a window key in
    // sub-tile j for jlo <= j <= jhi, every row has all 32 for ilo <= j <= ihi.  Per
    // sub-tile the wave takes one of three uniform branches: skipped, interior with every
    // key valid (no mask), or masked (band edge, invalid keys).
    const int ja = 2 * nb + rb;
    const int jlo = ja - ((w + 31) >> 5), jhi = ja + ((wr + 31) >> 5);
    const int ilo = ja - ((w - 31) >> 5), ihi = ja + ((wr - 31) >> 5);
    // Copies of band stage u into ring slot sl; returns its invalid-key bits and sets
    // ks_next.  A stage whose 64 keys all lie in [kb0, kend) without padding needs no
    // mask: its copy goes out in the scalar-base form at once.
    auto issue_band = [&](int u, int sl) __attribute__((always_inline)) -> uint64_t {
        const int ks = gbase + kStageKeys * band_bs(u);
        ks_next = ks;
        char* slot = ring + sl * T::kStageBytes;
        if (!pad && ks >= kb0 && ks + kStageKeys <= kend && direct_ok) {
            const size_t row0 = (size_t)(r + ks * dil) * rs;
            T::dma_stage_direct(slot, K + row0, V + row0, dl, wv);
            return 0ull;
        }
        const uint64_t inv = uniform64(band_invalid(u));
        if (inv == 0ull && direct_ok) {
            const size_t row0 = (size_t)(r + ks * dil) * rs;
            T::dma_stage_direct(slot, K + row0, V + row0, dl, wv);
        } else {
            T::dma_stage(slot, K, V, rs, [&](int kk) __attribute__((always_inline)) { return ((inv >> kk) & 1) ? -1 : r + (ks + kk) * dil; }, wv,
                         lane);
        }
        return inv;
    };
    // One band stage t in ring slot SL (t % 2), which the caller makes a compile-time
    // constant so that the operand reads address the slot with immediate offsets.
    auto band_step = [&](int t, auto slot_c) __attribute__((always_inline)) {
        constexpr int SL = decltype(slot_c)::value;
        const uint64_t inv = inv_next;  // stage t's bits (two-slot ring: issued last)
        const int ks = ks_next;
        wait_vmcnt<0>();
        barrier_nofence();
        if (t + 1 < n_run) {
            const int bn = t + 1 - n_lst;
            if (pad && bn % kMaskWindow == 0) {  // bn > 0: band stage 0 is never issued here
                fill_band_masks(bn / kMaskWindow);
                __syncthreads();
            }
            inv_next = issue_band(bn, SL ^ 1);
        }
        if (!rows_live) return;
        const char* slot = ring + SL * T::kStageBytes;
        const int j0 = (ks - gbase) >> 5;
        if constexpr (kSplit) {
            const int j = j0 + kh;
            const uint32_t inv32 = (uint32_t)(inv >> (32 * kh));
            if (j < jlo || j > jhi || inv32 == ~0u) return;
            const int bbase = ks + 32 * kh + 8 * h2 - qv + w;
            const int mode = (j >= ilo && j <= ihi && inv32 == 0u) ? 0 : 1;
            sub_step<T>(st, slot, 0, lo, qop, mode, inv32, h2, bbase, span, nullptr, 0, 1 << 30, nullptr);
            return;
        }
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int j = j0 + sub;
            const uint32_t inv32 = (uint32_t)(inv >> (32 * sub));
            if (j < jlo || j > jhi || inv32 == ~0u) continue;
            const int bbase = ks + 32 * sub + 8 * h2 - qv + w;
            const float* brow = kBias ? bias_lds + kBiasPad + bbase : nullptr;
            const int mode = (j >= ilo && j <= ihi && inv32 == 0u) ? 0 : 1;
            sub_step<T>(st, slot, sub, lo, qop, mode, inv32, h2, bbase, span, nullptr, 0, 1 << 30, brow);
        }
    };
    static_assert(T::kNS == 2, "the band loop alternates between two ring slots");
    {
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        int t = n_gen;
        if (t < n_run && (t & 1)) band_step(t++, S1{});
        for (; t + 1 < n_run; t += 2) {
            band_step(t, S0{});
            band_step(t + 1, S1{});
        }
        if (t < n_run) band_step(t, S0{});
    }

    if constexpr (kSplit) {
        // The odd wave of each row block hands its state (offset, weight sum, 32 output
        // values per lane) to the even one through the ring slot of the second-to-last
        // stage run, which every wave is done with; the even wave combines the two
        // log-sum-exp style and stores the rows.
        __shared__ float x_ml[2][2][64];
        // [2 rb][64 lanes][8 chunks of 4 values], chunk k of a lane at k ^ (lane % 8)
        float* xo = reinterpret_cast<float*>(ring + (n_run & 1) * T::kStageBytes);
        if (kh == 1) {
            x_ml[rb][0][lane] = state_offset(st);
            x_ml[rb][1][lane] = st.l;
            for (int k = 0; k < 8; ++k)
                *reinterpret_cast<f32x4*>(xo + ((rb * 64 + lane) * 8 + (k ^ (lane & 7))) * 4) =
                    f32x4{st.o[k >> 2][4 * (k & 3)], st.o[k >> 2][4 * (k & 3) + 1], st.o[k >> 2][4 * (k & 3) + 2],
                          st.o[k >> 2][4 * (k & 3) + 3]};
        }
        barrier_lds();
        if (kh == 0) {
            const float c1 = x_ml[rb][0][lane], l1 = x_ml[rb][1][lane];
            const float c0 = state_offset(st);
            const float m = fmaxf(c0, c1);
            const float M = m == kNegInf ? 0.f : m;  // both empty: weights 0, sum 0
            const float a0 = fast_exp2(c0 - M), a1 = fast_exp2(c1 - M);
            st.l = st.l * a0 + l1 * a1;
            for (int k = 0; k < 8; ++k) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(xo + ((rb * 64 + lane) * 8 + (k ^ (lane & 7))) * 4);
                for (int j = 0; j < 4; ++j) st.o[k >> 2][4 * (k & 3) + j] = st.o[k >> 2][4 * (k & 3) + j] * a0 + x[j] * a1;
            }
            st.cofs = M;
        }
    }
    const float scale = st.l > 0.f ? 1.f / st.l : 0.f;
    typename T::RowOut ro;
    T::pack_row(ro, st.o, scale);
    if (qv < Lr && kh == 0) {
        const int row = r + qv * dil;
        const int vr = qv - r0;  // global rows are written by the merge
        if (!((row_glob[vr >> 5] >> (vr & 31)) & 1u)) {
            T::store_row(O + (size_t)row * ors, h2, ro);
            if (p.lse && h2 == 0) p.lse[(size_t)bh * L + row] = lse_of(st.cofs, st.l);
        }
    }
    if (ng == 0) return;
    if (band_dead) {  // every home key is padded: nothing to fold
        empty_partials(p, bh, tph, t_in, tid);
        return;
    }

    // (c) Global rows: every key belongs to exactly one work-group's "home" range
    // [r0, r0 + 128) of its class, so each work-group folds the global queries over
    // its home keys and leaves one partial (max, sum, unnormalised output) per query.
    // The Q rows of the first 32 global queries were copied to LDS with the first
    // stage; for them the home keys are the last two band stages, still in the ring,
    // unless the global rows have their own key and value projections.
    __shared__ float red_ml[kWaves][32][2];
    float* red_o = reinterpret_cast<float*>(ring);  // kWaves x 32 x 64 floats = 32 KiB
    const int home_end = min(Lr, r0 + kRows);
    const size_t part0 = ((size_t)bh * tph + t_in) * p.n_gblk * kGlobalQueriesPerBlock;
    // wave wv folds home keys 32*wv .. 32*wv+31 (kSplit: waves 0 and 1, the tile's 64)
    const int hs = kSplit ? 0 : wv >> 1, hsub = kSplit ? kh : wv & 1;
    const int n_gblk_b = (ng + kGlobalQueriesPerBlock - 1) / kGlobalQueriesPerBlock;  // this sequence's blocks
    for (int gb = 0; gb < n_gblk_b; ++gb) {
        typename T::QOp gop;
        const char* hslot;
        uint32_t inv32;
        if (gb == 0) {
            T::load_q(gop, reinterpret_cast<const Elem*>(gq_rows) + (size_t)(lane & 31) * 64, h2);
        } else {
            const int gq = gb * kGlobalQueriesPerBlock + (lane & 31);
            T::load_q(gop, gq < ng ? QG + (size_t)p.g[gofs + gq] * rs : nullptr, h2);
        }
        T::scale_q(gop);
        if (gb == 0 && !sep) {
            const int u = n_band - kHome + hs;
            hslot = ring + ((n_lst + u) % T::kNS) * T::kStageBytes;
            inv32 = (uint32_t)(band_invalid(u) >> (32 * hsub));
        } else {
            uint64_t hinv[2] = {~0ull, ~0ull};
            for (int j = 0; j < kHome; ++j) {
                const int key = r0 + kStageKeys * j + lane;
                bool ok = key < home_end;
                if (ok && pad) ok = pad[r + key * dil] == 0;
                hinv[j] = ~ballot64(ok);
            }
            barrier_lds();  // the ring is free (every wave's reads of it are done)
            for (int j = 0; j < kHome; ++j) {
                const uint64_t iv = hinv[j];
                const int ks = r0 + kStageKeys * j;
                T::dma_stage(ring + j * T::kStageBytes, KG, VG, rs,
                             [&](int kk) __attribute__((always_inline)) { return ((iv >> kk) & 1) ? -1 : r + (ks + kk) * dil; }, wv, lane);
            }
            wait_vmcnt<0>();
            barrier_lds();
            hslot = ring + hs * T::kStageBytes;
            inv32 = (uint32_t)((hs ? hinv[1] : hinv[0]) >> (32 * hsub));
        }
        if (kSplit && rb == 1) inv32 = ~0u;  // the tile's 64 home keys are waves 0 and 1's
        State gs;
        state_init(gs);
        if (inv32 != ~0u) {
            if (causal) {
                // keys of this class at or before the global row: virtual index <= vlim
                const int gq = gb * kGlobalQueriesPerBlock + (lane & 31);
                const int g = gq < ng ? p.g[gofs + gq] : -1;
                const int vlim = g >= r ? (g - r) / dil : -1;
                const int kss = r0 + kStageKeys * hs + 32 * hsub;
                sub_step<T>(gs, hslot, kSplit ? 0 : hsub, lo, gop, 1, inv32, h2, kss + 8 * h2 - vlim + kLargeW, kLargeW,
                            nullptr, 0);
            } else {
                sub_step<T>(gs, hslot, kSplit ? 0 : hsub, lo, gop, inv32 != 0u ? 1 : 0, inv32, h2, 0, 2 * kLargeW,
                            nullptr, 0);
            }
        }
        // Done with the staged keys: the ring now holds the reduction.  The barriers of
        // this pass order LDS accesses only; the output rows stored above stay in flight.
        barrier_lds();
        if (lane < 32) {  // partial relative to its offset (-inf when it holds no weight)
            red_ml[wv][lane][0] = state_offset(gs);
            red_ml[wv][lane][1] = gs.l;
        }
        // Four columns 4c .. 4c+3 of query q (a 16-byte chunk c) sit at chunk c ^ (q % 16)
        // of row q: one 16-byte store per accumulator group, two 16-byte loads per
        // column block below.  Slots past the sequence's global count are never read.
        if (gb * kGlobalQueriesPerBlock + (lane & 31) < ng) {
            const int q = lane & 31;
            for (int db = 0; db < 2; ++db)
                for (int m = 0; m < 4; ++m) {
                    const int c = 8 * db + 2 * m + h2;  // columns 32 db + 8 m + 4 h2 .. + 3
                    *reinterpret_cast<f32x4*>(red_o + (wv * 32 + q) * 64 + 4 * (c ^ (q & 15))) =
                        f32x4{gs.o[db][4 * m], gs.o[db][4 * m + 1], gs.o[db][4 * m + 2], gs.o[db][4 * m + 3]};
                }
        }
        barrier_lds();
        {
            const int q = tid >> 3, dc = tid & 7;  // 32 queries x 8 column chunks
            const int gq2 = gb * kGlobalQueriesPerBlock + q;
            if (gq2 < ng) {
                float M = kNegInf;
                for (int x = 0; x < kWaves; ++x) M = fmaxf(M, red_ml[x][q][0]);
                float e[kWaves], l = 0.f;
                for (int x = 0; x < kWaves; ++x) {
                    e[x] = M == kNegInf ? 0.f : fast_exp2(red_ml[x][q][0] - M);
                    l += red_ml[x][q][1] * e[x];
                }
                const size_t idx = part0 + gq2;
                if (dc == 0) {
                    p.ws_ml[2 * idx] = M;
                    p.ws_ml[2 * idx + 1] = l;
                }
                f32x4 o4[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
                for (int x = 0; x < kWaves; ++x)
                    for (int u = 0; u < 2; ++u)
                        o4[u] += *reinterpret_cast<const f32x4*>(red_o + (x * 32 + q) * 64 + 4 * ((2 * dc + u) ^ (q & 15))) * e[x];
                *reinterpret_cast<f32x4*>(p.ws_acc + idx * 64 + 8 * dc) = o4[0];
                *reinterpret_cast<f32x4*>(p.ws_acc + idx * 64 + 8 * dc + 4) = o4[1];
            }
        }
        if (gb + 1 < n_gblk_b) barrier_lds();  // red_ml and the ring are reused
    }

}

// (d) Merge of the global-row partials: one work-group of W <= kMergeWaves waves per
// (global query, h, b) (grid x, y, z), lane = output column (W = blockDim / 64, chosen
// so that one chunk per wave covers a head's tiles).  Wave x takes tiles x, x + W, ...
// in chunks of kMergeChunk whose loads are issued together (slots past the head's tile
// count read tile 0 and are dropped after the load, so there is no branch between the
// loads; a slot the band grid holds no tile for carries an empty partial written by its
// work-group, so no slot needs a test of the head's tiling); within a chunk the maximum
// comes first and the weighted sums are added in tile order, and the wave states are
// combined in wave order: the result does not depend on timing.
//
// The leading arguments (p.tiles_per_head, the partial rows per tile n_gblk * 32, p.H,
// p.L, p.dil_u, p.ws_ml, p.ws_acc) are preloaded into scalar registers by the build, so
// the first partial loads wait for no argument; the other arguments are read while
// those loads are in flight.
template <class T>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(const int tph, const int n_gq, const int H,
                                                                 const int L, const int dil_u,
                                                                 const float* const ws_ml,
                                                                 const float* const ws_acc, const Params p) {
    using Elem = typename T::Elem;
    __shared__ float red[kMergeWaves][3][64];
    const int gi = blockIdx.x, h = blockIdx.y, bseq = blockIdx.z, d = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int bh = bseq * H + h;
    const int W = merge_waves(tph, kMergeChunk, kMergeWaves);  // = blockDim.x / 64
    // gi < n_g <= n_gq: the partial loads below stay in bounds even for a sequence with
    // fewer globals, whose work-groups drop what they loaded and return after the loop.
    const size_t base = (size_t)bh * tph * n_gq + gi;
    const int n_g = p.n_g, gstride = p.gstride, cnt = p.gcnt[bseq], g_shared = p.g[gi];
    Elem* const out_arg = reinterpret_cast<Elem*>(p.out);
    float* const lse_arg = p.lse;
    const long long o_b = p.o_b, o_h = p.o_h;
    const int o_r = p.o_r;
    float M = kNegInf, l = 0.f, o = 0.f;
    for (int c0 = 0; c0 * W < tph; c0 += kMergeChunk) {
        float mt[kMergeChunk], lt[kMergeChunk], ot[kMergeChunk];
        bool ex[kMergeChunk];
#pragma unroll
        for (int j = 0; j < kMergeChunk; ++j) {
            const int t = (c0 + j) * W + wv;
            ex[j] = t < tph;  // slots without a tile hold empty partials
        }
        __builtin_amdgcn_sched_barrier(0);  // every test before the first load
#pragma unroll
        for (int j = 0; j < kMergeChunk; ++j) {
            const size_t idx = base + (ex[j] ? (size_t)((c0 + j) * W + wv) * n_gq : 0);
            mt[j] = ws_ml[2 * idx];
            lt[j] = ws_ml[2 * idx + 1];
            ot[j] = ws_acc[idx * 64 + d];
        }
        float Mc = kNegInf;
#pragma unroll
        for (int j = 0; j < kMergeChunk; ++j) {
            mt[j] = ex[j] ? mt[j] : kNegInf;
            Mc = fmaxf(Mc, mt[j]);
        }
        if (Mc == kNegInf) continue;  // no tile of this chunk has a valid home key
        float lc = 0.f, oc = 0.f;
#pragma unroll
        for (int j = 0; j < kMergeChunk; ++j) {
            const float e = fast_exp2(mt[j] - Mc);  // 0 for absent tiles (mt = -inf)
            lc += (ex[j] ? lt[j] : 0.f) * e;
            oc += (ex[j] ? ot[j] : 0.f) * e;
        }
        const float Mn = fmaxf(M, Mc);
        const float a = fast_exp2(M - Mn), b = fast_exp2(Mc - Mn);
        l = l * a + lc * b;
        o = o * a + oc * b;
        M = Mn;
    }
    if (gi >= (gstride ? cnt : n_g)) return;  // this sequence has fewer globals
    const int g = gstride ? p.g[bseq * gstride + gi] : g_shared;  // position of this global row
    red[wv][0][d] = M;
    red[wv][1][d] = l;
    red[wv][2][d] = o;
    __syncthreads();
    if (wv != 0) return;
    M = kNegInf;
    for (int x = 0; x < W; ++x) M = fmaxf(M, red[x][0][d]);
    l = 0.f;
    o = 0.f;
    if (M != kNegInf)
        for (int x = 0; x < W; ++x) {
            const float e = fast_exp2(red[x][0][d] - M);  // 0 for an empty wave
            l += red[x][1][d] * e;
            o += red[x][2][d] * e;
        }
    const float res = l > 0.f ? o / l : 0.f;
    Elem* O = out_arg + (size_t)bseq * o_b + (size_t)h * o_h;
    O[(size_t)g * o_r + d] = T::from_float(res);
    if (lse_arg && d == 0) lse_arg[(size_t)bh * L + g] = lse_of(M, l);
}

}  // namespace

// Device scratch of the allocation-free forward (lf_attn_forward_static): the global-row
// partials of a call live in this array instead of a handle workspace.  Each GPU the
// library runs on holds its own copy until the process ends.
static __device__ __align__(256) char scratch[LF_STATIC_SCRATCH_BYTES];

hipError_t static_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        // The host-side name `scratch` is not a device address: take this device's
        // address of the array once, with the device current, and use only that.
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

namespace {
// The band kernel's dilation argument: the dilation every head shares; else, for at
// most 15 heads with dilations 1..4, -(1 + sum of (dil[h] - 1) << 2h) (decoded without a
// memory read); else 0 (each head's entry is read from the arguments).
int dil_code(const Params& p) {
    if (p.dil_u) return p.dil_u;
    if (p.H > 15) return 0;
    int packed = 0;
    for (int h = 0; h < p.H; ++h) {
        if (p.dil[h] < 1 || p.dil[h] > 4) return 0;
        packed |= (p.dil[h] - 1) << (2 * h);
    }
    return -(1 + packed);
}

template <class T, bool kCausal, bool kBias, bool kRandom>
void launch_band_t(const Params& p, int blocks, hipStream_t s) {
    if constexpr (!kBias && !kRandom) {
        if (p.rows_per_block == kSplitRows && !p.strided) {
            (void)launch_kernel(band_kernel<T, kCausal, false, false, false, true>, dim3(blocks), dim3(kThreads), s,
                                blocks, p.tiles_per_head, p.H, p.L, dil_code(p), p.q, p.B, p);
            return;
        }
    }
    if constexpr (std::is_same_v<T, Bf16>) {
        if (p.strided) {
            (void)launch_kernel(band_kernel<T, kCausal, kBias, kRandom, true>, dim3(blocks), dim3(kThreads), s, blocks,
                                p.tiles_per_head, p.H, p.L, dil_code(p), p.q, p.B, p);
            return;
        }
    }
    (void)launch_kernel(band_kernel<T, kCausal, kBias, kRandom>, dim3(blocks), dim3(kThreads), s, blocks,
                        p.tiles_per_head, p.H, p.L, dil_code(p), p.q, p.B, p);
}
}  // namespace

hipError_t launch_band(const Params& p, int dtype, hipStream_t s) {
    const int blocks = p.B * p.H * p.tiles_per_head;
    if (blocks <= 0) return hipSuccess;
    const bool bias = p.bias != nullptr, rnd = p.rnd != nullptr;
#define LF_BAND(T, C, Bi, R) launch_band_t<T, C, Bi, R>(p, blocks, s)
#define LF_BAND_R(T, C, Bi) \
    if (rnd) LF_BAND(T, C, Bi, true); else LF_BAND(T, C, Bi, false)
#define LF_BAND_BR(T, C) \
    if (bias) { LF_BAND_R(T, C, true); } else { LF_BAND_R(T, C, false); }
    if (dtype == LF_BF16) {
        if (p.causal) { LF_BAND_BR(Bf16, true); } else { LF_BAND_BR(Bf16, false); }
    } else {
        if (p.causal) { LF_BAND_BR(F32, true); } else { LF_BAND_BR(F32, false); }
    }
#undef LF_BAND_BR
#undef LF_BAND_R
#undef LF_BAND
    return hipGetLastError();
}

hipError_t launch_merge(const Params& p, int dtype, hipStream_t s) {
    if (p.n_g == 0 || p.B == 0) return hipSuccess;
    if (p.B > 65535) return hipErrorInvalidConfiguration;  // grid z
    const dim3 grid(p.n_g, p.H, p.B);
    const int waves = merge_waves(p.tiles_per_head, kMergeChunk, kMergeWaves);
    const int n_gq = p.n_gblk * kGlobalQueriesPerBlock;
#define LF_MERGE(T)                                                                                        \
    launch_kernel(merge_kernel<T>, grid, dim3(64 * waves), s, p.tiles_per_head, n_gq, p.H, p.L, p.dil_u, \
                  (const float*)p.ws_ml, (const float*)p.ws_acc, p)
    if (dtype == LF_BF16) {
        LF_MERGE(Bf16);
    } else {
        LF_MERGE(F32);
    }
#undef LF_MERGE
    return hipGetLastError();
}

}  // namespace lf
