// Internal interface between the host planner (lf_attn.cpp) and the gfx950
// kernel (lf_attn_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "lf_attn.h"

namespace lf {

// Rows of one work-group (4 waves x 32 query rows) and keys of one staged K/V tile.
constexpr int kRowsPerBlock = 128;
// Rows of a work-group of the split forward: two 32-row blocks, each computed by two
// waves that take alternate 32-key sub-tiles of every stage (twice the waves of a
// 128-row tiling for the same rows, for grids that would fill half the GPU or less).
constexpr int kSplitRows = 64;
constexpr int kKeysPerTile = 64;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kGlobalQueriesPerBlock = 32;
constexpr int kRandomBlock = LF_RANDOM_BLOCK;  // keys of one random block = one staged tile
static_assert(kRandomBlock == kKeysPerTile && kRowsPerBlock == 2 * kRandomBlock,
              "a row tile holds two query blocks and a stage one key block");

// Kernel parameters, passed by value (kernarg segment, < 2 KiB).
struct Params {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    // Separate projections of the global query rows (same layout as q, k, v), or all
    // nullptr: global rows then use q, k, v like every other row.
    const void* qg;
    const void* kg;
    const void* vg;
    const uint8_t* pad;  // [B][L] or nullptr
    float* lse;          // [B][H][L] natural-log sum of each row's exp(scores), or nullptr
    const float* bias;   // relative position bias [H][2*bias_w + 1] of window pairs, or nullptr
    int bias_w;
    // Random key blocks of kRandomBlock keys: row qb of head h at rnd[(h*rnd_nq + qb)*rnd_r]
    // lists the key blocks query block qb drew, ascending, then -1; or nullptr.
    const int* rnd;
    int rnd_nq, rnd_r;
    // Global-row partials: one (max, sum, 64 outputs) per (b*H + h, row tile, global
    // query), written by every work-group for its own 128 "home" keys.
    float* ws_ml;        // [B*H][tiles_per_head][n_gblk*32][2]
    float* ws_acc;       // [B*H][tiles_per_head][n_gblk*32][64]
    int B, H, L, w;
    int n_g;             // number of distinct global positions
    int n_gblk;          // ceil(n_g / 32)
    int tiles_per_head;  // work-groups per (b, h), max over heads (grid partition)
    int rows_per_block;  // rows of one residue class per forward work-group (128, or 64 split)
    int causal;          // one-sided variant: no pair with its key after its query
    // Global sets: g[0..n_g) shared by every sequence (gstride 0), or row b at
    // g[b*gstride ..] with gcnt[b] entries (n_g = the largest count).  Sorted, distinct.
    int gstride;
    int dil[LF_MAX_HEADS];
    int g[LF_MAX_GLOBALS];
    int gcnt[LF_MAX_GLOBALS];
    // Element strides: row i of (b, h) of q, k, v (and q_g, k_g, v_g) at
    // b*s_b + h*s_h + i*s_r, of out at b*o_b + h*o_h + i*o_r.  [B][H][L][64]:
    // (H*L*64, L*64, 64); the layer's QKV projection output [B][L][3][H][64]:
    // (3*L*E, 64, 3*E) with E = 64*H, and its merged-heads output (L*E, 64, E).
    long long s_b, s_h, o_b, o_h;
    int s_r, o_r;
    int strided;  // strides other than [B][H][L][64] (bf16 only)
    int dil_u;    // the dilation of every head when they share one, else 0
};

// Events of the kernel launch in progress, set by the host around one launch when
// per-launch timing is on.  The launchers pass them to hipExtLaunchKernel, which
// stamps them with the kernel's own start and end (no separate event packets
// between kernels); `used` tells the host that a kernel was launched with them.
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
    bool used = false;
};
LaunchEvents& launch_events();  // this thread's (defined in lf_attn.cpp)

// Launchers (defined in lf_attn_kernels.hip).  Return the launch error.
hipError_t launch_band(const Params& p, int dtype, hipStream_t s);
hipError_t launch_merge(const Params& p, int dtype, hipStream_t s);
// This device's address of the static scratch array of LF_STATIC_SCRATCH_BYTES bytes
// (taken with hipGetSymbolAddress on the first call per device, then cached).
hipError_t static_scratch(void** ptr);

// Backward parameters (bf16 tensors, fp32 statistics and partials).
struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;     // forward output
    const void* dout;  // gradient of the output
    void* dq;
    void* dk;
    void* dv;
    const uint8_t* pad;  // [B][L] or nullptr
    const float* lse;    // [B][H][L] natural-log row sums of the forward
    const float* bias;   // relative position bias as in Params, or nullptr
    int bias_w;
    const int* rnd;      // random key blocks as in Params, or nullptr
    int rnd_nq, rnd_r;
    // Inverse of rnd: row kb of head h at rnd_inv[(h*rnd_nq + kb)*rnd_inv_r] lists the
    // query blocks that drew key block kb, ascending, then -1.
    const int* rnd_inv;
    int rnd_inv_r;
    // Separate projections of the global rows (sep != 0): q_g, k_g, v_g inputs and their
    // gradients dq_g, dk_g, dv_g (same layout as q).  Global rows then attend with them
    // only; the other rows, and every key they attend, use q, k, v.
    int sep;
    const void* qg;
    const void* kg;
    const void* vg;
    void* dqg;
    void* dkg;
    void* dvg;
    // Row statistics written by the prep kernel, [B][H][L] each:
    float* lse2;       // lse in base-2 units of the pre-scaled scores; +inf for rows without keys
    float* lse2_band;  // same, and +inf for global rows (they are not window queries)
    float* dsum;       // D = dO . O of every row
    // Partials of the global rows and keys, [B*H][tiles_per_head][n_gblk*32][64]:
    float* ws_dq;  // dQ of global queries over each tile's home keys
    float* ws_dk;  // dK of global keys from each tile's home queries outside their window
    float* ws_dv;  // dV, same pairs
    // [B*H][n_gblk*32][64]: dK and dV of each global key from its own tile
    float* ws_dkg;
    float* ws_dvg;
    // Gradient of the relative position bias table (dbias != nullptr): each dQ work-group
    // writes its sums of dS per window offset to ws_db [B*H][tiles_per_head][2w+1]; the
    // reduction kernel adds them up per head into dbias [H][2w+1].
    float* ws_db;
    float* dbias;
    int B, H, L, w;
    int n_g;
    int n_gblk;
    int tiles_per_head;
    int causal;  // one-sided variant
    int gstride;  // global sets as in Params
    int dil[LF_MAX_HEADS];
    int g[LF_MAX_GLOBALS];
    int gcnt[LF_MAX_GLOBALS];
    int dtype;  // LF_BF16 or LF_F32 tensors
    int dil_u;  // the dilation of every head when they share one, else 0
};

// Launchers of the layer's pointwise passes (defined in lf_layer.hip).
// GEMM outputs: h bf16, y (the input of a LayerNorm) fp32.
hipError_t launch_bias_residual_ln(const float* y, const void* bias, const void* res, const void* gamma,
                                   const void* beta, float eps, void* out, int E, long long R, hipStream_t s);
hipError_t launch_bias_gelu(const void* h, const void* bias, void* out, int F, long long R, hipStream_t s);

// Launchers (defined in lf_attn_bwd.hip).
hipError_t launch_bwd_prep(const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_dkv(const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_dkv_global_proj(const BwdParams& p, hipStream_t s);  // dk_g, dv_g (sep only)
hipError_t launch_bwd_merge(const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_dbias(const BwdParams& p, hipStream_t s);  // dbias (only with p.dbias)

}  // namespace lf
