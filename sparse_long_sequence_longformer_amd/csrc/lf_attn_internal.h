// Internal interface between the host planner (lf_attn.cpp) and the gfx950
// kernel (lf_attn_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "lf_attn.h"

namespace lf {

// Rows of one work-group (4 waves x 32 query rows) and keys of one staged K/V tile.
constexpr int kRowsPerBlock = 128;
constexpr int kKeysPerTile = 64;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kGlobalQueriesPerBlock = 32;

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
    // Global-row partials: one (max, sum, 64 outputs) per (b*H + h, row tile, global
    // query), written by every work-group for its own 128 "home" keys.
    float* ws_ml;        // [B*H][tiles_per_head][n_gblk*32][2]
    float* ws_acc;       // [B*H][tiles_per_head][n_gblk*32][64]
    int B, H, L, w;
    int n_g;             // number of distinct global positions
    int n_gblk;          // ceil(n_g / 32)
    int tiles_per_head;  // work-groups per (b, h), max over heads (grid partition)
    int rows_per_block;  // rows of one residue class per work-group
    int dil[LF_MAX_HEADS];
    int g[LF_MAX_GLOBALS];          // sorted, distinct
};

// Launchers (defined in lf_attn_kernels.hip).  Return the launch error.
hipError_t launch_band(const Params& p, int dtype, hipStream_t s);
hipError_t launch_merge(const Params& p, int dtype, hipStream_t s);

}  // namespace lf
