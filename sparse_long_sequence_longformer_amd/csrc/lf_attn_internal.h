// Internal interface between the host planner (lf_attn.cpp) and the gfx950
// kernels (lf_attn_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "lf_attn.h"

namespace lf {

// Rows of one band work-group (4 waves x 32 query rows) and keys of one
// staged K/V tile.
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
    const uint8_t* pad;  // [B][L] or nullptr
    float* ws_ml;        // [B*H][n_gq][n_chunks][2]  (running max, sum) of each key chunk
    float* ws_acc;       // [B*H][n_gq][n_chunks][64] unnormalised output of each key chunk
    int B, H, L, w;
    int n_g;             // number of distinct global positions
    int n_gblk;          // ceil(n_g / 32)
    int tiles_per_head;  // band work-groups per (b, h), max over heads
    int chunk;           // keys per global-row work-group (multiple of 256)
    int n_chunks;        // ceil(L / chunk)
    int dil[LF_MAX_HEADS];
    int g[LF_MAX_GLOBALS];  // sorted, distinct
};

// Launchers (defined in lf_attn_kernels.hip).  Return the launch error.
hipError_t launch_band(const Params& p, int dtype, hipStream_t s);
hipError_t launch_global_rows(const Params& p, int dtype, hipStream_t s);
hipError_t launch_merge(const Params& p, int dtype, hipStream_t s);

}  // namespace lf
