// Host side of liblfattn.so: argument validation, launch planning, device
// workspace, per-stage timing.  Everything here runs before any kernel is
// enqueued; on error nothing is launched and `out` is untouched.

#include <hip/hip_runtime_api.h>
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "lf_attn.h"
#include "lf_attn_internal.h"

namespace {

struct TimedLaunch {
    hipEvent_t start;
    hipEvent_t stop;
    int stage;
};

}  // namespace

// One GEMM shape's hipBLASLt descriptors and the algorithm chosen for it.
struct GemmPlan {
    int M = 0, N = 0, K = 0;
    bool f32_out = false;
    bool bias = false;  // epilogue adds a bf16 bias vector of N entries (pointer set per call)
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    size_t ws = 0;
};

struct lf_attn_s {
    lf_dtype dtype;
    int window_mode = LF_WINDOW_SYMMETRIC;
    int global_mode = LF_GLOBALS_SHARED;
    const float* bias = nullptr;  // borrowed [bias_heads][2 * bias_w + 1], or null
    int bias_heads = 0;
    int bias_w = 0;
    // Random key blocks: per head and query block the sorted distinct draws (-1 after
    // them), [rnd_heads][rnd_nq][rnd_r], and the inverse lists (query blocks per key
    // block), [rnd_heads][rnd_nq][rnd_inv_r]; uploaded to rnd_dev on first use.
    bool rnd_on = false;
    int rnd_heads = 0, rnd_nq = 0, rnd_r = 0, rnd_inv_r = 0;
    std::vector<int32_t> rnd_tab, rnd_inv_tab;
    char* rnd_dev = nullptr;
    size_t rnd_dev_bytes = 0;
    int rnd_dev_device = -1;
    int rnd_uploaded = -1;  // device holding the current tables, or -1
    int device = -1;
    char* ws = nullptr;  // global-row partials of the forward
    size_t ws_bytes = 0;
    int ws_device = -1;
    char* ws_bwd = nullptr;  // row statistics and global partials of the backward
    size_t ws_bwd_bytes = 0;
    int ws_bwd_device = -1;
    char* ws_layer = nullptr;  // intermediates of the layer
    size_t ws_layer_bytes = 0;
    int ws_layer_device = -1;
    // hipBLASLt for the layer's GEMMs: one handle and plan cache per device in use.
    hipblasLtHandle_t lt = nullptr;
    int lt_device = -1;
    std::vector<GemmPlan> gemm_plans;
    char* ws_gemm = nullptr;  // hipBLASLt workspace
    size_t ws_gemm_bytes = 0;
    int ws_gemm_device = -1;
    std::string last_error;
    // Failure injection for tests, from the environment variable LF_ATTN_FAULT when
    // the handle is created: "alloc" fails the handle's next workspace allocation as if
    // hipMalloc had (LF_ERR_OOM), "launch" its next kernel launch before it is enqueued
    // (LF_ERR_HIP); once, then the handle works normally.  Anything else (or unset):
    // none.
    int fault = 0;
    // Rows per forward work-group (lf_attn_set_tile_rows): 0 chooses, 64 or 128 forces.
    int tile_rows = 0;
    int n_cu = 0, n_cu_device = -1;  // compute units of the device last asked
    bool timing = false;
    std::vector<TimedLaunch> pending;  // recorded, not yet read
    std::vector<hipEvent_t> event_pool;
    double stage_ms[LF_N_STAGES] = {};
    int64_t stage_n[LF_N_STAGES] = {};
};

namespace lf {

LaunchEvents& launch_events() {
    static thread_local LaunchEvents ev;
    return ev;
}

}  // namespace lf

namespace {

constexpr int kFaultAlloc = 1;
constexpr int kFaultLaunch = 2;

lf_status release_gemm(lf_attn_t h);

lf_status fail(lf_attn_t h, lf_status s, const char* fmt, ...) {
    if (h) {
        char buf[512];
        va_list ap;
        va_start(ap, fmt);
        std::vsnprintf(buf, sizeof(buf), fmt, ap);
        va_end(ap);
        h->last_error = buf;
    }
    return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, const void* b, size_t n) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + n && y < x + n;
}

// The dilation shared by every head of dil[0..H), or 0 when the heads differ (the
// kernels then read each head's own entry).
int uniform_dilation(const int* dil, int H) {
    for (int i = 1; i < H; ++i)
        if (dil[i] != dil[0]) return 0;
    return H > 0 ? dil[0] : 0;
}

// [a, a + na) and [b, b + nb) intersect.
bool overlaps2(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

hipEvent_t take_event(lf_attn_t h) {
    if (!h->event_pool.empty()) {
        hipEvent_t e = h->event_pool.back();
        h->event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

void release_events(lf_attn_t h) {
    for (auto& t : h->pending) {
        h->event_pool.push_back(t.start);
        h->event_pool.push_back(t.stop);
    }
    h->pending.clear();
}

}  // namespace

extern "C" {

const char* lf_attn_status_string(lf_status s) {
    switch (s) {
        case LF_OK: return "ok";
        case LF_ERR_INVALID_ARG: return "invalid argument";
        case LF_ERR_UNSUPPORTED: return "unsupported argument";
        case LF_ERR_HIP: return "HIP runtime error";
        case LF_ERR_OOM: return "device memory allocation failed";
    }
    return "unknown status";
}

lf_status lf_attn_create(lf_attn_t* out, lf_dtype dtype) {
    if (!out) return LF_ERR_INVALID_ARG;
    *out = nullptr;
    if (dtype != LF_F32 && dtype != LF_BF16) return LF_ERR_UNSUPPORTED;
    lf_attn_t h = new (std::nothrow) lf_attn_s;
    if (!h) return LF_ERR_OOM;
    h->dtype = dtype;
    if (const char* f = std::getenv("LF_ATTN_FAULT")) {
        if (std::strcmp(f, "alloc") == 0) h->fault = kFaultAlloc;
        if (std::strcmp(f, "launch") == 0) h->fault = kFaultLaunch;
    }
    *out = h;
    return LF_OK;
}

const char* lf_attn_last_error(lf_attn_t h) { return h ? h->last_error.c_str() : ""; }

lf_status lf_attn_destroy(lf_attn_t h) {
    if (!h) return LF_OK;
    lf_status st = LF_OK;
    if (h->ws && hipFree(h->ws) != hipSuccess) st = LF_ERR_HIP;
    if (h->ws_bwd && hipFree(h->ws_bwd) != hipSuccess) st = LF_ERR_HIP;
    if (h->ws_layer && hipFree(h->ws_layer) != hipSuccess) st = LF_ERR_HIP;
    if (h->rnd_dev && hipFree(h->rnd_dev) != hipSuccess) st = LF_ERR_HIP;
    if (h->ws_gemm && hipFree(h->ws_gemm) != hipSuccess) st = LF_ERR_HIP;
    if (release_gemm(h) != LF_OK) st = LF_ERR_HIP;
    release_events(h);
    for (hipEvent_t e : h->event_pool) (void)hipEventDestroy(e);
    delete h;
    return st;
}

lf_status lf_attn_set_global_mode(lf_attn_t h, int mode) {
    if (!h) return LF_ERR_INVALID_ARG;
    h->last_error.clear();
    if (mode != LF_GLOBALS_SHARED && mode != LF_GLOBALS_PER_SEQUENCE)
        return fail(h, LF_ERR_INVALID_ARG, "unknown global mode %d", mode);
    h->global_mode = mode;
    return LF_OK;
}

lf_status lf_attn_set_tile_rows(lf_attn_t h, int rows) {
    if (!h) return LF_ERR_INVALID_ARG;
    h->last_error.clear();
    if (rows != 0 && rows != lf::kSplitRows && rows != lf::kRowsPerBlock)
        return fail(h, LF_ERR_INVALID_ARG, "tile rows must be 0, %d or %d (got %d)", lf::kSplitRows,
                    lf::kRowsPerBlock, rows);
    h->tile_rows = rows;
    return LF_OK;
}

lf_status lf_attn_set_window_mode(lf_attn_t h, int mode) {
    if (!h) return LF_ERR_INVALID_ARG;
    h->last_error.clear();
    if (mode != LF_WINDOW_SYMMETRIC && mode != LF_WINDOW_CAUSAL)
        return fail(h, LF_ERR_INVALID_ARG, "unknown window mode %d", mode);
    h->window_mode = mode;
    return LF_OK;
}

lf_status lf_attn_set_position_bias(lf_attn_t h, const float* table, int n_heads, int w) {
    if (!h) return LF_ERR_INVALID_ARG;
    h->last_error.clear();
    if (!table) {
        h->bias = nullptr;
        h->bias_heads = h->bias_w = 0;
        return LF_OK;
    }
    if (n_heads < 1 || n_heads > LF_MAX_HEADS)
        return fail(h, LF_ERR_INVALID_ARG, "need 1 <= n_heads <= %d (got %d)", LF_MAX_HEADS, n_heads);
    if (w < 0) return fail(h, LF_ERR_INVALID_ARG, "need w >= 0 (got %d)", w);
    if (w > LF_MAX_BIAS_W)
        return fail(h, LF_ERR_UNSUPPORTED, "position bias: at most w = %d (got %d)", LF_MAX_BIAS_W, w);
    if ((reinterpret_cast<uintptr_t>(table) & 3u) != 0)
        return fail(h, LF_ERR_INVALID_ARG, "the bias table must be 4-byte aligned");
    h->bias = table;
    h->bias_heads = n_heads;
    h->bias_w = w;
    return LF_OK;
}

lf_status lf_attn_set_random_blocks(lf_attn_t h, const int32_t* blocks, int n_heads, int n_qblocks, int r) {
    if (!h) return LF_ERR_INVALID_ARG;
    h->last_error.clear();
    if (!blocks) {
        h->rnd_on = false;
        h->rnd_tab.clear();
        h->rnd_inv_tab.clear();
        h->rnd_uploaded = -1;
        return LF_OK;
    }
    if (n_heads < 1 || n_heads > LF_MAX_HEADS)
        return fail(h, LF_ERR_INVALID_ARG, "need 1 <= n_heads <= %d (got %d)", LF_MAX_HEADS, n_heads);
    if (n_qblocks < 1) return fail(h, LF_ERR_INVALID_ARG, "need n_qblocks >= 1 (got %d)", n_qblocks);
    if (r < 0) return fail(h, LF_ERR_INVALID_ARG, "need r >= 0 (got %d)", r);
    if (r > LF_MAX_RANDOM_DRAWS)
        return fail(h, LF_ERR_UNSUPPORTED, "at most %d random blocks per query block (got %d)", LF_MAX_RANDOM_DRAWS, r);
    const size_t rows = static_cast<size_t>(n_heads) * n_qblocks;
    std::vector<std::vector<int>> fwd(rows), inv(rows);
    size_t R = 1, RI = 1;
    for (size_t row = 0; row < rows; ++row) {
        for (int t = 0; t < r; ++t) {
            const int kb = blocks[row * r + t];
            if (kb < 0) continue;
            if (kb >= n_qblocks)
                return fail(h, LF_ERR_INVALID_ARG, "random block %d of head %zu, query block %zu outside [0, %d)", kb,
                            row / n_qblocks, row % n_qblocks, n_qblocks);
            fwd[row].push_back(kb);
        }
        std::sort(fwd[row].begin(), fwd[row].end());
        fwd[row].erase(std::unique(fwd[row].begin(), fwd[row].end()), fwd[row].end());
        R = std::max(R, fwd[row].size());
        const size_t hb = (row / n_qblocks) * n_qblocks;  // first row of this head
        for (int kb : fwd[row]) inv[hb + kb].push_back(static_cast<int>(row % n_qblocks));
    }
    for (const auto& v : inv) RI = std::max(RI, v.size());  // query blocks arrive in ascending order
    h->rnd_tab.assign(rows * R, -1);
    h->rnd_inv_tab.assign(rows * RI, -1);
    for (size_t row = 0; row < rows; ++row) {
        std::copy(fwd[row].begin(), fwd[row].end(), h->rnd_tab.begin() + row * R);
        std::copy(inv[row].begin(), inv[row].end(), h->rnd_inv_tab.begin() + row * RI);
    }
    h->rnd_on = true;
    h->rnd_heads = n_heads;
    h->rnd_nq = n_qblocks;
    h->rnd_r = static_cast<int>(R);
    h->rnd_inv_r = static_cast<int>(RI);
    h->rnd_uploaded = -1;
    return LF_OK;
}

lf_status lf_attn_set_stage_timing(lf_attn_t h, int enable) {
    if (!h) return LF_ERR_INVALID_ARG;
    h->timing = enable != 0;
    release_events(h);
    for (int i = 0; i < LF_N_STAGES; ++i) {
        h->stage_ms[i] = 0;
        h->stage_n[i] = 0;
    }
    return LF_OK;
}

lf_status lf_attn_stage_times(lf_attn_t h, double* ms, int64_t* launches) {
    if (!h) return LF_ERR_INVALID_ARG;
    for (auto& t : h->pending) {
        if (hipEventSynchronize(t.stop) != hipSuccess) return fail(h, LF_ERR_HIP, "hipEventSynchronize failed");
        float e = 0.f;
        if (hipEventElapsedTime(&e, t.start, t.stop) != hipSuccess)
            return fail(h, LF_ERR_HIP, "hipEventElapsedTime failed");
        h->stage_ms[t.stage] += e;
        h->stage_n[t.stage] += 1;
    }
    release_events(h);
    for (int i = 0; i < LF_N_STAGES; ++i) {
        if (ms) ms[i] = h->stage_ms[i];
        if (launches) launches[i] = h->stage_n[i];
        h->stage_ms[i] = 0;
        h->stage_n[i] = 0;
    }
    return LF_OK;
}

}  // extern "C"

namespace {

// Shape, pattern and plan shared by the forward and the backward: validated
// arguments, sorted distinct globals, per-head residue tiling.
struct Plan {
    int B, H, L, w;
    int dil[LF_MAX_HEADS];
    std::vector<int> g;     // shared set, or the per-sequence rows back to back (stride gstride)
    std::vector<int> gcnt;  // per-sequence counts (per-sequence mode)
    int n_g;                // shared count, or the largest per-sequence count
    int gstride;            // 0: shared
    int n_gblk;
    int tiles;
    size_t bytes;  // of one [B][H][L][d_h] tensor
};

lf_status make_plan(lf_attn_t h, Plan& pl, int B, int H, int L, int d_h, int w, const int32_t* dil_per_head,
                    const int32_t* global_idx, int n_global) {
    if (B < 1 || H < 1 || L < 1) return fail(h, LF_ERR_INVALID_ARG, "need B, H, L >= 1 (got %d, %d, %d)", B, H, L);
    if (d_h != LF_HEAD_DIM) return fail(h, LF_ERR_UNSUPPORTED, "only d_h = 64 is supported (got %d)", d_h);
    if (H > LF_MAX_HEADS) return fail(h, LF_ERR_UNSUPPORTED, "at most %d heads (got %d)", LF_MAX_HEADS, H);
    if (w < 0) return fail(h, LF_ERR_INVALID_ARG, "need w >= 0 (got %d)", w);
    if (!dil_per_head) return fail(h, LF_ERR_INVALID_ARG, "dil_per_head must be non-null");
    if (n_global < 0) return fail(h, LF_ERR_INVALID_ARG, "need n_global >= 0 (got %d)", n_global);
    if (n_global > LF_MAX_GLOBALS)
        return fail(h, LF_ERR_UNSUPPORTED, "at most %d global indices (got %d)", LF_MAX_GLOBALS, n_global);
    if (n_global > 0 && !global_idx) return fail(h, LF_ERR_INVALID_ARG, "global_idx is NULL but n_global > 0");
    if (h->bias && (H != h->bias_heads || w != h->bias_w))
        return fail(h, LF_ERR_INVALID_ARG, "the position bias table is for H = %d, w = %d (call: H = %d, w = %d)",
                    h->bias_heads, h->bias_w, H, w);
    if (h->rnd_on) {
        const int nq = (L + LF_RANDOM_BLOCK - 1) / LF_RANDOM_BLOCK;
        if (H != h->rnd_heads || nq != h->rnd_nq)
            return fail(h, LF_ERR_INVALID_ARG,
                        "the random blocks are for H = %d, %d query blocks (call: H = %d, L = %d gives %d)",
                        h->rnd_heads, h->rnd_nq, H, L, nq);
        for (int i = 0; i < H; ++i)
            if (dil_per_head[i] != 1)
                return fail(h, LF_ERR_UNSUPPORTED, "random blocks need every head undilated (dil_per_head[%d] = %d)",
                            i, dil_per_head[i]);
    }
    const size_t elem = h->dtype == LF_BF16 ? 2 : 4;
    const uint64_t n_elem = static_cast<uint64_t>(B) * H * L * LF_HEAD_DIM;
    if (n_elem / LF_HEAD_DIM / L / H != static_cast<uint64_t>(B) || n_elem > (uint64_t(1) << 40))
        return fail(h, LF_ERR_INVALID_ARG, "tensor size overflows");
    pl.bytes = static_cast<size_t>(n_elem) * elem;
    for (int i = 0; i < H; ++i) {
        if (dil_per_head[i] < 1) return fail(h, LF_ERR_INVALID_ARG, "dil_per_head[%d] = %d < 1", i, dil_per_head[i]);
        pl.dil[i] = dil_per_head[i];
    }
    if (h->global_mode == LF_GLOBALS_PER_SEQUENCE) {
        // global_idx is [B][n_global]; negative entries are unused.
        if (static_cast<int64_t>(B) * n_global > LF_MAX_GLOBALS || B > LF_MAX_GLOBALS)
            return fail(h, LF_ERR_UNSUPPORTED, "per-sequence globals: at most %d entries in all (got %d x %d)",
                        LF_MAX_GLOBALS, B, n_global);
        std::vector<std::vector<int>> rows(B);
        int mx = 0;
        for (int b = 0; b < B; ++b) {
            for (int i = 0; i < n_global; ++i) {
                const int g = global_idx[static_cast<size_t>(b) * n_global + i];
                if (g < 0) continue;
                if (g >= L) return fail(h, LF_ERR_INVALID_ARG, "global_idx[%d][%d] = %d outside [0, %d)", b, i, g, L);
                rows[b].push_back(g);
            }
            std::sort(rows[b].begin(), rows[b].end());
            rows[b].erase(std::unique(rows[b].begin(), rows[b].end()), rows[b].end());
            mx = std::max<int>(mx, static_cast<int>(rows[b].size()));
        }
        pl.gstride = mx;
        pl.n_g = mx;
        pl.g.assign(static_cast<size_t>(B) * mx, 0);
        pl.gcnt.assign(B, 0);
        for (int b = 0; b < B; ++b) {
            std::copy(rows[b].begin(), rows[b].end(), pl.g.begin() + static_cast<size_t>(b) * mx);
            pl.gcnt[b] = static_cast<int>(rows[b].size());
        }
    } else {
        pl.g.assign(global_idx, global_idx + n_global);
        for (int i = 0; i < n_global; ++i)
            if (pl.g[i] < 0 || pl.g[i] >= L)
                return fail(h, LF_ERR_INVALID_ARG, "global_idx[%d] = %d outside [0, %d)", i, pl.g[i], L);
        std::sort(pl.g.begin(), pl.g.end());
        pl.g.erase(std::unique(pl.g.begin(), pl.g.end()), pl.g.end());
        pl.n_g = static_cast<int>(pl.g.size());
        pl.gstride = 0;
    }
    pl.B = B;
    pl.H = H;
    pl.L = L;
    pl.w = std::min(w, L);  // |j - i| < L always, so a wider window changes nothing
    pl.n_gblk = (pl.n_g + lf::kGlobalQueriesPerBlock - 1) / lf::kGlobalQueriesPerBlock;
    int tiles = 0;
    for (int i = 0; i < H; ++i) {
        const int d = pl.dil[i];
        const int len0 = (L + d - 1) / d;  // rows of residue class 0 (the longest)
        const int per_class = (len0 + lf::kRowsPerBlock - 1) / lf::kRowsPerBlock;
        const int64_t t = static_cast<int64_t>(d) * per_class;
        if (t > 0x7fffffff) return fail(h, LF_ERR_UNSUPPORTED, "grid too large");
        tiles = std::max<int>(tiles, static_cast<int>(t));
    }
    pl.tiles = tiles;
    if (static_cast<int64_t>(B) * H * tiles > 0x7fffffff) return fail(h, LF_ERR_UNSUPPORTED, "grid too large");
    return LF_OK;
}

// Grow one of the handle's device workspaces to at least `need` bytes.
// Drop the hipBLASLt plans and handle (made on another device, or at destruction).
lf_status release_gemm(lf_attn_t h) {
    bool ok = true;
    for (GemmPlan& g : h->gemm_plans) {
        ok &= hipblasLtMatrixLayoutDestroy(g.c) == HIPBLAS_STATUS_SUCCESS;
        ok &= hipblasLtMatrixLayoutDestroy(g.b) == HIPBLAS_STATUS_SUCCESS;
        ok &= hipblasLtMatrixLayoutDestroy(g.a) == HIPBLAS_STATUS_SUCCESS;
        ok &= hipblasLtMatmulDescDestroy(g.desc) == HIPBLAS_STATUS_SUCCESS;
    }
    h->gemm_plans.clear();
    if (h->lt) ok &= hipblasLtDestroy(h->lt) == HIPBLAS_STATUS_SUCCESS;
    h->lt = nullptr;
    h->lt_device = -1;
    return ok ? LF_OK : LF_ERR_HIP;
}

lf_status reserve(lf_attn_t h, char** buf, size_t* have, int* dev, size_t need) {
    if (need <= *have && *dev == h->device) return LF_OK;
    if (h->fault == kFaultAlloc) {  // the old buffer stays: the handle remains usable
        h->fault = 0;
        return fail(h, LF_ERR_OOM, "hipMalloc of %zu workspace bytes failed (LF_ATTN_FAULT=alloc)", need);
    }
    if (*buf) (void)hipFree(*buf);
    *buf = nullptr;
    *have = 0;
    if (hipMalloc(reinterpret_cast<void**>(buf), need) != hipSuccess) {
        (void)hipGetLastError();
        return fail(h, LF_ERR_OOM, "hipMalloc of %zu workspace bytes failed", need);
    }
    *have = need;
    *dev = h->device;
    return LF_OK;
}

// Device copies of the random-block tables (synchronous upload after a change).
lf_status upload_random(lf_attn_t h) {
    if (!h->rnd_on || h->rnd_uploaded == h->device) return LF_OK;
    const size_t n_fwd = h->rnd_tab.size(), n_inv = h->rnd_inv_tab.size();
    lf_status st = reserve(h, &h->rnd_dev, &h->rnd_dev_bytes, &h->rnd_dev_device, (n_fwd + n_inv) * sizeof(int32_t));
    if (st != LF_OK) return st;
    // Earlier calls may still read the old tables.
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(h->rnd_dev, h->rnd_tab.data(), n_fwd * sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(h->rnd_dev + n_fwd * sizeof(int32_t), h->rnd_inv_tab.data(), n_inv * sizeof(int32_t),
                  hipMemcpyHostToDevice) != hipSuccess)
        return fail(h, LF_ERR_HIP, "upload of the random-block tables failed");
    h->rnd_uploaded = h->device;
    return LF_OK;
}

// Enqueue one launch.  With timing on, a kernel of this library is launched with a
// pair of events that hipExtLaunchKernel stamps with the kernel's own start and end;
// a library call (the layer's GEMMs) is bracketed by two recorded events instead.
template <class Launch>
lf_status launch_stage(lf_attn_t h, int stage, hipStream_t s, Launch launch) {
    if (h->fault == kFaultLaunch) {
        h->fault = 0;
        return fail(h, LF_ERR_HIP, "kernel launch failed (LF_ATTN_FAULT=launch)");
    }
    TimedLaunch tl{nullptr, nullptr, stage};
    const bool bracket = stage == LF_STAGE_LAYER_GEMM;
    lf::LaunchEvents& ev = lf::launch_events();
    if (h->timing) {
        tl.start = take_event(h);
        tl.stop = take_event(h);
        if (!tl.start || !tl.stop) return fail(h, LF_ERR_HIP, "hipEventCreate failed");
        if (bracket) {
            if (hipEventRecord(tl.start, s) != hipSuccess) return fail(h, LF_ERR_HIP, "hipEventRecord failed");
        } else {
            ev = lf::LaunchEvents{tl.start, tl.stop, false};
        }
    }
    const hipError_t e = launch();
    const bool stamped = ev.used;
    ev = lf::LaunchEvents{};
    if (e != hipSuccess) {
        if (h->timing) {
            h->event_pool.push_back(tl.start);
            h->event_pool.push_back(tl.stop);
        }
        return fail(h, LF_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    }
    if (h->timing) {
        if (bracket && hipEventRecord(tl.stop, s) != hipSuccess) return fail(h, LF_ERR_HIP, "hipEventRecord failed");
        if (bracket || stamped) {
            h->pending.push_back(tl);
        } else {  // nothing was launched (an empty grid)
            h->event_pool.push_back(tl.start);
            h->event_pool.push_back(tl.stop);
        }
    }
    return LF_OK;
}

// Every forward entry point.  qg, kg, vg are all null (one projection for every
// row) or all non-null (separate projections of the global rows); lse may be null.
// no_alloc: the partials go to the static scratch array (no allocation, no upload,
// no per-launch timing).
// Element strides of q, k, v and of out (see lf::Params); nullptr: [B][H][L][64] each.
struct Strides {
    long long s_b, s_h;
    int s_r;
    long long o_b, o_h;
    int o_r;
};

// Work-groups per head of a forward tiling of `rows` rows per residue class.
int forward_tiles(const Plan& pl, int rows) {
    int tiles = 0;
    for (int i = 0; i < pl.H; ++i) {
        const int d = pl.dil[i];
        const int per_class = ((pl.L + d - 1) / d + rows - 1) / rows;
        tiles = std::max(tiles, d * per_class);
    }
    return tiles;
}

// Rows per forward work-group.  A 128-row work-group gives each of its four waves 32
// rows; when the whole grid would fill at most half of the work-group slots of the
// device (three bf16 work-groups per compute unit, one fp32), the 64-row split tiling
// runs two waves per 32 rows instead (each takes every other 32-key sub-tile of a
// stage), i.e. twice the waves for the same work.  The split form has no variant with a
// position bias, random blocks or strided tensors; the handle setting forces either
// tiling where both exist.
lf_status forward_rows(lf_attn_t h, const Plan& pl, bool strided, int& rows) {
    rows = lf::kRowsPerBlock;
    if (h->bias || h->rnd_on || strided || h->tile_rows == lf::kRowsPerBlock) return LF_OK;
    if (h->tile_rows == lf::kSplitRows) {
        rows = lf::kSplitRows;
        return LF_OK;
    }
    if (h->n_cu_device != h->device) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess)
            return fail(h, LF_ERR_HIP, "hipDeviceGetAttribute(multiprocessor count) failed");
        h->n_cu = n;
        h->n_cu_device = h->device;
    }
    const int64_t slots = static_cast<int64_t>(h->n_cu) * (h->dtype == LF_BF16 ? 3 : 1);
    const int64_t blocks = static_cast<int64_t>(pl.B) * pl.H * pl.tiles;
    if (2 * blocks <= slots) rows = lf::kSplitRows;
    return LF_OK;
}

lf_status forward_impl(lf_attn_t h, const void* q, const void* k, const void* v, const void* qg, const void* kg,
                       const void* vg, void* out, float* lse, int B, int H, int L, int d_h, int w,
                       const int32_t* dil_per_head, const int32_t* global_idx, int n_global,
                       const uint8_t* key_pad_mask, void* stream, bool no_alloc = false,
                       const Strides* strides = nullptr) {
    if (!h) return LF_ERR_INVALID_ARG;
    h->last_error.clear();
    if (!q || !k || !v || !out) return fail(h, LF_ERR_INVALID_ARG, "q, k, v and out must be non-null");
    const bool sep = qg || kg || vg;
    if (sep && !(qg && kg && vg)) return fail(h, LF_ERR_INVALID_ARG, "q_g, k_g and v_g must all be non-null");
    if (sep && (!aligned16(qg) || !aligned16(kg) || !aligned16(vg)))
        return fail(h, LF_ERR_INVALID_ARG, "q_g, k_g and v_g must be 16-byte aligned");
    Plan pl;
    lf_status st = make_plan(h, pl, B, H, L, d_h, w, dil_per_head, global_idx, n_global);
    if (st != LF_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(h, LF_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
    const size_t bytes = pl.bytes;
    if (!strides && (overlaps(out, q, bytes) || overlaps(out, k, bytes) || overlaps(out, v, bytes)))
        return fail(h, LF_ERR_INVALID_ARG, "out must not overlap q, k or v");
    if (sep && (overlaps(out, qg, bytes) || overlaps(out, kg, bytes) || overlaps(out, vg, bytes)))
        return fail(h, LF_ERR_INVALID_ARG, "out must not overlap q_g, k_g or v_g");
    if (lse) {
        const size_t lb = static_cast<size_t>(B) * H * L * sizeof(float);
        if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return fail(h, LF_ERR_INVALID_ARG, "lse must be 4-byte aligned");
        if (overlaps2(lse, lb, q, bytes) || overlaps2(lse, lb, k, bytes) || overlaps2(lse, lb, v, bytes) ||
            overlaps2(lse, lb, out, bytes))
            return fail(h, LF_ERR_INVALID_ARG, "lse must not overlap q, k, v or out");
        if (sep && (overlaps2(lse, lb, qg, bytes) || overlaps2(lse, lb, kg, bytes) || overlaps2(lse, lb, vg, bytes)))
            return fail(h, LF_ERR_INVALID_ARG, "lse must not overlap q_g, k_g or v_g");
    }

    lf::Params p;
    std::memset(&p, 0, sizeof(p));
    std::copy(pl.dil, pl.dil + H, p.dil);
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.qg = qg;
    p.kg = kg;
    p.vg = vg;
    p.pad = key_pad_mask;
    p.lse = lse;
    p.B = B;
    p.H = H;
    p.L = L;
    p.w = pl.w;
    p.n_g = pl.n_g;
    p.gstride = pl.gstride;
    std::copy(pl.g.begin(), pl.g.end(), p.g);
    std::copy(pl.gcnt.begin(), pl.gcnt.end(), p.gcnt);
    p.n_gblk = pl.n_gblk;
    p.causal = h->window_mode == LF_WINDOW_CAUSAL;
    p.bias = h->bias;
    p.bias_w = h->bias_w;
    p.dil_u = uniform_dilation(pl.dil, H);
    if (strides) {
        if (h->dtype != LF_BF16) return fail(h, LF_ERR_UNSUPPORTED, "strided tensors need a bf16 handle");
        p.strided = 1;
        p.s_b = strides->s_b;
        p.s_h = strides->s_h;
        p.s_r = strides->s_r;
        p.o_b = strides->o_b;
        p.o_h = strides->o_h;
        p.o_r = strides->o_r;
    } else {
        p.s_h = p.o_h = static_cast<long long>(L) * LF_HEAD_DIM;
        p.s_b = p.o_b = p.s_h * H;
        p.s_r = p.o_r = LF_HEAD_DIM;
    }

    if (hipGetDevice(&h->device) != hipSuccess) return fail(h, LF_ERR_HIP, "hipGetDevice failed");
    int rows = lf::kRowsPerBlock;
    st = forward_rows(h, pl, p.strided != 0, rows);
    if (st != LF_OK) return st;
    const int tiles = rows == lf::kRowsPerBlock ? pl.tiles : forward_tiles(pl, rows);
    p.rows_per_block = rows;
    p.tiles_per_head = tiles;

    // Device workspace for the global-row partials.
    if (no_alloc) {
        if (h->rnd_on && h->rnd_uploaded != h->device)
            return fail(h, LF_ERR_UNSUPPORTED,
                        "random blocks are set but their tables are not on this device yet (the allocation-free "
                        "forward uploads nothing; call another entry point once on this device first)");
    } else {
        st = upload_random(h);
        if (st != LF_OK) return st;
    }
    if (h->rnd_on) {
        p.rnd = reinterpret_cast<const int*>(h->rnd_dev);
        p.rnd_nq = h->rnd_nq;
        p.rnd_r = h->rnd_r;
    }
    if (p.n_g > 0) {
        const size_t n_part = static_cast<size_t>(B) * H * tiles * p.n_gblk * lf::kGlobalQueriesPerBlock;
        const size_t need = n_part * (2 + 64) * sizeof(float);
        char* base = nullptr;
        if (no_alloc) {
            if (need > static_cast<size_t>(LF_STATIC_SCRATCH_BYTES))
                return fail(h, LF_ERR_UNSUPPORTED,
                            "the global-row partials need %zu bytes; the allocation-free forward has %d",
                            need, LF_STATIC_SCRATCH_BYTES);
            void* sp = nullptr;
            const hipError_t e = lf::static_scratch(&sp);
            if (e != hipSuccess)
                return fail(h, LF_ERR_HIP, "address of the static scratch array: %s", hipGetErrorString(e));
            base = static_cast<char*>(sp);
        } else {
            st = reserve(h, &h->ws, &h->ws_bytes, &h->ws_device, need);
            if (st != LF_OK) return st;
            base = h->ws;
        }
        p.ws_ml = reinterpret_cast<float*>(base);
        p.ws_acc = p.ws_ml + n_part * 2;
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int dt = h->dtype;
    if (no_alloc) {  // no events: their creation could allocate
        if (h->fault == kFaultLaunch) {
            h->fault = 0;
            return fail(h, LF_ERR_HIP, "kernel launch failed (LF_ATTN_FAULT=launch)");
        }
        hipError_t e = lf::launch_band(p, dt, s);
        if (e == hipSuccess && p.n_g > 0) e = lf::launch_merge(p, dt, s);
        if (e != hipSuccess) return fail(h, LF_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
        return LF_OK;
    }
    st = launch_stage(h, LF_STAGE_BAND, s, [&] { return lf::launch_band(p, dt, s); });
    if (st != LF_OK || p.n_g == 0) return st;
    return launch_stage(h, LF_STAGE_MERGE, s, [&] { return lf::launch_merge(p, dt, s); });
}

// Every backward entry point.  qg .. dvg are all null (one projection for every row) or
// all non-null (separate projections of the global rows and their gradients).
lf_status backward_impl(lf_attn_t h, const void* q, const void* k, const void* v, const void* qg, const void* kg,
                        const void* vg, const void* out, const void* dout, const float* lse, void* dq, void* dk,
                        void* dv, void* dqg, void* dkg, void* dvg, int B, int H, int L, int d_h, int w,
                        const int32_t* dil_per_head, const int32_t* global_idx, int n_global,
                        const uint8_t* key_pad_mask, void* stream, float* dbias = nullptr,
                        bool want_dbias = false) {
    if (!h) return LF_ERR_INVALID_ARG;
    h->last_error.clear();
    if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv)
        return fail(h, LF_ERR_INVALID_ARG, "q, k, v, out, dout, lse, dq, dk and dv must be non-null");
    const bool sep = qg || kg || vg || dqg || dkg || dvg;
    if (sep && !(qg && kg && vg && dqg && dkg && dvg))
        return fail(h, LF_ERR_INVALID_ARG, "q_g, k_g, v_g, dq_g, dk_g and dv_g must all be non-null");
    if (want_dbias && !dbias) return fail(h, LF_ERR_INVALID_ARG, "dbias must be non-null");
    if (want_dbias && !h->bias)
        return fail(h, LF_ERR_INVALID_ARG, "no position bias table is set on the handle (its gradient was asked for)");
    if (want_dbias && (reinterpret_cast<uintptr_t>(dbias) & 3u) != 0)
        return fail(h, LF_ERR_INVALID_ARG, "dbias must be 4-byte aligned");
    Plan pl;
    lf_status st = make_plan(h, pl, B, H, L, d_h, w, dil_per_head, global_idx, n_global);
    if (st != LF_OK) return st;
    const void* ins[] = {q, k, v, out, dout, qg, kg, vg};
    void* outs[] = {dq, dk, dv, dqg, dkg, dvg};
    const int n_ins = sep ? 8 : 5, n_outs = sep ? 6 : 3;
    for (int i = 0; i < n_ins; ++i)
        if (!aligned16(ins[i]))
            return fail(h, LF_ERR_INVALID_ARG, "q, k, v, out, dout (and q_g, k_g, v_g) must be 16-byte aligned");
    for (int i = 0; i < n_outs; ++i)
        if (!aligned16(outs[i]))
            return fail(h, LF_ERR_INVALID_ARG, "dq, dk, dv (and dq_g, dk_g, dv_g) must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return fail(h, LF_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    const size_t bytes = pl.bytes;
    const size_t lb = static_cast<size_t>(B) * H * L * sizeof(float);
    for (int i = 0; i < n_outs; ++i) {
        for (int j = 0; j < n_ins; ++j)
            if (overlaps(outs[i], ins[j], bytes)) return fail(h, LF_ERR_INVALID_ARG, "the gradients must not overlap the inputs");
        if (overlaps2(outs[i], bytes, lse, lb))
            return fail(h, LF_ERR_INVALID_ARG, "the gradients must not overlap the inputs");
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], outs[j], bytes)) return fail(h, LF_ERR_INVALID_ARG, "the gradients must not overlap");
    }
    if (want_dbias) {
        const size_t db = static_cast<size_t>(H) * (2 * w + 1) * sizeof(float);
        for (int i = 0; i < n_outs; ++i)
            if (overlaps2(dbias, db, outs[i], bytes)) return fail(h, LF_ERR_INVALID_ARG, "dbias must not overlap the gradients");
        for (int j = 0; j < n_ins; ++j)
            if (overlaps2(dbias, db, ins[j], bytes)) return fail(h, LF_ERR_INVALID_ARG, "dbias must not overlap the inputs");
        if (overlaps2(dbias, db, lse, lb) || overlaps2(dbias, db, h->bias, db))
            return fail(h, LF_ERR_INVALID_ARG, "dbias must not overlap lse or the bias table");
    }

    lf::BwdParams p;
    std::memset(&p, 0, sizeof(p));
    std::copy(pl.dil, pl.dil + H, p.dil);
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = out;
    p.dout = dout;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.sep = sep ? 1 : 0;
    p.qg = qg;
    p.kg = kg;
    p.vg = vg;
    p.dqg = dqg;
    p.dkg = dkg;
    p.dvg = dvg;
    p.pad = key_pad_mask;
    p.lse = lse;
    p.B = B;
    p.H = H;
    p.L = L;
    p.w = pl.w;
    p.n_g = pl.n_g;
    p.gstride = pl.gstride;
    std::copy(pl.g.begin(), pl.g.end(), p.g);
    std::copy(pl.gcnt.begin(), pl.gcnt.end(), p.gcnt);
    p.n_gblk = pl.n_gblk;
    p.tiles_per_head = pl.tiles;
    p.causal = h->window_mode == LF_WINDOW_CAUSAL;
    p.bias = h->bias;
    p.bias_w = h->bias_w;
    p.dtype = h->dtype;
    p.dil_u = uniform_dilation(pl.dil, H);

    // Workspace: three row-statistic arrays, then the global partials.
    if (hipGetDevice(&h->device) != hipSuccess) return fail(h, LF_ERR_HIP, "hipGetDevice failed");
    st = upload_random(h);
    if (st != LF_OK) return st;
    if (h->rnd_on) {
        p.rnd = reinterpret_cast<const int*>(h->rnd_dev);
        p.rnd_nq = h->rnd_nq;
        p.rnd_r = h->rnd_r;
        p.rnd_inv = p.rnd + h->rnd_tab.size();
        p.rnd_inv_r = h->rnd_inv_r;
    }
    const size_t rows = static_cast<size_t>(B) * H * L;
    const size_t ngq = static_cast<size_t>(p.n_gblk) * lf::kGlobalQueriesPerBlock;
    const size_t n_part = static_cast<size_t>(B) * H * pl.tiles * ngq * 64;
    const size_t n_own = static_cast<size_t>(B) * H * ngq * 64;
    const size_t rows_al = (rows + 63) & ~size_t(63);
    const size_t n_db = want_dbias ? static_cast<size_t>(B) * H * pl.tiles * (2 * pl.w + 1) : 0;
    st = reserve(h, &h->ws_bwd, &h->ws_bwd_bytes, &h->ws_bwd_device,
                 (3 * rows_al + 3 * n_part + 2 * n_own + n_db) * sizeof(float));
    if (st != LF_OK) return st;
    float* f = reinterpret_cast<float*>(h->ws_bwd);
    p.lse2 = f;
    p.lse2_band = f + rows_al;
    p.dsum = f + 2 * rows_al;
    f += 3 * rows_al;
    p.ws_dq = f;
    p.ws_dk = f + n_part;
    p.ws_dv = f + 2 * n_part;
    p.ws_dkg = f + 3 * n_part;
    p.ws_dvg = f + 3 * n_part + n_own;
    if (want_dbias) {
        p.ws_db = f + 3 * n_part + 2 * n_own;
        p.dbias = dbias;
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    st = launch_stage(h, LF_STAGE_BWD_PREP, s, [&] { return lf::launch_bwd_prep(p, s); });
    if (st == LF_OK) st = launch_stage(h, LF_STAGE_BWD_DQ, s, [&] { return lf::launch_bwd_dq(p, s); });
    if (st == LF_OK) st = launch_stage(h, LF_STAGE_BWD_DKV, s, [&] { return lf::launch_bwd_dkv(p, s); });
    if (st == LF_OK && sep)
        st = launch_stage(h, LF_STAGE_BWD_DKV_GLOBAL, s, [&] { return lf::launch_bwd_dkv_global_proj(p, s); });
    if (st == LF_OK && p.n_g > 0)
        st = launch_stage(h, LF_STAGE_BWD_MERGE, s, [&] { return lf::launch_bwd_merge(p, s); });
    if (st == LF_OK && want_dbias)
        st = launch_stage(h, LF_STAGE_BWD_DBIAS, s, [&] { return lf::launch_bwd_dbias(p, s); });
    return st;
}

constexpr size_t kGemmWorkspace = size_t(32) << 20;

// The descriptors and algorithm of Y[M][N] = X[M][K] W^T (see gemm_xwt), made once
// per shape and output type on the handle's current device.
lf_status gemm_plan(lf_attn_t h, int M, int N, int K, bool f32_out, bool bias, const GemmPlan** out) {
    for (const GemmPlan& g : h->gemm_plans)
        if (g.M == M && g.N == N && g.K == K && g.f32_out == f32_out && g.bias == bias) {
            *out = &g;
            return LF_OK;
        }
    GemmPlan g;
    g.M = M;
    g.N = N;
    g.K = K;
    g.f32_out = f32_out;
    g.bias = bias;
    const hipblasLtEpilogue_t epi = bias ? HIPBLASLT_EPILOGUE_BIAS : HIPBLASLT_EPILOGUE_DEFAULT;
    const hipDataType bias_t = HIP_R_16BF;
    const hipDataType yt = f32_out ? HIP_R_32F : HIP_R_16BF;
    const hipblasOperation_t opt = HIPBLAS_OP_T, opn = HIPBLAS_OP_N;
    hipblasLtMatmulPreference_t pref = nullptr;
    const uint64_t ws = kGemmWorkspace;
    hipblasLtMatmulHeuristicResult_t res[1];
    int n_res = 0;
    bool ok = hipblasLtMatmulDescCreate(&g.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opt, sizeof(opt)) ==
                  HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opn, sizeof(opn)) ==
                  HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi)) ==
                  HIPBLAS_STATUS_SUCCESS &&
              (!bias || hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bias_t,
                                                        sizeof(bias_t)) == HIPBLAS_STATUS_SUCCESS) &&
              hipblasLtMatrixLayoutCreate(&g.a, HIP_R_16BF, K, N, K) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&g.b, HIP_R_16BF, K, M, K) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&g.c, yt, N, M, N) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws,
                                                    sizeof(ws)) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulAlgoGetHeuristic(h->lt, g.desc, g.a, g.b, g.c, g.c, pref, 1, res, &n_res) ==
                  HIPBLAS_STATUS_SUCCESS &&
              n_res >= 1 && res[0].state == HIPBLAS_STATUS_SUCCESS && res[0].workspaceSize <= kGemmWorkspace;
    if (pref) (void)hipblasLtMatmulPreferenceDestroy(pref);
    if (!ok) {
        if (g.c) (void)hipblasLtMatrixLayoutDestroy(g.c);
        if (g.b) (void)hipblasLtMatrixLayoutDestroy(g.b);
        if (g.a) (void)hipblasLtMatrixLayoutDestroy(g.a);
        if (g.desc) (void)hipblasLtMatmulDescDestroy(g.desc);
        return fail(h, LF_ERR_HIP, "hipBLASLt has no algorithm for the %d x %d x %d GEMM", M, N, K);
    }
    g.algo = res[0].algo;
    g.ws = res[0].workspaceSize;
    h->gemm_plans.push_back(g);
    *out = &h->gemm_plans.back();
    return LF_OK;
}

// Y[M][N] (row-major; bf16, or fp32 when f32_out) = X[M][K] (bf16) W^T with W[N][K]
// (bf16), fp32 accumulation: in hipBLASLt's column-major terms Y^T = W X^T, i.e.
// op(A) = A^T with A = W^T stored K x N, and B = X^T stored K x M.
lf_status gemm_xwt(lf_attn_t h, const void* X, const void* Wt, void* Y, int M, int N, int K, bool f32_out,
                   hipStream_t s, const void* bias = nullptr) {
    const GemmPlan* g = nullptr;
    lf_status st = gemm_plan(h, M, N, K, f32_out, bias != nullptr, &g);
    if (st != LF_OK) return st;
    if (bias && hipblasLtMatmulDescSetAttribute(g->desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof(bias)) !=
                    HIPBLAS_STATUS_SUCCESS)
        return fail(h, LF_ERR_HIP, "setting the GEMM bias pointer failed");
    const float one = 1.f, zero = 0.f;
    const hipblasStatus_t rs = hipblasLtMatmul(h->lt, g->desc, &one, Wt, g->a, X, g->b, &zero, Y, g->c, Y, g->c,
                                               &g->algo, h->ws_gemm, g->ws, s);
    if (rs != HIPBLAS_STATUS_SUCCESS) return fail(h, LF_ERR_HIP, "hipblasLtMatmul failed (status %d)", (int)rs);
    return LF_OK;
}

lf_status layer_impl(lf_attn_t h, const void* x, const lf_layer_weights* wt, void* out, int B, int L, int E, int F,
                     float eps, int w, const int32_t* dil_per_head, const int32_t* global_idx, int n_global,
                     const uint8_t* key_pad_mask, void* stream) {
    if (!h) return LF_ERR_INVALID_ARG;
    h->last_error.clear();
    if (!x || !wt || !out) return fail(h, LF_ERR_INVALID_ARG, "x, wts and out must be non-null");
    if (h->dtype != LF_BF16) return fail(h, LF_ERR_UNSUPPORTED, "the layer supports bf16 handles only");
    if (B < 1 || L < 1) return fail(h, LF_ERR_INVALID_ARG, "need B, L >= 1 (got %d, %d)", B, L);
    if (E < LF_HEAD_DIM || E % LF_HEAD_DIM != 0 || E / LF_HEAD_DIM > LF_MAX_HEADS || E > 2048)
        return fail(h, LF_ERR_UNSUPPORTED, "hidden must be a multiple of 64, at most 2048 (got %d)", E);
    if (F < 8 || F % 8 != 0) return fail(h, LF_ERR_UNSUPPORTED, "ffn must be a positive multiple of 8 (got %d)", F);
    if (!(eps >= 0.f)) return fail(h, LF_ERR_INVALID_ARG, "ln_eps must be >= 0");
    const void* ptrs[] = {wt->w_qkv, wt->b_qkv, wt->w_o, wt->b_o, wt->ln1_g, wt->ln1_b,
                          wt->w_1,   wt->b_1,   wt->w_2, wt->b_2, wt->ln2_g, wt->ln2_b};
    for (const void* q : ptrs)
        if (!q || !aligned16(q)) return fail(h, LF_ERR_INVALID_ARG, "every weight pointer must be non-null and 16-byte aligned");
    if (!aligned16(x) || !aligned16(out)) return fail(h, LF_ERR_INVALID_ARG, "x and out must be 16-byte aligned");
    const int H = E / LF_HEAD_DIM;
    const size_t R = static_cast<size_t>(B) * L;
    if (R * static_cast<size_t>(std::max(3 * E, F)) > (size_t(1) << 40))
        return fail(h, LF_ERR_INVALID_ARG, "tensor size overflows");
    if (R > 0x7fffffff) return fail(h, LF_ERR_UNSUPPORTED, "too many tokens");
    if (overlaps(out, x, R * E * 2)) return fail(h, LF_ERR_INVALID_ARG, "out must not overlap x");
    Plan pl;  // validates the attention arguments before anything is enqueued
    lf_status st = make_plan(h, pl, B, H, L, LF_HEAD_DIM, w, dil_per_head, global_idx, n_global);
    if (st != LF_OK) return st;

    if (hipGetDevice(&h->device) != hipSuccess) return fail(h, LF_ERR_HIP, "hipGetDevice failed");
    if (h->lt && h->lt_device != h->device && release_gemm(h) != LF_OK)
        return fail(h, LF_ERR_HIP, "releasing the GEMM handle of another device failed");
    if (!h->lt) {
        if (hipblasLtCreate(&h->lt) != HIPBLAS_STATUS_SUCCESS) {
            h->lt = nullptr;
            return fail(h, LF_ERR_HIP, "hipblasLtCreate failed");
        }
        h->lt_device = h->device;
    }
    st = reserve(h, &h->ws_gemm, &h->ws_gemm_bytes, &h->ws_gemm_device, kGemmWorkspace);
    if (st != LF_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);

    // Workspace: one GEMM output ([R][3E] or [R][F] in bf16, or [R][E] in fp32), the
    // attention output in merged-heads layout [R][E] (reused for x1), and the
    // feed-forward activations [R][F], bf16.
    const size_t g_row = std::max<size_t>(std::max(3 * E, F) * size_t(2), E * size_t(4));
    const size_t t_elems = R * static_cast<size_t>(E);
    const size_t g_bytes = (R * g_row + 255) & ~size_t(255);
    const size_t need = g_bytes + (t_elems + R * F) * 2 + 256;
    st = reserve(h, &h->ws_layer, &h->ws_layer_bytes, &h->ws_layer_device, need);
    if (st != LF_OK) return st;
    void* gout = h->ws_layer;
    uint16_t* bm = reinterpret_cast<uint16_t*>(h->ws_layer + g_bytes);  // attention output [R][E], then x1
    uint16_t* bh = bm + t_elems;                                         // GELU activations [R][F]
    const int M = static_cast<int>(R);

    // QKV projection with its bias added in the GEMM epilogue: row t of gout holds
    // q, k, v of token t, head h at features 64h (+E, +2E).  The attention reads them
    // there and writes its output with the heads merged, ready for the output
    // projection: no split or merge passes.
    st = launch_stage(h, LF_STAGE_LAYER_GEMM, s, [&] {
        return gemm_xwt(h, x, wt->w_qkv, gout, M, 3 * E, E, false, s, wt->b_qkv) == LF_OK ? hipSuccess
                                                                                         : hipErrorUnknown;
    });
    if (st != LF_OK) return st;
    {
        const uint16_t* g16 = static_cast<const uint16_t*>(gout);
        Strides sd;
        sd.s_b = 3LL * L * E;
        sd.s_h = LF_HEAD_DIM;
        sd.s_r = 3 * E;
        sd.o_b = static_cast<long long>(L) * E;
        sd.o_h = LF_HEAD_DIM;
        sd.o_r = E;
        st = forward_impl(h, g16, g16 + E, g16 + 2 * E, nullptr, nullptr, nullptr, bm, nullptr, B, H, L, LF_HEAD_DIM,
                          w, dil_per_head, global_idx, n_global, key_pad_mask, stream, false, &sd);
    }
    if (st != LF_OK) return st;
    st = launch_stage(h, LF_STAGE_LAYER_GEMM, s, [&] {
        return gemm_xwt(h, bm, wt->w_o, gout, M, E, E, true, s) == LF_OK ? hipSuccess : hipErrorUnknown;
    });
    if (st != LF_OK) return st;
    st = launch_stage(h, LF_STAGE_LAYER_POINTWISE, s, [&] {
        return lf::launch_bias_residual_ln(static_cast<const float*>(gout), wt->b_o, x, wt->ln1_g, wt->ln1_b, eps, bm, E,
                                           (long long)R, s);
    });
    if (st != LF_OK) return st;
    st = launch_stage(h, LF_STAGE_LAYER_GEMM, s, [&] {
        return gemm_xwt(h, bm, wt->w_1, gout, M, F, E, false, s) == LF_OK ? hipSuccess : hipErrorUnknown;
    });
    if (st != LF_OK) return st;
    st = launch_stage(h, LF_STAGE_LAYER_POINTWISE, s,
                      [&] { return lf::launch_bias_gelu(gout, wt->b_1, bh, F, (long long)R, s); });
    if (st != LF_OK) return st;
    st = launch_stage(h, LF_STAGE_LAYER_GEMM, s, [&] {
        return gemm_xwt(h, bh, wt->w_2, gout, M, E, F, true, s) == LF_OK ? hipSuccess : hipErrorUnknown;
    });
    if (st != LF_OK) return st;
    return launch_stage(h, LF_STAGE_LAYER_POINTWISE, s, [&] {
        return lf::launch_bias_residual_ln(static_cast<const float*>(gout), wt->b_2, bm, wt->ln2_g, wt->ln2_b, eps, out, E,
                                           (long long)R, s);
    });
}

}  // namespace

extern "C" {

lf_status lf_attn_forward(lf_attn_t h, const void* q, const void* k, const void* v, void* out, int B, int H,
                          int L, int d_h, int w, const int32_t* dil_per_head, const int32_t* global_idx,
                          int n_global, const uint8_t* key_pad_mask, void* stream) {
    return forward_impl(h, q, k, v, nullptr, nullptr, nullptr, out, nullptr, B, H, L, d_h, w, dil_per_head,
                        global_idx, n_global, key_pad_mask, stream);
}

lf_status lf_attn_forward_static(lf_attn_t h, const void* q, const void* k, const void* v, void* out, int B,
                                 int H, int L, int d_h, int w, const int32_t* dil_per_head, const int32_t* global_idx,
                                 int n_global, const uint8_t* key_pad_mask, void* stream) {
    return forward_impl(h, q, k, v, nullptr, nullptr, nullptr, out, nullptr, B, H, L, d_h, w, dil_per_head,
                        global_idx, n_global, key_pad_mask, stream, true);
}

lf_status lf_attn_forward_lse(lf_attn_t h, const void* q, const void* k, const void* v, void* out, float* lse,
                              int B, int H, int L, int d_h, int w, const int32_t* dil_per_head,
                              const int32_t* global_idx, int n_global, const uint8_t* key_pad_mask, void* stream) {
    if (h && !lse) {
        h->last_error = "lse must be non-null";
        return LF_ERR_INVALID_ARG;
    }
    return forward_impl(h, q, k, v, nullptr, nullptr, nullptr, out, lse, B, H, L, d_h, w, dil_per_head, global_idx,
                        n_global, key_pad_mask, stream);
}

lf_status lf_attn_forward_global_proj(lf_attn_t h, const void* q, const void* k, const void* v, const void* q_g,
                                      const void* k_g, const void* v_g, void* out, int B, int H, int L, int d_h,
                                      int w, const int32_t* dil_per_head, const int32_t* global_idx, int n_global,
                                      const uint8_t* key_pad_mask, void* stream) {
    if (h && (!q_g || !k_g || !v_g)) {
        h->last_error = "q_g, k_g and v_g must be non-null";
        return LF_ERR_INVALID_ARG;
    }
    return forward_impl(h, q, k, v, q_g, k_g, v_g, out, nullptr, B, H, L, d_h, w, dil_per_head, global_idx,
                        n_global, key_pad_mask, stream);
}

lf_status lf_attn_forward_global_proj_lse(lf_attn_t h, const void* q, const void* k, const void* v,
                                          const void* q_g, const void* k_g, const void* v_g, void* out, float* lse,
                                          int B, int H, int L, int d_h, int w, const int32_t* dil_per_head,
                                          const int32_t* global_idx, int n_global, const uint8_t* key_pad_mask,
                                          void* stream) {
    if (h && (!q_g || !k_g || !v_g || !lse)) {
        h->last_error = "q_g, k_g, v_g and lse must be non-null";
        return LF_ERR_INVALID_ARG;
    }
    return forward_impl(h, q, k, v, q_g, k_g, v_g, out, lse, B, H, L, d_h, w, dil_per_head, global_idx,
                        n_global, key_pad_mask, stream);
}

lf_status lf_attn_backward(lf_attn_t h, const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv, int B, int H, int L,
                           int d_h, int w, const int32_t* dil_per_head, const int32_t* global_idx, int n_global,
                           const uint8_t* key_pad_mask, void* stream) {
    return backward_impl(h, q, k, v, nullptr, nullptr, nullptr, out, dout, lse, dq, dk, dv, nullptr, nullptr, nullptr,
                         B, H, L, d_h, w, dil_per_head, global_idx, n_global, key_pad_mask, stream);
}

lf_status lf_attn_backward_bias(lf_attn_t h, const void* q, const void* k, const void* v, const void* out,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv, float* dbias, int B,
                                int H, int L, int d_h, int w, const int32_t* dil_per_head, const int32_t* global_idx,
                                int n_global, const uint8_t* key_pad_mask, void* stream) {
    return backward_impl(h, q, k, v, nullptr, nullptr, nullptr, out, dout, lse, dq, dk, dv, nullptr, nullptr, nullptr,
                         B, H, L, d_h, w, dil_per_head, global_idx, n_global, key_pad_mask, stream, dbias, true);
}

lf_status lf_attn_backward_global_proj(lf_attn_t h, const void* q, const void* k, const void* v, const void* q_g,
                                       const void* k_g, const void* v_g, const void* out, const void* dout,
                                       const float* lse, void* dq, void* dk, void* dv, void* dq_g, void* dk_g,
                                       void* dv_g, int B, int H, int L, int d_h, int w,
                                       const int32_t* dil_per_head, const int32_t* global_idx, int n_global,
                                       const uint8_t* key_pad_mask, void* stream) {
    return backward_impl(h, q, k, v, q_g, k_g, v_g, out, dout, lse, dq, dk, dv, dq_g, dk_g, dv_g, B, H, L, d_h, w,
                         dil_per_head, global_idx, n_global, key_pad_mask, stream);
}

lf_status lf_layer_forward(lf_attn_t h, const void* x, const lf_layer_weights* wts, void* out, int B, int L,
                           int hidden, int ffn, float ln_eps, int w, const int32_t* dil_per_head,
                           const int32_t* global_idx, int n_global, const uint8_t* key_pad_mask, void* stream) {
    return layer_impl(h, x, wts, out, B, L, hidden, ffn, ln_eps, w, dil_per_head, global_idx, n_global,
                      key_pad_mask, stream);
}

}  // extern "C"
