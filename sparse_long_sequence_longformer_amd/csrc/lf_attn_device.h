// Device helpers shared by the forward (lf_attn_kernels.hip) and backward
// (lf_attn_bwd.hip) kernels for gfx950: vector types, the MFMA register layout
// helpers, the LDS swizzles, the global->LDS copy primitives and wait/barrier
// wrappers.  Internal to liblfattn.so.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lf_attn_internal.h"

namespace lf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

#define LF_LDS(T, ptr) ((__attribute__((address_space(3))) T*)(ptr))

// LDS byte address of a generic pointer into LDS.  A flat address in the shared
// aperture is the aperture base (its high 32 bits) plus the LDS address, so the low
// 32 bits are the LDS address itself; the address-space cast would also test for a
// null pointer (a compare and a select per copy on the scalar unit).
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// exp(x / sqrt(64)) = exp2(x * log2(e) / 8)
constexpr float kScaleLog2 = 1.4426950408889634f * 0.125f;
constexpr float kNegInf = -__builtin_inff();
constexpr int kStageKeys = kKeysPerTile;  // 64
constexpr int kNoPos = -(1 << 29);        // virtual position that is in no window
// Relative position bias tables in LDS: windows up to kMaxBiasW keys per side, with
// kBiasPad zeros on both ends (a processed 32-key sub-tile reads at most 94 entries
// beyond the window on either side).
constexpr int kMaxBiasW = LF_MAX_BIAS_W;
constexpr int kBiasPad = 96;
constexpr int kBiasLds = 2 * kMaxBiasW + 1 + 2 * kBiasPad;
constexpr float kLog2eF = 1.4426950408889634f;
constexpr int kLargeW = 1 << 28;  // band test that admits every key (|key - query| < 2^28)

// Source of every invalid key: 256 zero bytes (one fp32 row, two bf16 rows).
__device__ __attribute__((aligned(16))) uint32_t g_zero_row[64];

__device__ __forceinline__ int sigma(int M) {  // K row read by lane row M
    const int q = M >> 3, hh = (M >> 2) & 1, c = M & 3;
    return 16 * (q >> 1) + 8 * hh + 4 * (q & 1) + c;
}
__device__ __forceinline__ int key_local(int i, int h2) { return 16 * (i >> 3) + 8 * h2 + (i & 7); }

// LDS swizzles of 16-byte chunks.  K: every 8 consecutive lanes of the 128-bit
// operand reads (rows sigma(0..7) + c) hit 8 distinct chunks.  V: the four rows of
// each 16-lane transposed read land on four distinct 32-byte slots.
__device__ __forceinline__ int swz_k(int row) { return (row & 3) | ((row >> 1) & 4); }
__device__ __forceinline__ int swz_v(int row) { return 2 * (row & 3); }

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
__device__ __forceinline__ uint64_t ballot64(bool x) { return __ballot(x); }

// 16 bytes per lane from global memory into LDS at base + 16 * lane (base uniform).
// Issued as inline asm: the compiler then does not treat the in-flight copies as
// possibly aliasing later LDS reads (it would drain every copy with vmcnt(0) before
// each transposed read).  Completion is awaited explicitly with wait_vmcnt before
// the barrier that publishes a stage.  The instruction has no register results.
// M0 carries the LDS base; no other code in these kernels keeps a value in M0.
__device__ __forceinline__ void dma16(const void* src, char* lds_base) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(lds_base));
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(base) : "memory", "m0");
}

// Wave-uniform copy of a 64-bit value in scalar registers.  The builtin returns a
// signed int: both halves go through uint32_t so that the low half is not sign-extended.
__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
    return ((uint64_t)hi << 32) | (uint64_t)lo;
}

// 16 bytes per lane from base + off (base uniform, off a per-lane 32-bit byte offset)
// into LDS at lds_base + 16 * lane: the scalar-base form needs no per-lane 64-bit
// address arithmetic.
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, char* lds_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds_base));
    const uint64_t b64 = (uint64_t)(uintptr_t)base;
    const uint64_t sb = uniform64(b64);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sb), "s"(m0)
                 : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Work-group barrier once this wave's LDS accesses (and scalar loads) are done, its
// vector-memory loads still in flight: __syncthreads would also wait for every load
// this wave has issued (the Q rows and stage copies of a kernel's set-up).  The
// values an LDS write stores are awaited by the compiler before that write.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));  // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Work-group barrier without a memory fence: ordering of the staged LDS data is
// established by the explicit vmcnt waits; the empty asm keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void barrier_nofence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

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

// Element i of a 32-key score tile holds stage key 32*sub + kc(i) + 8*h2.
__device__ __forceinline__ constexpr int kc_of(int i) { return 16 * (i >> 3) + (i & 7); }

// Masks of a 32-key score tile.  MODE 0: none; 1: band, keep 0 <= base + kc <= span
// with base = (first key of the sub-tile) + 8*h2 - query + (left extent of the
// window); 2: global keys, masked where in the window (gp: in-window positions of the
// sub-tile's keys, test 0 <= gp + wq <= span) and from slot kc = climit on (global
// slots are sorted by position, so in the one-sided variant the keys after the query
// are a suffix); 3 (kRand only): random-block keys, the complement of mode 1's window
// range, and from kc = climit on.  Invalid keys (inv32 bits) are masked in modes 1-3.
template <bool kRand = false>
__device__ __forceinline__ void mask_scores(f32x16& s, int mode, uint32_t inv32, int h2, int base, int span,
                                            const int* gp, int wq, int climit = 1 << 30) {
    if (mode == 0) return;
    const uint32_t invl = inv32 >> (8 * h2);
    if (kRand && mode == 3) {
        // Random-block keys (contiguous, as in mode 1): keep those OUTSIDE the window
        // range 0 <= base + kc <= span (the band has them), minus invalid keys, and in
        // the one-sided variant only kc < climit (keys at or before the query).
        const int lo_k = max(0, -base), hi_k = min(31, span - base);
        uint32_t win = 0u;
        if (hi_k >= lo_k) win = (hi_k >= 31 ? ~0u : ((2u << hi_k) - 1u)) & ~((1u << lo_k) - 1u);
        uint32_t keep = ~win & ~invl;
        if (climit < 32) keep &= climit <= 0 ? 0u : ((1u << climit) - 1u);
        for (int i = 0; i < 16; ++i)
            if (!((keep >> kc_of(i)) & 1u)) s[i] = kNegInf;
        return;
    }
    if (mode == 1) {
        // Band test 0 <= base + kc <= span as one bit range over kc, minus invalid keys.
        const int lo_k = max(0, -base), hi_k = min(31, span - base);
        uint32_t keep = 0u;
        if (hi_k >= lo_k) keep = (hi_k >= 31 ? ~0u : ((2u << hi_k) - 1u)) & ~((1u << lo_k) - 1u);
        keep &= ~invl;
        for (int i = 0; i < 16; ++i)
            if (!((keep >> kc_of(i)) & 1u)) s[i] = kNegInf;
    } else {
        // The lane's 16 keys are gp[0..7] and gp[16..23]: four 16-byte LDS reads.
        typedef int i32x4 __attribute__((ext_vector_type(4)));
        const i32x4* g4 = reinterpret_cast<const i32x4*>(gp);
        const i32x4 a[4] = {g4[0], g4[1], g4[4], g4[5]};
        for (int i = 0; i < 16; ++i) {
            const int kc = kc_of(i);
            if (((invl >> kc) & 1) || kc >= climit || (unsigned)(a[i >> 2][i & 3] + wq) <= (unsigned)span)
                s[i] = kNegInf;
        }
    }
}

// Whether work-group tile t of a head exists: tile t covers rows [rows*(t - r*tpr), +rows)
// of residue class r = t / tpr (tpr tiles per class, classes 0..dil-1 of a length-L
// sequence).  Every argument is uniform, so this is scalar arithmetic.
__device__ __forceinline__ bool tile_exists(int t, int tpr, int dil, int L, int rows) {
    if (dil == 1) return t * rows < L;  // one class: no division
    const int r = t / tpr;
    return r < dil && (t - r * tpr) * rows < (L - r + dil - 1) / dil;
}

// Dilation of head h: the one every head shares (dil_u != 0, no memory access), else
// the head's own entry.  The empty asm keeps the load inside the branch: the compiler
// would otherwise issue it (and wait for it) unconditionally.
__device__ __forceinline__ int head_dil(int dil_u, const int* dil, int h) {
    int d = dil_u;
    if (d == 0) {
        asm volatile("");
        d = dil[h];
    }
    return d;
}

// Global count of sequence b: n_g for a set shared by every sequence (gstride 0), else
// gcnt[b], read only then (the empty asm keeps the compiler from issuing and awaiting
// that load unconditionally).
__device__ __forceinline__ int seq_globals(int gstride, int n_g, const int* gcnt, int b) {
    int n = n_g;
    if (gstride) {
        asm volatile("");
        n = gcnt[b];
    }
    return n;
}

// Residue class r, class length Lr and first class row r0 of work-group slot t_in of a
// head with dilation dil (tiles of kRows class rows, ceil(ceil(L/dil)/kRows) per
// class); false when the slot holds no tile.  dil == 1 needs no division.
template <int kRows = kRowsPerBlock>
__device__ __forceinline__ bool decode_tile(int t_in, int L, int dil, int& r, int& Lr, int& r0) {
    if (dil == 1) {
        r = 0;
        Lr = L;
        r0 = t_in * kRows;
        return r0 < L;
    }
    const int tpr = ((L + dil - 1) / dil + kRows - 1) / kRows;
    r = t_in / tpr;
    if (r >= dil) return false;
    Lr = (L - r + dil - 1) / dil;
    r0 = (t_in - r * tpr) * kRows;
    return r0 < Lr;
}

// Waves of a merge work-group: enough for one chunk of `chunk` tiles per wave, at most
// `most`.  The launch uses it for the block size and the kernel recomputes it from the
// same arguments (no read of the block size).
__host__ __device__ inline int merge_waves(int tiles, int chunk, int most) {
    const int w = (tiles + chunk - 1) / chunk;
    return w < 1 ? 1 : (w > most ? most : w);
}

// Number of entries of the sorted array pos[0..n) that are <= x (binary search).
__device__ __forceinline__ int count_le(const int* pos, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (pos[mid] <= x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// Launch a kernel on stream s, with the timing events of the launch in progress if
// there are any (see LaunchEvents).
template <class K, class... A>
hipError_t launch_kernel_shm(K kernel, dim3 grid, dim3 block, unsigned shm, hipStream_t s, A... args) {
    LaunchEvents& ev = launch_events();
    if (ev.start) {
        ev.used = true;
        hipExtLaunchKernelGGL(kernel, grid, block, shm, s, ev.start, ev.stop, 0, args...);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, shm, s, args...);
    }
    return hipGetLastError();
}
template <class K, class... A>
hipError_t launch_kernel(K kernel, dim3 grid, dim3 block, hipStream_t s, A... args) {
    return launch_kernel_shm(kernel, grid, block, 0, s, args...);
}

}  // namespace
}  // namespace lf
