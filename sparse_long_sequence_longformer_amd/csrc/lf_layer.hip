// gfx950 kernels of the Longformer layer around the sparse attention (bf16 tensors,
// fp32 arithmetic): the steps between the library GEMMs.  The wide GEMM outputs (the
// QKV projection, its bias added in the GEMM epilogue, and the first feed-forward
// product) arrive in bf16 (fp32 accumulation, rounded once); the two that feed a
// LayerNorm stay fp32.  The attention reads q, k, v from the QKV output in place and
// writes its output with the heads merged.  All passes are HBM-bound elementwise or
// row-wise, written for coalesced 16-byte accesses.
//
//   bias_residual_ln: LayerNorm(y + b + residual) over the features of a row
//   bias_gelu:        GELU(h + b), GELU(t) = 0.5 t (1 + erf(t / sqrt(2))), erf by the
//                     rational approximation of Abramowitz and Stegun, Handbook of
//                     Mathematical Functions, formula 7.1.26 (absolute error 1.5e-7;
//                     about 5e-7 in fp32 arithmetic, far under the bf16 rounding of
//                     the result)
//
// The layer is the post-LayerNorm block of page "基于Block-Sparse Attention的
// Longformer" §6 (attention, residual, LayerNorm, feed-forward, residual,
// LayerNorm) with RoBERTa's projections and feed-forward (page "基于自注意力机制的
// 长文本建模算法：Longformer详解" §6: Longformer starts from RoBERTa's weights).

#include "lf_attn_device.h"

namespace lf {
namespace {

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ f32x8 load8_bf16(const uint16_t* p) {
    return __builtin_convertvector(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p)), f32x8);
}
__device__ __forceinline__ f32x8 load8_f32(const float* p) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void store8_bf16(uint16_t* p, const f32x8& v) {
    *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, __builtin_convertvector(v, bf16x8));
}

__device__ __forceinline__ float wave_sum(float x) {
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

// One wave per row of E = 64 * n features (n <= kMaxPerLane); lane j owns features
// 8*j + 512*c .. +7 for c < n / 8.  Two passes over registers: mean, then variance.
constexpr int kMaxChunks = 4;  // E <= 2048
__global__ __launch_bounds__(256) void bias_residual_ln_kernel(const float* y, const uint16_t* bias,
                                                               const uint16_t* res, const uint16_t* gamma,
                                                               const uint16_t* beta, float eps, uint16_t* out,
                                                               int E, long long R) {
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= R) return;
    const int chunks = E / 512 + ((E % 512) ? 1 : 0);
    f32x8 t[kMaxChunks];
    float s = 0.f;
    for (int c = 0; c < kMaxChunks; ++c) {
        const int f = 512 * c + 8 * lane;
        if (c < chunks && f < E) {
            t[c] = load8_f32(y + row * E + f) + load8_bf16(bias + f) + load8_bf16(res + row * E + f);
            for (int j = 0; j < 8; ++j) s += t[c][j];
        } else {
            t[c] = f32x8{};
        }
    }
    const float mean = wave_sum(s) / (float)E;
    float s2 = 0.f;
    for (int c = 0; c < kMaxChunks; ++c) {
        const int f = 512 * c + 8 * lane;
        if (c < chunks && f < E)
            for (int j = 0; j < 8; ++j) {
                const float dlt = t[c][j] - mean;
                s2 += dlt * dlt;
            }
    }
    const float rstd = 1.0f / __builtin_sqrtf(wave_sum(s2) / (float)E + eps);
    for (int c = 0; c < kMaxChunks; ++c) {
        const int f = 512 * c + 8 * lane;
        if (c < chunks && f < E) {
            const f32x8 g = load8_bf16(gamma + f), be = load8_bf16(beta + f);
            store8_bf16(out + row * E + f, (t[c] - mean) * rstd * g + be);
        }
    }
}

// erf(x) = sign(x) (1 - (a1 k + a2 k^2 + a3 k^3 + a4 k^4 + a5 k^5) exp(-x^2)),
// k = 1 / (1 + p |x|), with the coefficients of formula 7.1.26.
__device__ __forceinline__ float erf_as(float x) {
    const float ax = __builtin_fabsf(x);
    const float k = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
    const float poly =
        ((((1.061405429f * k - 1.453152027f) * k + 1.421413741f) * k - 0.284496736f) * k + 0.254829592f) * k;
    const float e = __builtin_amdgcn_exp2f(-ax * ax * 1.4426950408889634f);
    const float r = 1.0f - poly * e;
    return x < 0.f ? -r : r;
}

// One thread per 8 features of h [R][F].
__global__ __launch_bounds__(256) void bias_gelu_kernel(const uint16_t* hpre, const uint16_t* bias, uint16_t* out,
                                                        int F, long long n8) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const int per_row = F / 8;
    const long long row = i / per_row;
    const int f = (int)(i - row * per_row) * 8;
    f32x8 t = load8_bf16(hpre + row * F + f) + load8_bf16(bias + f);
    for (int j = 0; j < 8; ++j) t[j] = 0.5f * t[j] * (1.0f + erf_as(t[j] * 0.70710678118654752f));
    store8_bf16(out + row * F + f, t);
}

unsigned blocks_for(long long n, int per_block) { return (unsigned)((n + per_block - 1) / per_block); }

}  // namespace

hipError_t launch_bias_residual_ln(const float* y, const void* bias, const void* res, const void* gamma,
                                   const void* beta, float eps, void* out, int E, long long R, hipStream_t s) {
    launch_kernel(bias_residual_ln_kernel, dim3(blocks_for(R, 4)), dim3(256), s, y,
                       static_cast<const uint16_t*>(bias), static_cast<const uint16_t*>(res),
                       static_cast<const uint16_t*>(gamma), static_cast<const uint16_t*>(beta), eps,
                       static_cast<uint16_t*>(out), E, R);
    return hipGetLastError();
}

hipError_t launch_bias_gelu(const void* h, const void* bias, void* out, int F, long long R, hipStream_t s) {
    const long long n8 = R * F / 8;
    launch_kernel(bias_gelu_kernel, dim3(blocks_for(n8, 256)), dim3(256), s, static_cast<const uint16_t*>(h),
                       static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(out), F, n8);
    return hipGetLastError();
}

}  // namespace lf
