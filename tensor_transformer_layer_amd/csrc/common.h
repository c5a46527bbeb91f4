// Shared device types and helpers for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }  // RNE

// Two fp32 -> packed bf16x2 (round to nearest even, one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(bf16)lo, (bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// 8 consecutive elements <-> fp32
__device__ __forceinline__ void load8(const bf16* p, float (&o)[8]) {
    bf16x8 v = *(const bf16x8*)p;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (float)v[e];
}
__device__ __forceinline__ void load8(const float* p, float (&o)[8]) {
    f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { o[e] = a[e]; o[e + 4] = b[e]; }
}
__device__ __forceinline__ void store8(bf16* p, const float (&v)[8]) {
    *(u32x4*)p = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7])};
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
    *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// Standard normal CDF Phi(x) = erfc(-x / sqrt 2) / 2, branch-free, through the Chebyshev-fitted
// complementary error function of Press, Teukolsky, Vetterling and Flannery (Numerical Recipes,
// 2nd ed., §6.2): erfc(z) = t exp(-z^2 + P(t)), t = 1 / (1 + z/2), P a degree-9 polynomial, with a
// fractional error below 1.2e-7 for all z >= 0 (1.05e-7 measured against a float64 erfc; in fp32
// the rounding of z^2 adds up to ~1e-5 relative where erfc < 1e-60, i.e. only for |x| > 13).
// Taking the smaller tail for x of either sign keeps Phi's relative accuracy for negative x, where
// GeLU is tiny. About 17 VALU operations (one v_rcp, one v_exp), against the two-branch library erff
// that made the GeLU epilogues VALU-bound.
__device__ __forceinline__ float normal_cdf(float x) {
    const float z = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
    float p = 0.17087277f;
    p = fmaf(p, t, -0.82215223f);
    p = fmaf(p, t, 1.48851587f);
    p = fmaf(p, t, -1.13520398f);
    p = fmaf(p, t, 0.27886807f);
    p = fmaf(p, t, -0.18628806f);
    p = fmaf(p, t, 0.09678418f);
    p = fmaf(p, t, 0.37409196f);
    p = fmaf(p, t, 1.00002368f);
    p = fmaf(p, t, -1.26551223f);
    const float tail = 0.5f * t * __expf(fmaf(-z, z, p));   // erfc(|x| / sqrt 2) / 2
    return x < 0.0f ? tail : 1.0f - tail;
}

// GeLU, erf form: x * Phi(x). Derivative: Phi(x) + x * phi(x).
__device__ __forceinline__ float gelu_f(float x) { return x * normal_cdf(x); }
__device__ __forceinline__ float gelu_grad_f(float x) {
    const float pdf = 0.39894228040143268f * __expf(-0.5f * x * x);
    return fmaf(x, pdf, normal_cdf(x));
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// out[c] (+)= sum_{b=0}^{nb-1} part[b][c] over the 16 columns of column block cb (n % 4 == 0), by a
// block of 256 threads: 4 columns per thread x 64 row phases; phase p sums rows p, p+64, ... in
// order, then the 64 phase sums are added in a fixed pairwise tree. Every thread of the block calls it.
constexpr int RR_COLS = 16;
template <typename T>
__device__ __forceinline__ void rowsum_block(const float* __restrict__ part, T* __restrict__ out, int nb, int n,
                                             int accumulate, int cb) {
    __shared__ f32x4 red[64][4];
    const int cg = threadIdx.x & 3, ph = threadIdx.x >> 2;
    const int c = cb * RR_COLS + cg * 4;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    if (c < n) {
#pragma unroll 8
        for (int b = ph; b < nb; b += 64) a += *(const f32x4*)(part + (size_t)b * n + c);
    }
    red[ph][cg] = a;
    __syncthreads();
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) {
        if (ph < s) red[ph][cg] += red[ph + s][cg];
        __syncthreads();
    }
    if (ph == 0 && c < n) {
        f32x4 r = red[0][cg];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = r[e];
            if (accumulate) v += to_f32(out[c + e]);
            out[c + e] = from_f32<T>(v);
        }
    }
}

// A column-sum job (bf16 output) carried by another kernel's launch as extra blocks.
struct ColSumJob {
    const float* part; void* out; int nb, n, accumulate;
};

}  // namespace tp
