// Bandwidth-bound kernels of the replicated layer parts: LayerNorm forward/backward, the
// on-device sum of rank partials (+ bias + residual), and column sums. Every reduction has a
// fixed order (wave butterflies, then block partials reduced in block order): no atomics.
#pragma once
#include "common.h"

namespace tp {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// ---------------------------------------------------------------------------------------------
// LayerNorm forward: one wave per row, the row held in registers (C chunks of 8 per lane).
// ---------------------------------------------------------------------------------------------
template <typename T, int C>
__global__ __launch_bounds__(256) void ln_fwd_kernel(int rows, int h, float eps, const T* __restrict__ x,
                                                     const T* __restrict__ gamma, const T* __restrict__ beta,
                                                     T* __restrict__ y, float* __restrict__ mean,
                                                     float* __restrict__ rstd) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const T* xr = x + (size_t)row * h;
    float v[C][8];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < C; ++k) {
        int c = (lane + 64 * k) * 8;
        if (c < h) {
            load8(xr + c, v[k]);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += v[k][e];
        }
    }
    const float mu = wave_sum(s) / (float)h;
    float q = 0.f;
#pragma unroll
    for (int k = 0; k < C; ++k) {
        int c = (lane + 64 * k) * 8;
        if (c < h) {
#pragma unroll
            for (int e = 0; e < 8; ++e) { float d = v[k][e] - mu; q += d * d; }
        }
    }
    const float rs = rsqrtf(wave_sum(q) / (float)h + eps);
#pragma unroll
    for (int k = 0; k < C; ++k) {
        int c = (lane + 64 * k) * 8;
        if (c < h) {
            float g[8], b[8], o[8];
            load8(gamma + c, g);
            load8(beta + c, b);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = (v[k][e] - mu) * rs * g[e] + b[e];
            store8(y + (size_t)row * h + c, o);
        }
    }
    if (lane == 0) {
        if (mean) mean[row] = mu;
        if (rstd) rstd[row] = rs;
    }
}

// ---------------------------------------------------------------------------------------------
// LayerNorm backward. Block b handles rows b*4 + w + k*(4*nblocks) (wave w). dx is written per
// row; dgamma/dbeta partials are accumulated per lane, merged over the block's waves in wave
// order through LDS, and written as one row per block into part[b][h] (reduced afterwards).
// The row's x and dy stay in registers in their storage type (packed bf16) between the two passes.
// ---------------------------------------------------------------------------------------------
template <typename T> struct Raw8;
template <> struct Raw8<bf16> {
    u32x4 v;
    __device__ __forceinline__ void load(const bf16* p) { v = *(const u32x4*)p; }
    __device__ __forceinline__ float operator[](int e) const {
        uint32_t w = v[e >> 1];
        return __builtin_bit_cast(float, (e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};
template <> struct Raw8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) { a = *(const f32x4*)p; b = *(const f32x4*)(p + 4); }
    __device__ __forceinline__ float operator[](int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

template <typename T, int C>
__global__ __launch_bounds__(256) void ln_bwd_kernel(int rows, int h, const T* __restrict__ x,
                                                     const T* __restrict__ gamma, const float* __restrict__ mean,
                                                     const float* __restrict__ rstd, const T* __restrict__ dy,
                                                     const T* __restrict__ dres, T* __restrict__ dx,
                                                     float* __restrict__ part_g, float* __restrict__ part_b) {
    extern __shared__ float lds[];   // [2][h]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float pg[C][8], pb[C][8];
#pragma unroll
    for (int k = 0; k < C; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) { pg[k][e] = 0.f; pb[k][e] = 0.f; }
    const float inv_h = 1.0f / (float)h;
    for (int row = blockIdx.x * 4 + wave; row < rows; row += 4 * gridDim.x) {
        const float mu = mean[row], rs = rstd[row];
        Raw8<T> xr[C], dr[C];
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int k = 0; k < C; ++k) {
            int c = (lane + 64 * k) * 8;
            if (c < h) {
                xr[k].load(x + (size_t)row * h + c);
                dr[k].load(dy + (size_t)row * h + c);
                float gm[8];
                load8(gamma + c, gm);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float xh = (xr[k][e] - mu) * rs, d = dr[k][e];
                    float g = d * gm[e];
                    s1 += g;
                    s2 += g * xh;
                    pg[k][e] += d * xh;
                    pb[k][e] += d;
                }
            }
        }
        s1 = wave_sum(s1) * inv_h;
        s2 = wave_sum(s2) * inv_h;
#pragma unroll
        for (int k = 0; k < C; ++k) {
            int c = (lane + 64 * k) * 8;
            if (c < h) {
                float o[8], rr[8], gm[8];
                load8(gamma + c, gm);
                if (dres) load8(dres + (size_t)row * h + c, rr);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float xh = (xr[k][e] - mu) * rs;
                    o[e] = rs * (dr[k][e] * gm[e] - s1 - xh * s2);
                    if (dres) o[e] += rr[e];
                }
                store8(dx + (size_t)row * h + c, o);
            }
        }
    }
    if (!part_g) return;   // uniform across the block
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
#pragma unroll
            for (int k = 0; k < C; ++k) {
                int c = (lane + 64 * k) * 8;
                if (c < h) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (w == 0) { lds[c + e] = pg[k][e]; lds[h + c + e] = pb[k][e]; }
                        else { lds[c + e] += pg[k][e]; lds[h + c + e] += pb[k][e]; }
                    }
                }
            }
        }
        __syncthreads();
    }
    for (int c = threadIdx.x; c < h; c += 256) {
        part_g[(size_t)blockIdx.x * h + c] = lds[c];
        part_b[(size_t)blockIdx.x * h + c] = lds[h + c];
    }
}

// out[c] (+)= sum_{b=0}^{nb-1} part[b][c]. Block = 64 columns x 4 row phases: phase p sums rows
// p, p+4, ... in order, then the four phase sums are added in phase order.
template <typename T>
__global__ __launch_bounds__(256) void reduce_rows_kernel(const float* __restrict__ part, int nb, int n,
                                                          T* __restrict__ out, int accumulate) {
    __shared__ float red[4][64];
    const int cl = threadIdx.x & 63, ph = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + cl;
    float a = 0.f;
    if (c < n) {
#pragma unroll 8
        for (int b = ph; b < nb; b += 4) a += part[(size_t)b * n + c];
    }
    red[ph][cl] = a;
    __syncthreads();
    if (ph == 0 && c < n) {
        a = ((red[0][cl] + red[1][cl]) + red[2][cl]) + red[3][cl];
        if (accumulate) a += to_f32(out[c]);
        out[c] = from_f32<T>(a);
    }
}

// ---------------------------------------------------------------------------------------------
// Column sums of G [rows, n]: grid (ceil(n/8/64), RB), 64 threads; a thread owns 8 columns and
// rows y, y + RB, ...; partial row y goes to part[y][n].
// ---------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void colsum_partial_kernel(int rows, int n, const T* __restrict__ G,
                                                            float* __restrict__ part) {
    int c = (blockIdx.x * 64 + threadIdx.x) * 8;
    if (c >= n) return;
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 16
    for (int r = blockIdx.y; r < rows; r += gridDim.y) {
        float v[8];
        load8(G + (size_t)r * n + c, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] += v[e];
    }
    store8(part + (size_t)blockIdx.y * n + c, a);
}

// ---------------------------------------------------------------------------------------------
// out = sum_r parts[r] + bias + residual (fp32 sum in rank order), 8 elements per thread.
// ---------------------------------------------------------------------------------------------
constexpr int SUM_MAX_T = 64;
struct PartPtrs { const void* p[SUM_MAX_T]; };

template <typename TI, typename TO>
__global__ __launch_bounds__(256) void sum_partials_kernel(size_t n_elems, int cols, int t, PartPtrs parts,
                                                           const TO* __restrict__ bias,
                                                           const TO* __restrict__ residual, TO* __restrict__ out) {
    size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= n_elems) return;
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int r = 0; r < t; ++r) {
        float v[8];
        load8((const TI*)parts.p[r] + i, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] += v[e];
    }
    if (bias) {
        float b[8];
        load8(bias + (i % cols), b);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] += b[e];
    }
    if (residual) {
        float rr[8];
        load8(residual + i, rr);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] += rr[e];
    }
    store8(out + i, a);
}

}  // namespace tp
