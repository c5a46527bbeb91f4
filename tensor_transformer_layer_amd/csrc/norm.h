// Bandwidth-bound kernels of the replicated layer parts: LayerNorm forward/backward, the
// on-device sum of rank partials (+ bias + residual), and column sums. Every reduction has a
// fixed order (wave butterflies, then block partials reduced in block order): no atomics.
#pragma once
#include "common.h"
#include "rng.h"

namespace tp {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

constexpr int LN_MAX_H = 8192;
template <typename T> struct Raw8;
template <> struct Raw8<bf16> {
    u32x4 v;
    __device__ __forceinline__ void load(const bf16* p) { v = *(const u32x4*)p; }
    __device__ __forceinline__ void zero() { v = u32x4{0u, 0u, 0u, 0u}; }
    // the eight values rounded to bf16 (as store8 writes them)
    __device__ __forceinline__ void set(const float (&a)[8]) {
        v = u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7])};
    }
    __device__ __forceinline__ float operator[](int e) const {
        uint32_t w = v[e >> 1];
        return __builtin_bit_cast(float, (e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};
template <> struct Raw8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) { a = *(const f32x4*)p; b = *(const f32x4*)(p + 4); }
    __device__ __forceinline__ void zero() { a = f32x4{0.f, 0.f, 0.f, 0.f}; b = a; }
    __device__ __forceinline__ void set(const float (&x)[8]) {
        a = f32x4{x[0], x[1], x[2], x[3]};
        b = f32x4{x[4], x[5], x[6], x[7]};
    }
    __device__ __forceinline__ float operator[](int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// Sums NV per-thread values over the block: returns the totals in v (every thread).
template <int NV>
__device__ __forceinline__ void block_sum(float (&v)[NV], float (*red)[NV], int lane, int wave, int nw) {
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = wave_sum(v[k]);
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < NV; ++k) red[wave][k] = v[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        float a = red[0][k];
        for (int w = 1; w < nw; ++w) a += red[w][k];
        v[k] = a;
    }
}

// ---------------------------------------------------------------------------------------------
// LayerNorm forward: one wave per row, the row held in registers (C chunks of 8 per lane) in its
// storage type (bf16 rows take half the registers of fp32 copies: more waves resident).
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
    Raw8<T> v[C];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < C; ++k) {
        int c = (lane + 64 * k) * 8;
        if (c < h) v[k].load(xr + c);
        else v[k].zero();
    }
#pragma unroll
    for (int k = 0; k < C; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) s += v[k][e];
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
// Fused partial sum + LayerNorm forward (the consumer of the forward g in a pre-LN block): one
// wave per row; out = sum_r parts[r] + bias + residual (fp32, rank order, rounded to T and
// stored), then y = LayerNorm(out) computed from the rounded values, as a separate LN would see
// them.
// ---------------------------------------------------------------------------------------------
constexpr int ADDLN_MAX_T = 64;
struct AddLnParts { const void* p[ADDLN_MAX_T]; };

template <typename T, int C>
__global__ __launch_bounds__(256) void add_ln_fwd_kernel(int rows, int h, int t, AddLnParts parts,
                                                         const T* __restrict__ bias, const T* __restrict__ residual,
                                                         T* __restrict__ out, float eps, const T* __restrict__ gamma,
                                                         const T* __restrict__ beta, T* __restrict__ y,
                                                         float* __restrict__ mean, float* __restrict__ rstd,
                                                         DropParams drop) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const size_t ro = (size_t)row * h;
    Raw8<T> v[C];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < C; ++k) {
        int c = (lane + 64 * k) * 8;
        if (c < h) {
            float a[8];
            load8((const T*)parts.p[0] + ro + c, a);
            for (int r = 1; r < t; ++r) {
                float b[8];
                load8((const T*)parts.p[r] + ro + c, b);
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] += b[e];
            }
            if (bias) {
                float b[8];
                load8(bias + c, b);
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] += b[e];
            }
            // residual dropout of the summed branch: element (row, c..c+7) is one call
            if (drop.thr) apply_keep8(a, keep8((uint64_t)row * (h >> 3) + (c >> 3), drop), drop.scale);
            if (residual) {
                float b[8];
                load8(residual + ro + c, b);
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] += b[e];
            }
            store8(out + ro + c, a);
            v[k].set(a);   // the stored (rounded) values
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
            store8(y + ro + c, o);
        }
    }
    if (lane == 0) {
        if (mean) mean[row] = mu;
        if (rstd) rstd[row] = rs;
    }
}

// ---------------------------------------------------------------------------------------------
// LayerNorm backward: a group of nt = ceil(h/512)*64 threads spans a row, 8 columns per thread
// (h <= 8192); a block holds G groups (blockDim = G*nt). Each group takes RPI rows per iteration;
// with PF the next iteration's rows (x, dy, dres, mean, rstd) are loaded while the current ones
// are reduced and written, so two iterations are in flight per group. Row sums are wave
// butterflies followed by a sum over the group's waves in wave order through LDS (double-buffered:
// one barrier per iteration). Group g of block b takes rows (b*G + g)*RPI + j + k*(RPI*G*nblocks);
// NTMAX bounds the block size, which sets the register budget. dx is written per row; each thread
// accumulates, for its 8 columns over its group's rows, the column sums wanted (dgamma, dbeta,
// and the plain sums of dres and of dx); the G groups' sums are added in group order through LDS
// and written as row b of part_* [nblocks][h] (NULL: not wanted); they are reduced afterwards.
// ---------------------------------------------------------------------------------------------
template <typename T, int RPI>
struct LnBwdRows {
    Raw8<T> x[RPI], dy[RPI], dr[RPI];
    float mu[RPI], rs[RPI];
    __device__ __forceinline__ void load(int r0, int rows, int h, int c, bool act, const T* __restrict__ xp,
                                         const T* __restrict__ dyp, const T* __restrict__ dresp,
                                         const float* __restrict__ mean, const float* __restrict__ rstd) {
#pragma unroll
        for (int j = 0; j < RPI; ++j) {
            const int row = r0 + j;
            const size_t ro = (size_t)row * h + c;
            if (act && row < rows) {
                x[j].load(xp + ro);
                dy[j].load(dyp + ro);
                if (dresp) dr[j].load(dresp + ro);
                else dr[j].zero();
            } else {
                x[j].zero(); dy[j].zero(); dr[j].zero();
            }
            mu[j] = row < rows ? mean[row] : 0.f;
            rs[j] = row < rows ? rstd[row] : 0.f;
        }
    }
};

template <typename T, int NTMAX, int RPI, int G, bool PF>
__global__ __launch_bounds__(NTMAX) void ln_bwd_kernel(int rows, int h, const T* __restrict__ x,
                                                      const T* __restrict__ gamma, const float* __restrict__ mean,
                                                      const float* __restrict__ rstd, const T* __restrict__ dy,
                                                      const T* __restrict__ dres, T* __restrict__ dx,
                                                      float* __restrict__ part_g, float* __restrict__ part_b,
                                                      float* __restrict__ part_r, float* __restrict__ part_x) {
    __shared__ float red[2][16][2 * RPI];
    const int nt = blockDim.x / G, grp = threadIdx.x / nt, tid = threadIdx.x - grp * nt;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwg = nt >> 6, w0 = grp * nwg;
    const int c = tid * 8;
    const bool act = c < h;
    const float inv_h = 1.0f / (float)h;
    Raw8<T> gm;
    if (act) gm.load(gamma + c);
    else gm.zero();
    float pg[8], pb[8], pr[8], px[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { pg[e] = 0.f; pb[e] = 0.f; pr[e] = 0.f; px[e] = 0.f; }
    auto process = [&](const LnBwdRows<T, RPI>& b, int r0, int it) {
        float s[2 * RPI];
#pragma unroll
        for (int j = 0; j < RPI; ++j) {
            float s1 = 0.f, s2 = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float xh = (b.x[j][e] - b.mu[j]) * b.rs[j], d = b.dy[j][e];
                float g = d * gm[e];
                s1 += g;
                s2 += g * xh;
                pg[e] += d * xh;
                pb[e] += d;
            }
            s[2 * j] = s1;
            s[2 * j + 1] = s2;
        }
        // sum over the group's waves (every thread of the block reaches the barrier)
        float (*rd)[2 * RPI] = red[it & 1];
#pragma unroll
        for (int k = 0; k < 2 * RPI; ++k) s[k] = wave_sum(s[k]);
        if (lane == 0) {
#pragma unroll
            for (int k = 0; k < 2 * RPI; ++k) rd[wave][k] = s[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 2 * RPI; ++k) {
            float a = rd[w0][k];
            for (int w = 1; w < nwg; ++w) a += rd[w0 + w][k];
            s[k] = a;
        }
#pragma unroll
        for (int j = 0; j < RPI; ++j) {
            const int row = r0 + j;
            if (act && row < rows) {
                const float s1 = s[2 * j] * inv_h, s2 = s[2 * j + 1] * inv_h;
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float xh = (b.x[j][e] - b.mu[j]) * b.rs[j];
                    o[e] = b.rs[j] * (b.dy[j][e] * gm[e] - s1 - xh * s2) + b.dr[j][e];
                    pr[e] += b.dr[j][e];
                    px[e] += o[e];
                }
                store8(dx + (size_t)row * h + c, o);
            }
        }
    };
    // The loop bounds depend on blockIdx only (uniform), so every thread of the block reaches the
    // same barriers; a group's rows past the end are masked. PF: two register sets, alternating.
    const int stride = RPI * G * (int)gridDim.x;
    int base = (int)blockIdx.x * G * RPI, it = 0;
    const int off = grp * RPI;
    if constexpr (PF) {
        LnBwdRows<T, RPI> A, B;
        if (base < rows) A.load(base + off, rows, h, c, act, x, dy, dres, mean, rstd);
        while (base < rows) {
            const int b1 = base + stride;
            if (b1 < rows) B.load(b1 + off, rows, h, c, act, x, dy, dres, mean, rstd);
            process(A, base + off, it++);
            if (b1 >= rows) break;
            const int b2 = b1 + stride;
            if (b2 < rows) A.load(b2 + off, rows, h, c, act, x, dy, dres, mean, rstd);
            process(B, b1 + off, it++);
            base = b2;
        }
    } else {
        for (; base < rows; base += stride) {
            LnBwdRows<T, RPI> A;
            A.load(base + off, rows, h, c, act, x, dy, dres, mean, rstd);
            process(A, base + off, it++);
        }
    }
    // the groups' column sums, added in group order: group g > 0 hands its 8 values per column to
    // group 0 through LDS, one job at a time
    const size_t po = (size_t)blockIdx.x * h + c;
    auto finish = [&](float* __restrict__ out, float (&v)[8]) {
        if (!out) return;   // uniform
        if constexpr (G > 1) {
            __shared__ f32x4 xg[2][512];   // one group's 8 values per thread
            static_assert(NTMAX / G <= 512, "group exchange buffer too small");
            for (int g = 1; g < G; ++g) {
                __syncthreads();
                if (grp == g) {
                    xg[0][tid] = f32x4{v[0], v[1], v[2], v[3]};
                    xg[1][tid] = f32x4{v[4], v[5], v[6], v[7]};
                }
                __syncthreads();
                if (grp == 0) {
                    const f32x4 lo = xg[0][tid], hi = xg[1][tid];
#pragma unroll
                    for (int e = 0; e < 4; ++e) { v[e] += lo[e]; v[4 + e] += hi[e]; }
                }
            }
        }
        if (grp == 0 && act) store8(out + po, v);
    };
    finish(part_g, pg);
    finish(part_b, pb);
    finish(part_r, pr);
    finish(part_x, px);
}

// out_j[c] (+)= sum_{b=0}^{nb-1} part_j[b][c] for job j = blockIdx.y (n % 4 == 0): rowsum_block over
// column block blockIdx.x.
constexpr int RR_JOBS = 4;
struct RowSumJobs { const float* part[RR_JOBS]; void* out[RR_JOBS]; };
template <typename T>
__global__ __launch_bounds__(256) void reduce_rows_kernel(RowSumJobs jobs, int nb, int n, int accumulate) {
    rowsum_block<T>(jobs.part[blockIdx.y], (T*)jobs.out[blockIdx.y], nb, n, accumulate, (int)blockIdx.x);
}

// ---------------------------------------------------------------------------------------------
// Column partial sums of G [rows, n] (n % 8 == 0): grid (ceil(n/512), RB), 256 threads. Lane owns
// 8 columns; block y covers the row range [y*rpb, (y+1)*rpb), wave w its rows w, w+4, ...; the
// four wave sums are added in wave order and written as part[y][n].
// ---------------------------------------------------------------------------------------------
// DROP: y = D(G) is written (in place allowed: each element is read, then written, by one thread)
// and the column sums are those of D(G) (fp32 values before rounding to T).
template <typename T, bool DROP = false>
__global__ __launch_bounds__(256) void colsum_partial_kernel(int rows, int n, int rpb, const T* G,
                                                            float* __restrict__ part, DropParams dp = DropParams{},
                                                            T* y = nullptr) {
    __shared__ float red[4][512];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = (blockIdx.x * 64 + lane) * 8;
    const int r0 = blockIdx.y * rpb, r1 = min(rows, r0 + rpb);
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (c < n) {
#pragma unroll 8
        for (int r = r0 + wave; r < r1; r += 4) {
            float v[8];
            load8(G + (size_t)r * n + c, v);
            if constexpr (DROP) {
                const size_t i = (size_t)r * n + c;
                apply_keep8(v, keep8(i >> 3, dp), dp.scale);
                store8(y + i, v);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] += v[e];
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][lane * 8 + e] = a[e];
    __syncthreads();
    if (wave == 0 && c < n) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            a[e] = ((red[0][lane * 8 + e] + red[1][lane * 8 + e]) + red[2][lane * 8 + e]) + red[3][lane * 8 + e];
        store8(part + (size_t)blockIdx.y * n + c, a);
    }
}

// ---------------------------------------------------------------------------------------------
// out = residual + D(sum_r parts[r] + bias) (fp32 sum in rank order; D = residual dropout or the
// identity), 8 elements per thread. With cols % 8 == 0, flat index i / 8 is the dropout call of
// the thread's 8 elements.
// ---------------------------------------------------------------------------------------------
constexpr int SUM_MAX_T = 64;
struct PartPtrs { const void* p[SUM_MAX_T]; };

template <typename TI, typename TO>
__global__ __launch_bounds__(256) void sum_partials_kernel(size_t n_elems, int cols, int t, PartPtrs parts,
                                                           const TO* __restrict__ bias,
                                                           const TO* __restrict__ residual, TO* __restrict__ out,
                                                           DropParams drop) {
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
    if (drop.thr) apply_keep8(a, keep8(i >> 3, drop), drop.scale);
    if (residual) {
        float rr[8];
        load8(residual + i, rr);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] += rr[e];
    }
    store8(out + i, a);
}

// y = D(x) over a contiguous [rows, cols] tensor (cols % 8 == 0): the residual-site mapping,
// 8 elements (one call) per thread. In place is allowed.
template <typename T>
__global__ __launch_bounds__(256) void dropout_kernel(size_t n_elems, const T* x, T* y, DropParams drop) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= n_elems) return;
    float v[8];
    load8(x + i, v);
    apply_keep8(v, keep8(i >> 3, drop), drop.scale);
    store8(y + i, v);
}

}  // namespace tp
