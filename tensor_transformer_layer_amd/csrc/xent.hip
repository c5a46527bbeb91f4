// Launchers of the cross-entropy merge / combine kernels (xent.h). The fused GEMM itself is
// launched through the K-contiguous GEMM unit with the EPI_XENT epilogue.
#include "launch.h"
#include "xent.h"

namespace tp {

// Per token: merge the tiles' partials. Block = 64 tokens x 4 phases; phase p merges tiles
// p, p+4, ... in order, then the four phase results are merged in phase order.
struct XentAcc {
    float mx, se, tv;
    int am;
    __device__ __forceinline__ void init() { mx = -INFINITY; se = 0.f; tv = 0.f; am = INT_MAX; }
    __device__ __forceinline__ void add(float pmx, float pse, float ptv, int pam) {
        float m2 = mx;
        int a2 = am;
        xent_better(m2, a2, pmx, pam);
        xent_merge_se(mx, se, pmx, pse);
        am = a2;
        tv += ptv;
    }
};

__global__ __launch_bounds__(256) void xent_merge_kernel(const XentPartial* __restrict__ part, int tiles_m, int N,
                                                         int col0, float* __restrict__ max_r,
                                                         float* __restrict__ sumexp_r, float* __restrict__ tgt_r,
                                                         int32_t* __restrict__ argmax_r) {
    __shared__ XentPartial red[4][64];
    const int tl = threadIdx.x & 63, ph = threadIdx.x >> 6;
    const int n = blockIdx.x * 64 + tl;
    XentAcc a;
    a.init();
    if (n < N) {
        // up to eight of the phase's partials in flight at once, then merged in tile order
        for (int t0 = ph; t0 < tiles_m; t0 += 32) {
            XentPartial q[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int tm = t0 + 4 * j;
                q[j] = tm < tiles_m ? part[(size_t)tm * N + n] : XentPartial{-INFINITY, 0.f, 0.f, INT_MAX};
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (t0 + 4 * j < tiles_m) a.add(q[j].mx, q[j].se, q[j].tv, q[j].am);
        }
    }
    red[ph][tl] = XentPartial{a.mx, a.se, a.tv, a.am};
    __syncthreads();
    if (ph != 0 || n >= N) return;
    for (int q = 1; q < 4; ++q) {
        XentPartial p = red[q][tl];
        a.add(p.mx, p.se, p.tv, p.am);
    }
    max_r[n] = a.mx;
    sumexp_r[n] = a.se;
    tgt_r[n] = a.tv;
    if (argmax_r) argmax_r[n] = (a.am == INT_MAX) ? -1 : col0 + a.am;
}

constexpr int XENT_MAX_T = 64;
struct XentPtrs {
    const float* mx[XENT_MAX_T];
    const float* se[XENT_MAX_T];
    const float* tg[XENT_MAX_T];
};

// loss_n = M + log(sum_r se_r exp(mx_r - M)) - sum_r tg_r: the global max first, then the sums
// relative to it, ranks in order. Ranks are read eight at a time so their loads are in flight
// together.
__global__ __launch_bounds__(64) void xent_combine_kernel(int N, int t, XentPtrs p, float* __restrict__ loss,
                                                          float* __restrict__ max_all, float* __restrict__ sumexp_all) {
    int n = blockIdx.x * 64 + threadIdx.x;
    if (n >= N) return;
    float M = -INFINITY;
    for (int r0 = 0; r0 < t; r0 += 8) {
        float mx[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) mx[k] = (r0 + k < t) ? p.mx[r0 + k][n] : -INFINITY;
#pragma unroll
        for (int k = 0; k < 8; ++k) M = fmaxf(M, mx[k]);
    }
    float S = 0.f, T = 0.f;
    for (int r0 = 0; r0 < t; r0 += 8) {
        float mx[8], se[8], tg[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const bool in = r0 + k < t;
            mx[k] = in ? p.mx[r0 + k][n] : -INFINITY;
            se[k] = in ? p.se[r0 + k][n] : 0.f;
            tg[k] = in ? p.tg[r0 + k][n] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (mx[k] != -INFINITY) S += se[k] * expf(mx[k] - M);
            T += tg[k];
        }
    }
    loss[n] = M + logf(S) - T;
    if (max_all) max_all[n] = M;
    if (sumexp_all) sumexp_all[n] = S;
}

// mean of x[0..N) with one block, fixed order: each thread sums a stride with four running
// partials (added in order), then a tree over the threads.
__global__ __launch_bounds__(1024) void mean_kernel(const float* __restrict__ x, int N, float* __restrict__ out) {
    __shared__ float red[1024];
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    int i = threadIdx.x;
    for (; i + 3 * 1024 < N; i += 4 * 1024) {
#pragma unroll
        for (int k = 0; k < 4; ++k) a[k] += x[i + k * 1024];
    }
    for (int k = 0; i < N; i += 1024, ++k) a[k] += x[i];
    red[threadIdx.x] = (a[0] + a[1]) + (a[2] + a[3]);
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = red[0] / (float)N;
}


// ---------------------------------------------------------------------------------------------
// Per-token statistics of materialised fp32 logits (the unfused form: the logits are in memory).
// One wave per token row; lane l takes 4-column chunks l, l+64, ... (each load instruction of a
// wave reads 1 KB of the row), U chunks in flight per lane. A lane keeps a running max (strict >,
// so the lowest column wins a tie among its own columns, which it visits in increasing order), its
// column, and the sum of exp(y - max) rescaled when a chunk raises the max; the 64 lanes' triples
// are merged by a butterfly (ties to the lower column). The target logit is read directly.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void xent_row_merge(float& m, float& s, int& a, float m2, float s2, int a2) {
    const float mn = fmaxf(m, m2);
    const bool take = m2 > m || (m2 == m && a2 < a);
    if (mn == -INFINITY) {
        s = 0.f;
    } else {
        s = (m == -INFINITY ? 0.f : s * __expf(m - mn)) + (m2 == -INFINITY ? 0.f : s2 * __expf(m2 - mn));
    }
    if (take) a = a2;
    m = mn;
}

template <int U>
__global__ __launch_bounds__(256) void xent_rows_kernel(const float* __restrict__ logits, int ld, int N, int Vt,
                                                        int col0, int vend, const int32_t* __restrict__ targets,
                                                        float* __restrict__ max_r, float* __restrict__ sumexp_r,
                                                        float* __restrict__ tgt_r, int32_t* __restrict__ argmax_r) {
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;
    const float* row = logits + (size_t)n * ld;
    const int nch = (vend + 3) >> 2;
    float m = -INFINITY, s = 0.f;
    int a = INT_MAX;
    for (int j0 = 0; j0 < nch; j0 += 64 * U) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + 64 * u + lane;
            v[u] = j < nch ? *(const f32x4*)(row + 4 * j) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c0 = 4 * (j0 + 64 * u + lane);
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = c0 + e < vend ? v[u][e] : -INFINITY;
            float cm = y[0];
            int ca = c0;
#pragma unroll
            for (int e = 1; e < 4; ++e)
                if (y[e] > cm) { cm = y[e]; ca = c0 + e; }
            if (cm > m) {
                s = (m == -INFINITY) ? 0.f : s * __expf(m - cm);
                m = cm;
                a = ca;
            }
            if (m != -INFINITY) {
#pragma unroll
                for (int e = 0; e < 4; ++e) s += (y[e] == -INFINITY) ? 0.f : __expf(y[e] - m);
            }
        }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
        const int a2 = __shfl_xor(a, o);
        xent_row_merge(m, s, a, m2, s2, a2);
    }
    if (lane == 0) {
        const int local = targets[n] - col0;
        max_r[n] = m;
        sumexp_r[n] = s;
        tgt_r[n] = (local >= 0 && local < Vt) ? row[local] : 0.f;
        if (argmax_r) argmax_r[n] = (a == INT_MAX) ? -1 : col0 + a;
    }
}

hipError_t xent_stats_from_logits(const float* logits, int ld, int N, int Vt, int col0, int Vreal, int mask,
                                  const int32_t* targets, float* mx, float* se, float* tg, int32_t* am,
                                  hipStream_t st) {
    if (N == 0) return hipSuccess;
    const int vend = mask ? max(0, min(Vt, Vreal - col0)) : Vt;
    hipLaunchKernelGGL(xent_rows_kernel<4>, dim3((N + 3) / 4), dim3(256), 0, st, logits, ld, N, Vt, col0, vend, targets,
                       mx, se, tg, am);
    return hipGetLastError();
}

hipError_t xent_merge(const void* part, int tiles_m, int N, int col0, float* mx, float* se, float* tg,
                      int32_t* am, hipStream_t st) {
    if (N == 0) return hipSuccess;
    hipLaunchKernelGGL(xent_merge_kernel, dim3((N + 63) / 64), dim3(256), 0, st, (const XentPartial*)part,
                       tiles_m, N, col0, mx, se, tg, am);
    return hipGetLastError();
}

hipError_t xent_combine(int N, int t, const float* const* mx, const float* const* se, const float* const* tg,
                        float* loss, float* mean, float* max_all, float* sumexp_all, hipStream_t st) {
    if (N == 0) return hipSuccess;
    XentPtrs p;
    for (int r = 0; r < t; ++r) { p.mx[r] = mx[r]; p.se[r] = se[r]; p.tg[r] = tg[r]; }
    hipLaunchKernelGGL(xent_combine_kernel, dim3((N + 63) / 64), dim3(64), 0, st, N, t, p, loss, max_all, sumexp_all);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !mean) return e;
    hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(1024), 0, st, (const float*)loss, N, mean);
    return hipGetLastError();
}

}  // namespace tp
