// Launchers of the cross-entropy merge / combine kernels (xent.h). The fused GEMM itself is
// launched through the K-contiguous GEMM unit with the EPI_XENT epilogue.
#include "launch.h"
#include "xent.h"

namespace tp {

// Per token: merge the tiles' partials in tile order.
__global__ __launch_bounds__(256) void xent_merge_kernel(const XentPartial* __restrict__ part, int tiles_m, int N,
                                                         int col0, float* __restrict__ max_r,
                                                         float* __restrict__ sumexp_r, float* __restrict__ tgt_r,
                                                         int32_t* __restrict__ argmax_r) {
    int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    float mx = -INFINITY, se = 0.f, tv = 0.f;
    int am = INT_MAX;
    for (int tm = 0; tm < tiles_m; ++tm) {
        XentPartial p = part[(size_t)tm * N + n];
        float m2 = mx;
        int a2 = am;
        xent_better(m2, a2, p.mx, p.am);
        xent_merge_se(mx, se, p.mx, p.se);
        am = a2;
        tv += p.tv;
    }
    max_r[n] = mx;
    sumexp_r[n] = se;
    tgt_r[n] = tv;
    if (argmax_r) argmax_r[n] = (am == INT_MAX) ? -1 : col0 + am;
}

constexpr int XENT_MAX_T = 64;
struct XentPtrs {
    const float* mx[XENT_MAX_T];
    const float* se[XENT_MAX_T];
    const float* tg[XENT_MAX_T];
};

// loss_n = M + log(sum_r se_r exp(mx_r - M)) - sum_r tg_r, ranks merged in order.
__global__ __launch_bounds__(256) void xent_combine_kernel(int N, int t, XentPtrs p, float* __restrict__ loss) {
    int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    float M = -INFINITY;
    for (int r = 0; r < t; ++r) M = fmaxf(M, p.mx[r][n]);
    float S = 0.f, T = 0.f;
    for (int r = 0; r < t; ++r) {
        float m = p.mx[r][n];
        if (m != -INFINITY) S += p.se[r][n] * expf(m - M);
        T += p.tg[r][n];
    }
    loss[n] = M + logf(S) - T;
}

// mean of x[0..N) with one block, fixed order: thread partials over a stride, then a tree.
__global__ __launch_bounds__(256) void mean_kernel(const float* __restrict__ x, int N, float* __restrict__ out) {
    __shared__ float red[256];
    float a = 0.f;
    for (int i = threadIdx.x; i < N; i += 256) a += x[i];
    red[threadIdx.x] = a;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = red[0] / (float)N;
}


hipError_t xent_merge(const void* part, int tiles_m, int N, int col0, float* mx, float* se, float* tg,
                      int32_t* am, hipStream_t st) {
    if (N == 0) return hipSuccess;
    hipLaunchKernelGGL(xent_merge_kernel, dim3((N + 255) / 256), dim3(256), 0, st, (const XentPartial*)part,
                       tiles_m, N, col0, mx, se, tg, am);
    return hipGetLastError();
}

hipError_t xent_combine(int N, int t, const float* const* mx, const float* const* se, const float* const* tg,
                        float* loss, float* mean, hipStream_t st) {
    if (N == 0) return hipSuccess;
    XentPtrs p;
    for (int r = 0; r < t; ++r) { p.mx[r] = mx[r]; p.se[r] = se[r]; p.tg[r] = tg[r]; }
    hipLaunchKernelGGL(xent_combine_kernel, dim3((N + 255) / 256), dim3(256), 0, st, N, t, p, loss);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !mean) return e;
    hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(256), 0, st, (const float*)loss, N, mean);
    return hipGetLastError();
}

}  // namespace tp
