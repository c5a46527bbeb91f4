// Launchers of the LayerNorm / column-sum / partial-sum kernels (norm.h).
#include "launch.h"
#include "norm.h"

namespace tp {

// chunks of 8 per lane needed for a row of h
static int ln_chunks(int h) {
    int c = (h + 511) / 512;
    static const int opts[] = {1, 2, 3, 4, 6, 8, 12, 16};
    for (int o : opts)
        if (o >= c) return o;
    return -1;
}

template <typename T>
static hipError_t ln_fwd_t(int rows, int h, float eps, const void* x, const void* g, const void* b, void* y,
                           float* mean, float* rstd, hipStream_t st) {
    dim3 grid((rows + 3) / 4);
#define LNF(C) hipLaunchKernelGGL((ln_fwd_kernel<T, C>), grid, dim3(256), 0, st, rows, h, eps, (const T*)x, \
                                  (const T*)g, (const T*)b, (T*)y, mean, rstd)
    switch (ln_chunks(h)) {
        case 1: LNF(1); break;
        case 2: LNF(2); break;
        case 3: LNF(3); break;
        case 4: LNF(4); break;
        case 6: LNF(6); break;
        case 8: LNF(8); break;
        case 12: LNF(12); break;
        case 16: LNF(16); break;
        default: return hipErrorInvalidValue;
    }
#undef LNF
    return hipGetLastError();
}

hipError_t layernorm_fwd(int dt, int rows, int h, float eps, const void* x, const void* g, const void* b, void* y,
                         float* mean, float* rstd, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    return dt == 1 ? ln_fwd_t<bf16>(rows, h, eps, x, g, b, y, mean, rstd, st)
                   : ln_fwd_t<float>(rows, h, eps, x, g, b, y, mean, rstd, st);
}

hipError_t sum_partials_layernorm(int dt, int rows, int h, int t, const void* const* parts, const void* bias,
                                  const void* residual, void* out, float eps, const void* g, const void* b, void* y,
                                  float* mean, float* rstd, const DropParams& drop, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    if (t < 1 || t > ADDLN_MAX_T) return hipErrorInvalidValue;
    AddLnParts pp;
    for (int r = 0; r < t; ++r) pp.p[r] = parts[r];
    dim3 grid((rows + 3) / 4);
#define ADDLN(TT, C) hipLaunchKernelGGL((add_ln_fwd_kernel<TT, C>), grid, dim3(256), 0, st, rows, h, t, pp, (const TT*)bias, \
                                        (const TT*)residual, (TT*)out, eps, (const TT*)g, (const TT*)b, (TT*)y, mean, rstd, drop)
#define ADDLN_T(TT)                        \
    switch (ln_chunks(h)) {                \
        case 1: ADDLN(TT, 1); break;       \
        case 2: ADDLN(TT, 2); break;       \
        case 3: ADDLN(TT, 3); break;       \
        case 4: ADDLN(TT, 4); break;       \
        case 6: ADDLN(TT, 6); break;       \
        case 8: ADDLN(TT, 8); break;       \
        case 12: ADDLN(TT, 12); break;     \
        case 16: ADDLN(TT, 16); break;     \
        default: return hipErrorInvalidValue; \
    }
    if (dt == 1) { ADDLN_T(bf16) } else { ADDLN_T(float) }
#undef ADDLN_T
#undef ADDLN
    return hipGetLastError();
}

// threads of a LayerNorm backward block: 8 columns each, whole waves
static int ln_threads(int h) { return (h + 511) / 512 * 64; }

// Blocks of the LayerNorm backward: at least 32 rows each (16 per row group), at most 256 (one per
// CU; fewer blocks also mean fewer column-sum partial rows to write and reduce).
int ln_bwd_blocks(int rows) {
    int nb = (rows + 31) / 32;
    return nb < 256 ? (nb > 0 ? nb : 1) : 256;
}

// out_j (+)= column sums of part_j [nb][n] for the non-null outputs (nb may be 0: zeros)
template <typename T>
static hipError_t reduce_rows(const float* const* parts, void* const* outs, int nb, int n, int accumulate,
                              hipStream_t st) {
    RowSumJobs jobs;
    int nj = 0;
    for (int j = 0; j < RR_JOBS; ++j)
        if (outs[j]) { jobs.part[nj] = parts[j]; jobs.out[nj] = outs[j]; ++nj; }
    if (nj == 0) return hipSuccess;
    hipLaunchKernelGGL((reduce_rows_kernel<T>), dim3((n + RR_COLS - 1) / RR_COLS, nj), dim3(256), 0, st, jobs, nb, n,
                       accumulate);
    return hipGetLastError();
}

template <typename T>
static hipError_t ln_bwd_t(int rows, int h, const void* x, const void* g, const float* mean, const float* rstd,
                           const void* dy, const void* dres, void* dx, void* dg, void* db, void* dsr, void* dsx,
                           int accumulate, float* ws, hipStream_t st) {
    if (h <= 0 || h > LN_MAX_H) return hipErrorInvalidValue;
    const int nb = rows > 0 ? ln_bwd_blocks(rows) : 0;
    void* outs[RR_JOBS] = {dg, db, dsr, dsx};
    float* parts[RR_JOBS];
    for (int j = 0; j < RR_JOBS; ++j) parts[j] = outs[j] ? ws + (size_t)j * ln_bwd_blocks(rows) * h : nullptr;
    if (rows > 0) {
        // Up to 384 threads per row: two row groups per block, one row per iteration and group with
        // the next in flight (two rows per group spill at this block size). Against one group of
        // two rows per iteration on 512 blocks, inside the layer step at T = 8192, h = 3072 (inputs
        // not in the MALL), kernel + reduction: 60.8 -> 53.0 us with dres and four column sums,
        // 49.9 -> 47.5 us with two: ~4.5 TB/s, near a plain copy's 5.05. Up to 512 threads: one
        // group, two rows, prefetched. Wider (register budget 128 per lane): no prefetch.
        const int nt = ln_threads(h);
#define TP_LN_BWD(NTMAX, RPI, G, PF)                                                                          \
    hipLaunchKernelGGL((ln_bwd_kernel<T, NTMAX, RPI, G, PF>), dim3(nb), dim3(G * nt), 0, st, rows, h, (const T*)x,  \
                       (const T*)g, mean, rstd, (const T*)dy, (const T*)dres, (T*)dx, parts[0], parts[1], parts[2],   \
                       parts[3])
        if (nt <= 384) TP_LN_BWD(768, 1, 2, true);
        else if (nt <= 512) TP_LN_BWD(512, 2, 1, true);
        else TP_LN_BWD(1024, 2, 1, false);
#undef TP_LN_BWD
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // no rows: a zero-row reduction writes zero gradients (unchanged when accumulating)
    return reduce_rows<T>(parts, outs, nb, h, accumulate, st);
}

hipError_t layernorm_bwd(int dt, int rows, int h, const void* x, const void* g, const float* mean,
                         const float* rstd, const void* dy, const void* dres, void* dx, void* dg, void* db,
                         void* dres_sum, void* dx_sum, int accumulate, float* ws, hipStream_t st) {
    return dt == 1 ? ln_bwd_t<bf16>(rows, h, x, g, mean, rstd, dy, dres, dx, dg, db, dres_sum, dx_sum, accumulate, ws, st)
                   : ln_bwd_t<float>(rows, h, x, g, mean, rstd, dy, dres, dx, dg, db, dres_sum, dx_sum, accumulate, ws, st);
}

// Row blocks of the column-sum pass: about 64 rows each, at most 128 blocks.
int colsum_row_blocks(int rows) {
    if (rows <= 0) return 1;
    int rb = (rows + 63) / 64;
    return rb < 128 ? rb : 128;
}

hipError_t colsum(int dt, int rows, int n, const void* G, void* out, int accumulate, float* ws, hipStream_t st) {
    int rb = colsum_row_blocks(rows);
    if (rows > 0) {
        int rpb = (rows + rb - 1) / rb;
        dim3 grid((n / 8 + 63) / 64, rb);
        if (dt == 1) hipLaunchKernelGGL((colsum_partial_kernel<bf16>), grid, dim3(256), 0, st, rows, n, rpb, (const bf16*)G, ws);
        else hipLaunchKernelGGL((colsum_partial_kernel<float>), grid, dim3(256), 0, st, rows, n, rpb, (const float*)G, ws);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int nb = rows > 0 ? rb : 0;
    const float* parts[RR_JOBS] = {ws, nullptr, nullptr, nullptr};
    void* outs[RR_JOBS] = {out, nullptr, nullptr, nullptr};
    return dt == 1 ? reduce_rows<bf16>(parts, outs, nb, n, accumulate, st)
                   : reduce_rows<float>(parts, outs, nb, n, accumulate, st);
}

hipError_t colsum_reduce(int dt, int nb, int n, const float* part, void* out, int accumulate, hipStream_t st) {
    const float* parts[RR_JOBS] = {part, nullptr, nullptr, nullptr};
    void* outs[RR_JOBS] = {out, nullptr, nullptr, nullptr};
    return dt == 1 ? reduce_rows<bf16>(parts, outs, nb, n, accumulate, st)
                   : reduce_rows<float>(parts, outs, nb, n, accumulate, st);
}

hipError_t dropout_colsum(int dt, int rows, int n, const void* x, void* y, const DropParams& dp, void* out,
                          int accumulate, float* ws, hipStream_t st) {
    int rb = colsum_row_blocks(rows);
    if (rows > 0) {
        int rpb = (rows + rb - 1) / rb;
        dim3 grid((n / 8 + 63) / 64, rb);
        if (dt == 1)
            hipLaunchKernelGGL((colsum_partial_kernel<bf16, true>), grid, dim3(256), 0, st, rows, n, rpb, (const bf16*)x,
                               ws, dp, (bf16*)y);
        else
            hipLaunchKernelGGL((colsum_partial_kernel<float, true>), grid, dim3(256), 0, st, rows, n, rpb,
                               (const float*)x, ws, dp, (float*)y);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int nb = rows > 0 ? rb : 0;
    const float* parts[RR_JOBS] = {ws, nullptr, nullptr, nullptr};
    void* outs[RR_JOBS] = {out, nullptr, nullptr, nullptr};
    return dt == 1 ? reduce_rows<bf16>(parts, outs, nb, n, accumulate, st)
                   : reduce_rows<float>(parts, outs, nb, n, accumulate, st);
}

hipError_t sum_partials(int in_dt, int out_dt, size_t rows, int cols, int t, const void* const* parts,
                        const void* bias, const void* residual, void* out, const DropParams& drop, hipStream_t st) {
    size_t n = rows * (size_t)cols;
    if (t < 1 || t > SUM_MAX_T) return hipErrorInvalidValue;
    if (n == 0) return hipSuccess;
    PartPtrs pp;
    for (int r = 0; r < t; ++r) pp.p[r] = parts[r];
    dim3 grid((unsigned)((n / 8 + 255) / 256));
    if (in_dt == 1 && out_dt == 1)
        hipLaunchKernelGGL((sum_partials_kernel<bf16, bf16>), grid, dim3(256), 0, st, n, cols, t, pp,
                           (const bf16*)bias, (const bf16*)residual, (bf16*)out, drop);
    else if (in_dt == 1 && out_dt == 0)
        hipLaunchKernelGGL((sum_partials_kernel<bf16, float>), grid, dim3(256), 0, st, n, cols, t, pp,
                           (const float*)bias, (const float*)residual, (float*)out, drop);
    else if (in_dt == 0 && out_dt == 1)
        hipLaunchKernelGGL((sum_partials_kernel<float, bf16>), grid, dim3(256), 0, st, n, cols, t, pp,
                           (const bf16*)bias, (const bf16*)residual, (bf16*)out, drop);
    else
        hipLaunchKernelGGL((sum_partials_kernel<float, float>), grid, dim3(256), 0, st, n, cols, t, pp,
                           (const float*)bias, (const float*)residual, (float*)out, drop);
    return hipGetLastError();
}

hipError_t dropout(int dt, size_t n, const void* x, void* y, const DropParams& drop, hipStream_t st) {
    if (n == 0) return hipSuccess;
    dim3 grid((unsigned)((n / 8 + 255) / 256));
    if (dt == 1)
        hipLaunchKernelGGL(dropout_kernel<bf16>, grid, dim3(256), 0, st, n, (const bf16*)x, (bf16*)y, drop);
    else
        hipLaunchKernelGGL(dropout_kernel<float>, grid, dim3(256), 0, st, n, (const float*)x, (float*)y, drop);
    return hipGetLastError();
}

}  // namespace tp
