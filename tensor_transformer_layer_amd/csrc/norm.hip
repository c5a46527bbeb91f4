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

int ln_bwd_blocks(int rows) {
    int nb = (rows + 7) / 8;
    return nb < 512 ? nb : 512;
}

template <typename T>
static hipError_t ln_bwd_t(int rows, int h, const void* x, const void* g, const float* mean, const float* rstd,
                           const void* dy, const void* dres, void* dx, void* dg, void* db, int accumulate, float* ws,
                           hipStream_t st) {
    int nb = ln_bwd_blocks(rows);
    bool params = dg != nullptr || db != nullptr;
    float* pg = params ? ws : nullptr;
    float* pb = params ? ws + (size_t)nb * h : nullptr;
    size_t lds = params ? 2 * (size_t)h * sizeof(float) : 0;
#define LNB(C) hipLaunchKernelGGL((ln_bwd_kernel<T, C>), dim3(nb), dim3(256), lds, st, rows, h, (const T*)x, \
                                  (const T*)g, mean, rstd, (const T*)dy, (const T*)dres, (T*)dx, pg, pb)
    switch (ln_chunks(h)) {
        case 1: LNB(1); break;
        case 2: LNB(2); break;
        case 3: LNB(3); break;
        case 4: LNB(4); break;
        case 6: LNB(6); break;
        case 8: LNB(8); break;
        case 12: LNB(12); break;
        case 16: LNB(16); break;
        default: return hipErrorInvalidValue;
    }
#undef LNB
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !params) return e;
    dim3 rg((h + 63) / 64);
    if (dg) hipLaunchKernelGGL((reduce_rows_kernel<T>), rg, dim3(256), 0, st, (const float*)pg, nb, h, (T*)dg, accumulate);
    if (db) hipLaunchKernelGGL((reduce_rows_kernel<T>), rg, dim3(256), 0, st, (const float*)pb, nb, h, (T*)db, accumulate);
    return hipGetLastError();
}

hipError_t layernorm_bwd(int dt, int rows, int h, const void* x, const void* g, const float* mean,
                         const float* rstd, const void* dy, const void* dres, void* dx, void* dg, void* db,
                         int accumulate, float* ws, hipStream_t st) {
    if (rows == 0) {
        // no rows: parameter gradients are zero (unchanged when accumulating); a zero-block reduction writes them
        dim3 rg((h + 63) / 64);
        if (dt == 1) {
            if (dg) hipLaunchKernelGGL((reduce_rows_kernel<bf16>), rg, dim3(256), 0, st, (const float*)ws, 0, h, (bf16*)dg, accumulate);
            if (db) hipLaunchKernelGGL((reduce_rows_kernel<bf16>), rg, dim3(256), 0, st, (const float*)ws, 0, h, (bf16*)db, accumulate);
        } else {
            if (dg) hipLaunchKernelGGL((reduce_rows_kernel<float>), rg, dim3(256), 0, st, (const float*)ws, 0, h, (float*)dg, accumulate);
            if (db) hipLaunchKernelGGL((reduce_rows_kernel<float>), rg, dim3(256), 0, st, (const float*)ws, 0, h, (float*)db, accumulate);
        }
        return hipGetLastError();
    }
    return dt == 1 ? ln_bwd_t<bf16>(rows, h, x, g, mean, rstd, dy, dres, dx, dg, db, accumulate, ws, st)
                   : ln_bwd_t<float>(rows, h, x, g, mean, rstd, dy, dres, dx, dg, db, accumulate, ws, st);
}

int colsum_row_blocks(int rows) { return rows < 512 ? (rows > 0 ? rows : 1) : 512; }

hipError_t colsum(int dt, int rows, int n, const void* G, void* out, int accumulate, float* ws, hipStream_t st) {
    int rb = colsum_row_blocks(rows);
    if (rows > 0) {
        dim3 grid((n / 8 + 63) / 64, rb);
        if (dt == 1) hipLaunchKernelGGL((colsum_partial_kernel<bf16>), grid, dim3(64), 0, st, rows, n, (const bf16*)G, ws);
        else hipLaunchKernelGGL((colsum_partial_kernel<float>), grid, dim3(64), 0, st, rows, n, (const float*)G, ws);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int nb = rows > 0 ? rb : 0;
    dim3 rg((n + 63) / 64);
    if (dt == 1) hipLaunchKernelGGL((reduce_rows_kernel<bf16>), rg, dim3(256), 0, st, (const float*)ws, nb, n, (bf16*)out, accumulate);
    else hipLaunchKernelGGL((reduce_rows_kernel<float>), rg, dim3(256), 0, st, (const float*)ws, nb, n, (float*)out, accumulate);
    return hipGetLastError();
}

hipError_t sum_partials(int in_dt, int out_dt, size_t rows, int cols, int t, const void* const* parts,
                        const void* bias, const void* residual, void* out, hipStream_t st) {
    size_t n = rows * (size_t)cols;
    if (n == 0) return hipSuccess;
    PartPtrs pp;
    for (int r = 0; r < t; ++r) pp.p[r] = parts[r];
    dim3 grid((unsigned)((n / 8 + 255) / 256));
    if (in_dt == 1 && out_dt == 1)
        hipLaunchKernelGGL((sum_partials_kernel<bf16, bf16>), grid, dim3(256), 0, st, n, cols, t, pp,
                           (const bf16*)bias, (const bf16*)residual, (bf16*)out);
    else if (in_dt == 1 && out_dt == 0)
        hipLaunchKernelGGL((sum_partials_kernel<bf16, float>), grid, dim3(256), 0, st, n, cols, t, pp,
                           (const float*)bias, (const float*)residual, (float*)out);
    else if (in_dt == 0 && out_dt == 1)
        hipLaunchKernelGGL((sum_partials_kernel<float, bf16>), grid, dim3(256), 0, st, n, cols, t, pp,
                           (const bf16*)bias, (const bf16*)residual, (bf16*)out);
    else
        hipLaunchKernelGGL((sum_partials_kernel<float, float>), grid, dim3(256), 0, st, n, cols, t, pp,
                           (const float*)bias, (const float*)residual, (float*)out);
    return hipGetLastError();
}

}  // namespace tp
