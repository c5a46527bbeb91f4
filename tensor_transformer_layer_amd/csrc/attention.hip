// Launchers of the attention kernels (attention.h).
#include <math.h>
#include "attention.h"
#include "launch.h"

namespace tp {

template <int D>
static hipError_t fwd_d(int b, int s, int h_t, int heads_t, int causal, const void* QKV, void* O, float* lse,
                        const DropParams& dp, hipStream_t st) {
    dim3 grid(b * heads_t, (s + ATT_B - 1) / ATT_B);
    float scale_log2 = kLog2e / sqrtf((float)D);
    if (dp.thr)
        hipLaunchKernelGGL((attn_fwd_kernel<D, true>), grid, dim3(ATT_NT), 0, st, (const bf16*)QKV, 3 * h_t, h_t, s,
                           heads_t, scale_log2, causal, (bf16*)O, h_t, lse, dp);
    else
        hipLaunchKernelGGL((attn_fwd_kernel<D, false>), grid, dim3(ATT_NT), 0, st, (const bf16*)QKV, 3 * h_t, h_t, s,
                           heads_t, scale_log2, causal, (bf16*)O, h_t, lse, dp);
    return hipGetLastError();
}

template <int D>
static hipError_t bwd_d(int b, int s, int h_t, int heads_t, int causal, const void* QKV, const void* O,
                        const float* lse, const void* dO, float* Dws, void* dSws, void* dQKV, float* colpart,
                        const DropParams& dp, hipStream_t st) {
    size_t rows = (size_t)b * s * heads_t;
    hipLaunchKernelGGL((attn_bwd_dot_kernel<D>), dim3((unsigned)((rows * 4 + 255) / 256)), dim3(256), 0, st,
                       (const bf16*)dO, (const bf16*)O, h_t, b, s, heads_t, Dws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid(b * heads_t, (s + ATT_B - 1) / ATT_B);
    float scale = 1.0f / sqrtf((float)D);
    float scale_log2 = kLog2e * scale;
#define TP_ATT_BWD(DR)                                                                                           \
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, DR>), grid, dim3(ATT_NT), 0, st, (const bf16*)QKV, 3 * h_t, h_t, s, \
                       heads_t, (const bf16*)dO, h_t, lse, (const float*)Dws, scale_log2, scale, causal,            \
                       (bf16*)dQKV, 3 * h_t, (bf16*)dSws, colpart, dp)
    if (dp.thr) TP_ATT_BWD(true);
    else TP_ATT_BWD(false);
#undef TP_ATT_BWD
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D>), grid, dim3(ATT_NT), 0, st, (const bf16*)QKV, 3 * h_t, h_t, s, heads_t,
                       (const bf16*)dSws, scale, causal, (bf16*)dQKV, 3 * h_t, colpart);
    return hipGetLastError();
}

size_t attn_bwd_ds_bytes(int b, int s, int heads_t) {
    const size_t nq = ((size_t)s + ATT_B - 1) / ATT_B;
    return (size_t)b * heads_t * nq * nq * ATT_B * ATT_B * sizeof(bf16);
}

hipError_t attn_fwd(int b, int s, int h_t, int heads_t, int d, int causal, const void* QKV, void* O, float* lse,
                    const DropParams& dp, hipStream_t st) {
    switch (d) {
        case 64: return fwd_d<64>(b, s, h_t, heads_t, causal, QKV, O, lse, dp, st);
        case 96: return fwd_d<96>(b, s, h_t, heads_t, causal, QKV, O, lse, dp, st);
        case 128: return fwd_d<128>(b, s, h_t, heads_t, causal, QKV, O, lse, dp, st);
        case 192: return fwd_d<192>(b, s, h_t, heads_t, causal, QKV, O, lse, dp, st);
    }
    return hipErrorInvalidValue;
}

hipError_t attn_bwd(int b, int s, int h_t, int heads_t, int d, int causal, const void* QKV, const void* O,
                    const float* lse, const void* dO, float* Dws, void* dSws, void* dQKV, float* colpart,
                    const DropParams& dp, hipStream_t st) {
    switch (d) {
        case 64: return bwd_d<64>(b, s, h_t, heads_t, causal, QKV, O, lse, dO, Dws, dSws, dQKV, colpart, dp, st);
        case 96: return bwd_d<96>(b, s, h_t, heads_t, causal, QKV, O, lse, dO, Dws, dSws, dQKV, colpart, dp, st);
        case 128: return bwd_d<128>(b, s, h_t, heads_t, causal, QKV, O, lse, dO, Dws, dSws, dQKV, colpart, dp, st);
        case 192: return bwd_d<192>(b, s, h_t, heads_t, causal, QKV, O, lse, dO, Dws, dSws, dQKV, colpart, dp, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace tp
