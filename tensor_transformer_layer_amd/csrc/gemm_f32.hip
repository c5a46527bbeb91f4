// fp32 SIMT GEMM instantiations (true fp32 products for the fp32 workloads).
#include "gemm.h"
#include "launch.h"

namespace tp {

// 64x64 tiles, or 32x32 when 64x64 would give fewer than 128 workgroups (the small fp32 shapes are
// bound by the latency of their K loop, so more and shorter-running workgroups pay)
template <int LA, int LB, class Epi>
static hipError_t f32_launch(const GemmReq& r, const Epi& e, hipStream_t st) {
    const int tiles64 = ((r.M + 63) / 64) * ((r.N + 63) / 64);
    if (tiles64 == 0) return hipSuccess;
    if (tiles64 >= 128) {
        hipLaunchKernelGGL((gemm_f32_kernel<64, LA, LB, Epi>), dim3(tiles64, 1), dim3(256), 0, st, (const float*)r.A,
                           r.lda, (const float*)r.B, r.ldb, r.M, r.N, r.K, r.K, e);
    } else {
        const int tiles32 = ((r.M + 31) / 32) * ((r.N + 31) / 32);
        hipLaunchKernelGGL((gemm_f32_kernel<32, LA, LB, Epi>), dim3(tiles32, 1), dim3(256), 0, st, (const float*)r.A,
                           r.lda, (const float*)r.B, r.ldb, r.M, r.N, r.K, r.K, e);
    }
    return hipGetLastError();
}

template <int LA, int LB>
static hipError_t f32_run(const GemmReq& r, hipStream_t st) {
    switch (r.epi) {
        case EPI_STORE: return f32_launch<LA, LB>(r, EpiStore<float>{(float*)r.out, r.ldc, (const float*)r.bias, r.accumulate}, st);
        case EPI_BIAS_GELU: return f32_launch<LA, LB>(r, EpiBiasGelu<float>{(float*)r.out, (float*)r.out2, r.ldc, (const float*)r.bias}, st);
        case EPI_DGELU: return f32_launch<LA, LB>(r, EpiDGelu<float>{(float*)r.out, (const float*)r.aux, r.ldc}, st);
    }
    return hipErrorInvalidValue;
}

hipError_t gemm_f32(const GemmReq& r, hipStream_t st) {
    if (!r.a_mn && r.b_mn) return f32_run<KCONTIG, MNCONTIG>(r, st);
    if (!r.a_mn && !r.b_mn) return f32_run<KCONTIG, KCONTIG>(r, st);
    if (r.a_mn && r.b_mn) return f32_run<MNCONTIG, MNCONTIG>(r, st);
    return hipErrorInvalidValue;
}

}  // namespace tp
