// bf16 GEMM, A K-contiguous x B MN-contiguous (forward projections: X W with W [K, N]).
#include "gemm_dispatch.h"
namespace tp {
hipError_t gemm_bf16_nn(const GemmReq& r, const GemmPlan& p, void* ws, hipStream_t st) {
    return gemm_run<KCONTIG, MNCONTIG, (1 << EPI_STORE) | (1 << EPI_BIAS_GELU)>(r, p, ws, st);
}
}  // namespace tp
