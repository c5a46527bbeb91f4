// bf16 GEMM, both operands MN-contiguous (weight gradients X^T dY over the token dimension).
#include "gemm_dispatch.h"
namespace tp {
hipError_t gemm_bf16_tn(const GemmReq& r, const GemmPlan& p, void* ws, hipStream_t st) {
    return gemm_run<MNCONTIG, MNCONTIG, (1 << EPI_STORE)>(r, p, ws, st);
}
}  // namespace tp
