// bf16 GEMM, both operands K-contiguous (input gradients G W^T, and the vocabulary logits E_r X^T).
#include "gemm_dispatch.h"
namespace tp {
hipError_t gemm_bf16_nt(const GemmReq& r, const GemmPlan& p, void* ws, hipStream_t st) {
    return gemm_run<KCONTIG, KCONTIG,
                    (1 << EPI_STORE) | (1 << EPI_DGELU) | (1 << EPI_STORE_T) | (1 << EPI_XENT) |
                        (1 << EPI_XENT_GRAD)>(r, p, ws, st);
}
}  // namespace tp
