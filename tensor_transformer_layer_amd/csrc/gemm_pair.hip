// Paired launch of two independent bf16 GEMMs that each leave most of the chip idle: the attention
// backward's dO = G Wo_r^T (both operands K-contiguous, plain store) and dWo_r = O_r^T G (both
// MN-contiguous, split over K into fp32 partials, then reduced in split order), on 128x128 tiles
// with two workgroups per CU.
#include "gemm_dispatch.h"

namespace tp {

static constexpr int kPairSlots = 2 * 256;   // resident 128x128 workgroups: two per CU

bool plan_gemm_pair(const GemmReq& r1, const GemmReq& r2, int& splits2) {
    typedef Cfg128x128 C;
    if (r1.a_mn || r1.b_mn || !r2.a_mn || !r2.b_mn) return false;
    if (r1.epi != EPI_STORE || r1.accumulate || r1.bias || r2.epi != EPI_STORE || r2.bias) return false;
    if (r1.M <= 0 || r1.N <= 0 || r1.K <= 0 || r2.M <= 0 || r2.N <= 0 || r2.K <= 0) return false;
    if (r1.N % 8 || r1.ldc % 8 || r2.N % 8 || r2.ldc % 8) return false;
    const long n1 = (long)cdiv_h(r1.M, C::BM) * cdiv_h(r1.N, C::BN);
    const long t2 = (long)cdiv_h(r2.M, C::BM) * cdiv_h(r2.N, C::BN);
    if (n1 > kPairSlots / 2) return false;   // the first GEMM alone fills the CUs
    static const int opts[] = {8, 6, 4, 3, 2};
    const int k1 = cdiv_h(r1.K, C::BK);
    for (int s : opts) {
        if (n1 + t2 * s > kPairSlots || r2.K / s < 512) continue;
        // per-unit K tiles of the two GEMMs within 2x of each other, so neither part's units
        // outlast the other's by much
        const int k2 = cdiv_h(cdiv_h(r2.K, s), C::BK);
        if (k1 > 2 * k2 || k2 > 2 * k1) continue;
        splits2 = s;
        return true;
    }
    return false;
}

hipError_t gemm_bf16_pair(const GemmReq& r1, const GemmReq& r2, int splits2, void* ws2, hipStream_t st) {
    typedef Cfg128x128 C;
    if (splits2 < 2 || ws2 == nullptr) return hipErrorInvalidValue;
    const size_t a1 = (size_t)r1.M * r1.lda * 2, b1 = (size_t)r1.N * r1.ldb * 2;
    const size_t a2 = (size_t)r2.K * r2.lda * 2, b2 = (size_t)r2.K * r2.ldb * 2;
    if (a1 >= (size_t)kOOB || b1 >= (size_t)kOOB || a2 >= (size_t)kOOB || b2 >= (size_t)kOOB) return hipErrorInvalidValue;
    GemmArgs<EpiStore<bf16>> p{(const bf16*)r1.A, r1.lda, (const bf16*)r1.B, r1.ldb, r1.M, r1.N, r1.K,
                               cdiv_h(r1.K, C::BK) * C::BK, (uint32_t)a1, (uint32_t)b1,
                               EpiStore<bf16>{(bf16*)r1.out, r1.ldc, nullptr, 0}};
    GemmArgs<EpiPartial> q{(const bf16*)r2.A, r2.lda, (const bf16*)r2.B, r2.ldb, r2.M, r2.N, r2.K,
                           cdiv_h(cdiv_h(r2.K, splits2), C::BK) * C::BK, (uint32_t)a2, (uint32_t)b2,
                           EpiPartial{(float*)ws2, r2.N, (size_t)r2.M * r2.N, 0}};
    const int n1 = cdiv_h(r1.M, C::BM) * cdiv_h(r1.N, C::BN);
    const int n2 = cdiv_h(r2.M, C::BM) * cdiv_h(r2.N, C::BN) * splits2;
    hipLaunchKernelGGL((gemm_bf16_pair_kernel<C, KCONTIG, KCONTIG, EpiStore<bf16>, MNCONTIG, MNCONTIG, EpiPartial>),
                       dim3(n1 + n2), dim3(C::NT), 0, st, p, q, n1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_splitk_reduce(r2, GemmPlan{1, splits2, C::BM, C::BN}, ws2, st);
}

}  // namespace tp
