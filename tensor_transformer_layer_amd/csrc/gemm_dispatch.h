// Instantiation helper for the bf16 GEMM: plan -> tile configuration -> epilogue -> launch.
// Included by the per-layout translation units only.
#pragma once
#include "gemm.h"
#include "launch.h"
#include "xent.h"

namespace tp {

static inline int cdiv_h(long a, long b) { return (int)((a + b - 1) / b); }

// out = sum of the split partials in ws, in split order, through the plain bf16 store epilogue;
// the request's column-sum job (r.cs_out set), if any, rides along as extra blocks
static inline hipError_t launch_splitk_reduce(const GemmReq& r, const GemmPlan& p, const void* ws, hipStream_t st) {
    EpiStore<bf16> fin{(bf16*)r.out, r.ldc, (const bf16*)r.bias, r.accumulate};
    size_t n = (size_t)r.M * r.N;
    if (n == 0 || p.splits <= 1) return hipSuccess;
    const unsigned nsk = (unsigned)((n / 8 + 255) / 256);
    ColSumJob cj{r.cs_part, r.cs_out, r.cs_nb, r.cs_n, r.cs_accumulate};
    const unsigned ncs = r.cs_out ? (unsigned)((r.cs_n + RR_COLS - 1) / RR_COLS) : 0u;
    if (r.cs_out && r.cs_n % 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL((splitk_reduce_kernel<EpiStore<bf16>>), dim3(nsk + ncs), dim3(256), 0, st, (const float*)ws,
                       p.splits, n, r.M, r.N, fin, cj, (int)nsk);
    return hipGetLastError();
}

template <class C, int LA, int LB, class Epi>
static hipError_t launch_cfg(const GemmReq& r, int splits, const Epi& e, hipStream_t st) {
    int tiles = cdiv_h(r.M, C::BM) * cdiv_h(r.N, C::BN);
    if (tiles == 0) return hipSuccess;
    int kps = cdiv_h(cdiv_h(r.K, splits), C::BK) * C::BK;
    // bytes addressable through each operand (buffer loads beyond them return 0)
    size_t a_bytes = (size_t)(LA == KCONTIG ? r.M : r.K) * r.lda * 2;
    size_t b_bytes = (size_t)(LB == KCONTIG ? r.N : r.K) * r.ldb * 2;
    if (a_bytes >= (size_t)kOOB || b_bytes >= (size_t)kOOB) return hipErrorInvalidValue;
    // vector epilogues move 8 columns at a time
    if (Epi::kVec8 && (r.N % 8 != 0 || r.ldc % 8 != 0)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_bf16_kernel<C, LA, LB, Epi>), dim3(tiles * splits), dim3(C::NT), 0, st,
                       (const bf16*)r.A, r.lda, (const bf16*)r.B, r.ldb, r.M, r.N, r.K, kps, (uint32_t)a_bytes,
                       (uint32_t)b_bytes, e);
    return hipGetLastError();
}

template <int LA, int LB, class Epi>
static hipError_t launch_plan(const GemmReq& r, const GemmPlan& p, const Epi& e, hipStream_t st) {
    switch (p.cfg) {
        case 0: return launch_cfg<Cfg256x256, LA, LB>(r, p.splits, e, st);
        case 1: return launch_cfg<Cfg128x128, LA, LB>(r, p.splits, e, st);
        case 2: return launch_cfg<Cfg256x192, LA, LB>(r, p.splits, e, st);
        // multi-stage shapes need both operands on DMA; other layouts take the two-stage 128x128
        case 3:
            if constexpr (LA == KCONTIG && LB == KCONTIG) return launch_cfg<Cfg64x64s4, LA, LB>(r, p.splits, e, st);
            else return launch_cfg<Cfg128x128, LA, LB>(r, p.splits, e, st);
        case 4:
            if constexpr (LA == KCONTIG && LB == KCONTIG) return launch_cfg<Cfg128x128s3, LA, LB>(r, p.splits, e, st);
            else return launch_cfg<Cfg128x128, LA, LB>(r, p.splits, e, st);
    }
    return hipErrorInvalidValue;
}

// kinds: bit mask of the EpiKinds this layout instantiates.
template <int LA, int LB, int KINDS>
static hipError_t gemm_run(const GemmReq& r, const GemmPlan& p, void* ws, hipStream_t st) {
    if (p.splits > 1) {
        if constexpr ((KINDS & (1 << EPI_STORE)) != 0) {
            if (r.epi != EPI_STORE || ws == nullptr) return hipErrorInvalidValue;
            EpiPartial e{(float*)ws, r.N, (size_t)r.M * r.N, 0};
            hipError_t err = launch_plan<LA, LB>(r, p, e, st);
            if (err != hipSuccess) return err;
            return launch_splitk_reduce(r, p, ws, st);
        }
        return hipErrorInvalidValue;
    }
    switch (r.epi) {
        case EPI_STORE:
            if constexpr ((KINDS & (1 << EPI_STORE)) != 0)
                return launch_plan<LA, LB>(r, p, EpiStore<bf16>{(bf16*)r.out, r.ldc, (const bf16*)r.bias, r.accumulate}, st);
            break;
        case EPI_BIAS_GELU:
            if constexpr ((KINDS & (1 << EPI_BIAS_GELU)) != 0)
                return launch_plan<LA, LB>(r, p, EpiBiasGelu<bf16>{(bf16*)r.out, (bf16*)r.out2, r.ldc, (const bf16*)r.bias}, st);
            break;
        case EPI_DGELU:
            if constexpr ((KINDS & (1 << EPI_DGELU)) != 0)
                return launch_plan<LA, LB>(r, p, EpiDGelu<bf16>{(bf16*)r.out, (const bf16*)r.aux, r.ldc, r.colpart}, st);
            break;
        case EPI_STORE_T:
            if constexpr ((KINDS & (1 << EPI_STORE_T)) != 0)
                return launch_plan<LA, LB>(r, p, EpiStoreT<float>{(float*)r.out, r.ldc}, st);
            break;
        case EPI_XENT:
            if constexpr ((KINDS & (1 << EPI_XENT)) != 0)
                return launch_plan<LA, LB>(r, p, EpiXent{(XentPartial*)r.out, r.targets, r.col0, r.Vreal, r.mask, r.row0}, st);
            break;
        case EPI_XENT_GRAD:
            if constexpr ((KINDS & (1 << EPI_XENT_GRAD)) != 0) {
                if (r.ldc % 8 != 0 || r.ldc < r.N || r.ld2 % 4 != 0) return hipErrorInvalidValue;
                return launch_plan<LA, LB>(r, p, EpiXentGrad{(bf16*)r.out, r.ldc, (bf16*)r.out2, r.ld2, r.stat_m,
                                                             r.stat_s, r.dloss, r.targets, r.col0, r.Vreal, r.mask},
                                           st);
            }
            break;
    }
    return hipErrorInvalidValue;
}

}  // namespace tp
