// fp8 (OCP E4M3) GEMM for gfx950: C[M,N] = descale_a * descale_b * sum_k A[m,k] B[n,k], both code
// matrices K-contiguous (A [M, K], B [N, K], row strides in bytes), fp32 accumulation,
// v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales.
//
// The tile machinery is the bf16 kernel's (gemm.h): a K tile is 128 codes deep, so one tile
// row is again 128 bytes and the DMA (buffer_load ... lds), the 16-byte chunk swizzle and the
// XCD-aware tile map carry over unchanged. What differs:
//   * an MFMA consumes 64 k per step: lane half h of the wave supplies 32 bytes, logical
//     chunks 4s + 2h and 4s + 2h + 1 of the row for step s (0, 1). A and B use the same
//     lane/byte -> k assignment, so the hardware's own ordering of k inside the instruction
//     cannot change the sum. Each chunk read is a conflict-free ds_read_b128 under the swizzle
//     (16 consecutive rows cover all 16 (row parity, chunk) bank groups).
//   * two MFMA steps per K tile instead of four.
//   * the per-tensor descales (powers of two written by the quantiser) multiply the fp32
//     accumulators before the shared epilogues run, so every epilogue sees dequantised values.
#include "gemm.h"
#include "launch.h"

namespace tp {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
// one MFMA operand: the lane's 32 bytes as two 16-byte LDS reads
struct Frag8 {
    i32x4 lo, hi;
};
constexpr int BK8 = 128;   // k codes per K tile (128 bytes per tile row)

template <int R, int NT> struct Operand8 {
    static constexpr int BYTES = R * 128;
    static constexpr int IPW = BYTES / 1024 / (NT / 64);
    static_assert(IPW >= 1 && BYTES % (1024 * (NT / 64)) == 0, "tile/threads mismatch");
    int a[4];   // [2*s + q]: byte offset of 16-byte half q of the lane's 32 bytes at step s
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int ld, int mn0, int MN, int k0, int K, int tid,
                                         char* lds) const {
        const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            const int blk = wave * IPW + j;
            const int c = blk * 64 + lane, row = c >> 3, p = c & 7;
            const int kc = p ^ ((row ^ (row >> 3)) & 7);
            const int mn = mn0 + row, k = k0 + kc * 16;
            dma16(rs, (mn < MN && k < K) ? mn * ld + k : kOOB, lds + blk * 1024);
        }
    }
    // rows row + 32i with i odd have the swizzle XOR 4, i.e. steps 0 and 1 trade places
    __device__ __forceinline__ void init(int row, int lane) {
        const int f = (row ^ (row >> 3)) & 7, h = lane >> 5;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int q = 0; q < 2; ++q) a[2 * s + q] = row * 128 + (((4 * s + 2 * h + q) ^ f) << 4);
    }
    __device__ __forceinline__ void frag(const char* lds, int i, int s, Frag8& f) const {
        const int ss = s ^ (i & 1);
        const char* base = lds + i * 32 * 128;
        f.lo = *(const i32x4*)(base + a[2 * ss]);
        f.hi = *(const i32x4*)(base + a[2 * ss + 1]);
    }
};

template <class C>
struct Gemm8State {
    Operand8<C::BM, C::NT> oa;
    Operand8<C::BN, C::NT> ob;
    __amdgpu_buffer_rsrc_t ra, rb;
    int lda, ldb, m0, n0, M, N, kbeg, kend, tid;
    Frag8 a0[C::TM], b0[C::TN], a1[C::TM], b1[C::TN];
};

template <class C, int ST>
__device__ __forceinline__ void read_frags8(const Gemm8State<C>& g, const char* smem, int s, Frag8 (&af)[C::TM],
                                            Frag8 (&bf)[C::TN]) {
    const char* As = smem + ST * C::A_BYTES;
    const char* Bs = smem + 2 * C::A_BYTES + ST * C::B_BYTES;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) g.oa.frag(As, i, s, af[i]);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) g.ob.frag(Bs, j, s, bf[j]);
}

// One K step of MFMAs, issued at raised wave priority (s_setprio 1, restored to 0 after) so the
// two waves sharing a SIMD fall out of phase instead of alternating MFMAs in lockstep.
template <class C>
__device__ __forceinline__ void mfma_step8(f32x16 (&acc)[C::TM][C::TN], const Frag8 (&af)[C::TM],
                                           const Frag8 (&bf)[C::TN]) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const i32x8 a = __builtin_shufflevector(af[i].lo, af[i].hi, 0, 1, 2, 3, 4, 5, 6, 7);
            const i32x8 b = __builtin_shufflevector(bf[j].lo, bf[j].hi, 0, 1, 2, 3, 4, 5, 6, 7);
            // formats 0/0: E4M3 x E4M3; scale bytes 127 = 2^0 (E8M0) for both operands
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i][j], 0, 0, 0, 127, 0, 127);
        }
    __builtin_amdgcn_s_setprio(0);
}

template <class C>
__device__ __forceinline__ void load_stage8(Gemm8State<C>& g, char* smem, int stage, int k0) {
    g.oa.load(g.ra, g.lda, g.m0, g.M, k0, g.kend, g.tid, smem + stage * C::A_BYTES);
    g.ob.load(g.rb, g.ldb, g.n0, g.N, k0, g.kend, g.tid, smem + 2 * C::A_BYTES + stage * C::B_BYTES);
}

// One K tile in LDS stage ST (fragments of its step 0 already in a0/b0); the next tile's DMA goes
// into the other stage at the start, its step-0 fragments are read after the barrier. The body
// is branch-free: after the last tile the "next" tile lies past kend, so its DMA fills the idle
// stage with zeros and the fragments read from it are never used. (With the loads and reads
// under a branch, the compiler sank the MFMAs below the barrier and doubled the fragment
// registers.)
template <class C, int ST>
__device__ __forceinline__ void gemm8_tile(Gemm8State<C>& g, char* smem, f32x16 (&acc)[C::TM][C::TN], int kt) {
    constexpr int NR = 2 * (C::TM + C::TN), NM = C::TM * C::TN;
    load_stage8(g, smem, ST ^ 1, g.kbeg + (kt + 1) * BK8);
    read_frags8<C, ST>(g, smem, 1, g.a1, g.b1);
    mfma_step8<C>(acc, g.a0, g.b0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, NR, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, NM, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step8<C>(acc, g.a1, g.b1);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    read_frags8<C, ST ^ 1>(g, smem, 0, g.a0, g.b0);
}

template <class C, class Epi>
__global__ __launch_bounds__(C::NT, 1) void gemm_fp8_kernel(const uint8_t* __restrict__ A, int lda,
                                                            const uint8_t* __restrict__ B, int ldb,
                                                            const float* __restrict__ descale_a,
                                                            const float* __restrict__ descale_b, int M, int N, int K,
                                                            int k_per_split, uint32_t a_bytes, uint32_t b_bytes,
                                                            Epi epi) {
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WGN, wn = wave % C::WGN;
    const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = (N + C::BN - 1) / C::BN;
    int tm, tn;
    map_tile(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    Epi ep = epi;
    ep.set_split(blockIdx.y);

    Gemm8State<C> g;
    g.ra = make_rsrc(A, a_bytes);
    g.rb = make_rsrc(B, b_bytes);
    g.lda = lda; g.ldb = ldb;
    g.m0 = tm * C::BM; g.n0 = tn * C::BN;
    g.M = M; g.N = N;
    g.kbeg = blockIdx.y * k_per_split;
    g.kend = min(K, g.kbeg + k_per_split);
    g.tid = tid;
    g.oa.init(wm * C::WM + (lane & 31), lane);
    g.ob.init(wn * C::WN + (lane & 31), lane);

    f32x16 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int nk = g.kend > g.kbeg ? (g.kend - g.kbeg + BK8 - 1) / BK8 : 0;
    if (nk > 0) load_stage8(g, smem, 0, g.kbeg);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (nk > 0) read_frags8<C, 0>(g, smem, 0, g.a0, g.b0);
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        gemm8_tile<C, 0>(g, smem, acc, kt);
        gemm8_tile<C, 1>(g, smem, acc, kt + 1);
    }
    if (kt < nk) gemm8_tile<C, 0>(g, smem, acc, kt);
    // both descales are powers of two: the product and the scaling are exact
    const float ds = descale_a[0] * descale_b[0];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] *= ds;
    ep.template apply<C>(acc, g.m0, g.n0, g.m0 + wm * C::WM, g.n0 + wn * C::WN, lane, M, N, smem);
}

template <class C, class Epi>
static hipError_t launch8(const GemmReq& r, int splits, const Epi& e, hipStream_t st) {
    const int tiles = ((r.M + C::BM - 1) / C::BM) * ((r.N + C::BN - 1) / C::BN);
    if (tiles == 0) return hipSuccess;
    const int kps = ((r.K + splits - 1) / splits + BK8 - 1) / BK8 * BK8;
    const size_t a_bytes = (size_t)r.M * r.lda, b_bytes = (size_t)r.N * r.ldb;
    if (a_bytes >= (size_t)kOOB || b_bytes >= (size_t)kOOB) return hipErrorInvalidValue;
    if (Epi::kVec8 && (r.N % 8 != 0 || r.ldc % 8 != 0)) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_fp8_kernel<C, Epi>), dim3(tiles, splits), dim3(C::NT), 0, st, (const uint8_t*)r.A, r.lda,
                       (const uint8_t*)r.B, r.ldb, r.descale_a, r.descale_b, r.M, r.N, r.K, kps, (uint32_t)a_bytes,
                       (uint32_t)b_bytes, e);
    return hipGetLastError();
}

template <class Epi>
static hipError_t launch8_plan(const GemmReq& r, const GemmPlan& p, const Epi& e, hipStream_t st) {
    switch (p.cfg) {
        case 1: return launch8<Cfg128x128>(r, p.splits, e, st);
        case 2: return launch8<Cfg256x192>(r, p.splits, e, st);
    }
    return hipErrorInvalidValue;
}

hipError_t gemm_fp8(const GemmReq& r, const GemmPlan& p, void* ws, hipStream_t st) {
    if (r.M == 0 || r.N == 0) return hipSuccess;
    if (r.a_mn || r.b_mn) return hipErrorInvalidValue;
    if (p.splits > 1) {
        if (r.epi != EPI_STORE || ws == nullptr) return hipErrorInvalidValue;
        EpiPartial e{(float*)ws, r.N, (size_t)r.M * r.N, 0};
        hipError_t err = launch8_plan(r, p, e, st);
        if (err != hipSuccess) return err;
        EpiStore<bf16> fin{(bf16*)r.out, r.ldc, (const bf16*)r.bias, r.accumulate};
        const size_t n = (size_t)r.M * r.N;
        const unsigned nsk = (unsigned)((n / 8 + 255) / 256);
        hipLaunchKernelGGL((splitk_reduce_kernel<EpiStore<bf16>>), dim3(nsk), dim3(256), 0, st, (const float*)ws,
                           p.splits, n, r.M, r.N, fin, ColSumJob{nullptr, nullptr, 0, 0, 0}, (int)nsk);
        return hipGetLastError();
    }
    switch (r.epi) {
        case EPI_STORE:
            return launch8_plan(r, p, EpiStore<bf16>{(bf16*)r.out, r.ldc, (const bf16*)r.bias, r.accumulate}, st);
        case EPI_BIAS_GELU:
            return launch8_plan(r, p, EpiBiasGelu<bf16>{(bf16*)r.out, (bf16*)r.out2, r.ldc, (const bf16*)r.bias}, st);
        case EPI_DGELU:
            return launch8_plan(r, p, EpiDGelu<bf16>{(bf16*)r.out, (const bf16*)r.aux, r.ldc}, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace tp
