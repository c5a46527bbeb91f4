// GEMM core for gfx950: C[M,N] = sum_k A(m,k) B(k,n), fp32 accumulation, fused epilogues.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 on LDS-staged, double-buffered 64-deep K tiles.
//   * Each operand is either K-contiguous (element (mn,k) at p[mn*ld + k]) or MN-contiguous
//     (element (mn,k) at p[k*ld + mn]). Both are stored in LDS K-contiguous, in 16-byte chunks
//     of 8 k-values, so every MFMA fragment is one 128-bit LDS read per lane. MN-contiguous tiles
//     are transposed in registers (8x8 or 4x8 blocks of bf16) between the global load and the
//     LDS store; nothing is transposed in HBM.
//   * LDS chunk index is XOR-swizzled with the row so that the 8 rows a wave reads (MFMA A/B
//     fragments) and the 8 rows a transposing thread group writes land in distinct banks.
//   * Global loads of tile k+1 are issued before the MFMAs of tile k and written to the other
//     LDS buffer after them: one barrier per K tile.
//   * Tiles are mapped XCD-aware: consecutive workgroups go round-robin to the 8 XCDs, so the
//     block id is remapped to give each XCD a contiguous, grouped range of output tiles that
//     share A and B panels in that XCD's L2.
// fp32 path (used for the fp32 MLP workload, which needs true fp32 products): LDS-tiled SIMT
//   FMA, 64x64 tiles, 4x4 outputs per thread.
//
// Accumulator layout of one 32x32 MFMA tile (lane l, register v):
//   column = l % 32, row = 8*(v/4) + 4*(l/32) + (v%4).
#pragma once
#include "common.h"

namespace tp {

enum Layout { KCONTIG = 0, MNCONTIG = 1 };

template <int BM_, int BN_, int WGM_, int WGN_>
struct GemmCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 64;
    static constexpr int WGM = WGM_, WGN = WGN_;
    static constexpr int NW = WGM * WGN, NT = 64 * NW;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int TM = WM / 32, TN = WN / 32;
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = 2 * STAGE;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
};

typedef GemmCfg<256, 256, 2, 2> Cfg256x256;
typedef GemmCfg<256, 128, 2, 2> Cfg256x128;
typedef GemmCfg<128, 256, 2, 2> Cfg128x256;
typedef GemmCfg<128, 128, 2, 2> Cfg128x128;

// Byte offset of 16-byte chunk kc (0..7) of tile row `row` (rows are 64 bf16 = 128 bytes).
__device__ __forceinline__ int lds_off(int row, int kc) {
    return row * 128 + ((kc ^ ((row ^ (row >> 3)) & 7)) << 4);
}

template <int R, int NT, int L> struct TileLoader;

// K-contiguous operand: R rows x 64 k, in 16-byte chunks.
template <int R, int NT> struct TileLoader<R, NT, KCONTIG> {
    static constexpr int CH = R * 8 / NT;
    static_assert(CH >= 1 && (R * 8) % NT == 0, "tile/threads mismatch");
    u32x4 v[CH];
    __device__ __forceinline__ void load(const bf16* __restrict__ p, int ld, int mn0, int MN, int k0, int K, int tid) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            int c = tid + i * NT, row = c >> 3, kc = c & 7;
            int mn = mn0 + row, k = k0 + kc * 8;
            if (mn < MN && k < K) v[i] = *(const u32x4*)(p + (size_t)mn * ld + k);
            else v[i] = u32x4{0, 0, 0, 0};
        }
    }
    __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            int c = tid + i * NT, row = c >> 3, kc = c & 7;
            *(u32x4*)(lds + lds_off(row, kc)) = v[i];
        }
    }
};

// MN-contiguous operand: each thread loads KB k-rows x 8 mn (16 bytes per row) and writes them
// transposed as 8 rows of KB k-values.
template <int R, int NT> struct TileLoader<R, NT, MNCONTIG> {
    static constexpr int EPT = R * 64 / NT;   // elements per thread
    static constexpr int KB = EPT / 8;        // k-rows per thread (8 or 4)
    static constexpr int MC = R / 8;          // 8-wide mn chunks across the tile
    static_assert(KB == 8 || KB == 4, "unsupported tile/threads ratio");
    static_assert(MC * (64 / KB) == NT, "thread mapping must cover the tile exactly");
    u32x4 v[KB];
    __device__ __forceinline__ void load(const bf16* __restrict__ p, int ld, int mn0, int MN, int k0, int K, int tid) {
        int mc = tid % MC, kg = tid / MC;
        int mn = mn0 + mc * 8;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            int k = k0 + kg * KB + j;
            if (mn < MN && k < K) v[j] = *(const u32x4*)(p + (size_t)k * ld + mn);
            else v[j] = u32x4{0, 0, 0, 0};
        }
    }
    __device__ __forceinline__ void store(char* lds, int tid) const {
        int mc = tid % MC, kg = tid / MC;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int dw = m >> 1;
            uint32_t o[KB / 2];
#pragma unroll
            for (int q = 0; q < KB / 2; ++q) {
                uint32_t a = v[2 * q][dw], b = v[2 * q + 1][dw];
                o[q] = (m & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
            }
            int row = mc * 8 + m;
            if constexpr (KB == 8) {
                *(u32x4*)(lds + lds_off(row, kg)) = u32x4{o[0], o[1], o[2], o[3]};
            } else {
                *(u32x2*)(lds + lds_off(row, kg >> 1) + ((kg & 1) << 3)) = u32x2{o[0], o[1]};
            }
        }
    }
};

// Block id -> output tile. XCD-aware: block i runs on XCD i % 8; give each XCD a contiguous
// slice of the tile sequence, walked in groups of GROUP_M tile-rows.
__device__ __forceinline__ void map_tile(int bid, int nblocks, int tiles_m, int tiles_n, int& tm, int& tn) {
    if ((nblocks & 7) == 0) bid = (bid & 7) * (nblocks >> 3) + (bid >> 3);
    const int GROUP_M = 4;
    int per_group = GROUP_M * tiles_n;
    int g = bid / per_group;
    int first_m = g * GROUP_M;
    int gsz = min(tiles_m - first_m, GROUP_M);
    int in = bid - g * per_group;
    tm = first_m + in % gsz;
    tn = in / gsz;
}

// ----------------------------------------------------------------------------------------------
// Epilogues. Elementwise ones expose op(row, col, value); the MFMA kernel calls apply().
// ----------------------------------------------------------------------------------------------
template <class C, class Op>
__device__ __forceinline__ void apply_elementwise(const Op& op, f32x16 (&acc)[C::TM][C::TN], int mw0, int nw0,
                                                  int lane, int M, int N) {
    const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
        int col = nw0 + j * 32 + l32;
        if (col >= N) continue;
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                int row = mw0 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                if (row < M) op(row, col, acc[i][j][v]);
            }
            // one 32x32 tile at a time: keeps the scheduler from hoisting every tile's loads
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// out[r*ld + c] = v (+ bias[c]) (+ out[r*ld + c] if accumulate)
template <typename T> struct EpiStore {
    __device__ __forceinline__ void set_split(int) {}
    T* out; int ld; const T* bias; int accumulate;
    __device__ __forceinline__ void operator()(int r, int c, float v) const {
        if (bias) v += to_f32(bias[c]);
        T* p = out + (size_t)r * ld + c;
        if (accumulate) v += to_f32(*p);
        *p = from_f32<T>(v);
    }
    template <class C> __device__ __forceinline__ void apply(f32x16 (&acc)[C::TM][C::TN], int, int, int mw0, int nw0,
                                                            int lane, int M, int N, char*) const {
        apply_elementwise<C>(*this, acc, mw0, nw0, lane, M, N);
    }
};

// out[c*ld + r] = v  (transposed store; fp32 logits of the vocab shard)
template <typename T> struct EpiStoreT {
    __device__ __forceinline__ void set_split(int) {}
    T* out; int ld;
    __device__ __forceinline__ void operator()(int r, int c, float v) const { out[(size_t)c * ld + r] = from_f32<T>(v); }
    template <class C> __device__ __forceinline__ void apply(f32x16 (&acc)[C::TM][C::TN], int, int, int mw0, int nw0,
                                                            int lane, int M, int N, char*) const {
        apply_elementwise<C>(*this, acc, mw0, nw0, lane, M, N);
    }
};

// U = v + bias; Y = GeLU(U)
template <typename T> struct EpiBiasGelu {
    __device__ __forceinline__ void set_split(int) {}
    T* U; T* Y; int ld; const T* bias;
    __device__ __forceinline__ void operator()(int r, int c, float v) const {
        if (bias) v += to_f32(bias[c]);
        size_t o = (size_t)r * ld + c;
        U[o] = from_f32<T>(v);
        Y[o] = from_f32<T>(gelu_f(v));
    }
    template <class C> __device__ __forceinline__ void apply(f32x16 (&acc)[C::TM][C::TN], int, int, int mw0, int nw0,
                                                            int lane, int M, int N, char*) const {
        apply_elementwise<C>(*this, acc, mw0, nw0, lane, M, N);
    }
};

// dU = v * GeLU'(U)
template <typename T> struct EpiDGelu {
    __device__ __forceinline__ void set_split(int) {}
    T* dU; const T* U; int ld;
    __device__ __forceinline__ void operator()(int r, int c, float v) const {
        size_t o = (size_t)r * ld + c;
        dU[o] = from_f32<T>(v * gelu_grad_f(to_f32(U[o])));
    }
    template <class C> __device__ __forceinline__ void apply(f32x16 (&acc)[C::TM][C::TN], int, int, int mw0, int nw0,
                                                            int lane, int M, int N, char*) const {
        apply_elementwise<C>(*this, acc, mw0, nw0, lane, M, N);
    }
};

// Split-K partial: part[split][r*ld + c] = v (fp32). Reduced later in split order.
struct EpiPartial {
    float* part; int ld; size_t split_stride;
    int split;
    __device__ __forceinline__ void set_split(int s) { split = s; }
    __device__ __forceinline__ void operator()(int r, int c, float v) const {
        part[(size_t)split * split_stride + (size_t)r * ld + c] = v;
    }
    template <class C> __device__ __forceinline__ void apply(f32x16 (&acc)[C::TM][C::TN], int, int, int mw0, int nw0,
                                                            int lane, int M, int N, char*) const {
        apply_elementwise<C>(*this, acc, mw0, nw0, lane, M, N);
    }
};

// ----------------------------------------------------------------------------------------------
// bf16 MFMA kernel. gridDim.x = output tiles; gridDim.y = K splits (each covers k_per_split).
// ----------------------------------------------------------------------------------------------
template <class C, int LA, int LB, class Epi>
__global__ __launch_bounds__(C::NT, 1) void gemm_bf16_kernel(const bf16* __restrict__ A, int lda,
                                                             const bf16* __restrict__ B, int ldb,
                                                             int M, int N, int K, int k_per_split, Epi epi) {
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WGN, wn = wave % C::WGN;
    const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = (N + C::BN - 1) / C::BN;
    int tm, tn;
    map_tile(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * C::BM, n0 = tn * C::BN;
    const int kbeg = blockIdx.y * k_per_split;
    const int kend = min(K, kbeg + k_per_split);
    Epi ep = epi;
    ep.set_split(blockIdx.y);

    TileLoader<C::BM, C::NT, LA> la;
    TileLoader<C::BN, C::NT, LB> lb;
    f32x16 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int nk = (kend - kbeg + C::BK - 1) / C::BK;
    if (nk > 0) {
        la.load(A, lda, m0, M, kbeg, kend, tid);
        lb.load(B, ldb, n0, N, kbeg, kend, tid);
        la.store(smem, tid);
        lb.store(smem + C::A_BYTES, tid);
    }
    __syncthreads();
    const int arow = wm * C::WM + (lane & 31);
    const int brow = wn * C::WN + (lane & 31);
    const int khalf = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        char* cur = smem + (kt & 1) * C::STAGE;
        const bool more = kt + 1 < nk;
        if (more) {
            int k0 = kbeg + (kt + 1) * C::BK;
            la.load(A, lda, m0, M, k0, kend, tid);
            lb.load(B, ldb, n0, N, k0, kend, tid);
        }
#pragma unroll
        for (int s = 0; s < C::BK / 16; ++s) {
            bf16x8 af[C::TM], bfr[C::TN];
#pragma unroll
            for (int i = 0; i < C::TM; ++i) af[i] = *(const bf16x8*)(cur + lds_off(arow + i * 32, 2 * s + khalf));
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
                bfr[j] = *(const bf16x8*)(cur + C::A_BYTES + lds_off(brow + j * 32, 2 * s + khalf));
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            char* nxt = smem + ((kt + 1) & 1) * C::STAGE;
            la.store(nxt, tid);
            lb.store(nxt + C::A_BYTES, tid);
        }
        __syncthreads();
    }
    ep.template apply<C>(acc, m0, n0, m0 + wm * C::WM, n0 + wn * C::WN, lane, M, N, smem);
}

// ----------------------------------------------------------------------------------------------
// fp32 SIMT kernel: 64x64 tile, BK = 16, 256 threads, 4x4 outputs per thread.
// ----------------------------------------------------------------------------------------------
template <int LA, int LB, class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int lda,
                                                       const float* __restrict__ B, int ldb,
                                                       int M, int N, int K, int k_per_split, Epi epi) {
    __shared__ float As[16][64 + 4];
    __shared__ float Bs[16][64 + 4];
    const int tid = threadIdx.x;
    const int tiles_n = (N + 63) / 64;
    const int m0 = (blockIdx.x / tiles_n) * 64, n0 = (blockIdx.x % tiles_n) * 64;
    const int kbeg = blockIdx.y * k_per_split, kend = min(K, kbeg + k_per_split);
    Epi ep = epi;
    ep.set_split(blockIdx.y);
    const int ty = tid / 16, tx = tid % 16;
    float acc[4][4] = {};
    for (int k0 = kbeg; k0 < kend; k0 += 16) {
        // 64 x 16 elements of each operand, 4 per thread
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int e = tid + i * 256;
            int mn, k;
            if (LA == KCONTIG) { mn = e / 16; k = e % 16; } else { k = e / 64; mn = e % 64; }
            int gm = m0 + mn, gk = k0 + k;
            float va = 0.f;
            if (gm < M && gk < kend) va = (LA == KCONTIG) ? A[(size_t)gm * lda + gk] : A[(size_t)gk * lda + gm];
            As[k][mn] = va;
            if (LB == KCONTIG) { mn = e / 16; k = e % 16; } else { k = e / 64; mn = e % 64; }
            int gn = n0 + mn;
            gk = k0 + k;
            float vb = 0.f;
            if (gn < N && gk < kend) vb = (LB == KCONTIG) ? B[(size_t)gn * ldb + gk] : B[(size_t)gk * ldb + gn];
            Bs[k][mn] = vb;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int r = m0 + ty * 4 + i, c = n0 + tx * 4 + j;
            if (r < M && c < N) ep(r, c, acc[i][j]);
        }
}

// Split-K reduction: out = epi(sum_{s=0}^{splits-1} part[s][r*ld + c]) in split order.
template <class Epi>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits,
                                                            size_t split_stride, int M, int N, int ld, Epi epi) {
    size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)M * N) return;
    int r = (int)(idx / N), c = (int)(idx % N);
    size_t o = (size_t)r * ld + c;
    float acc = 0.f;
    for (int s = 0; s < splits; ++s) acc += part[(size_t)s * split_stride + o];
    epi(r, c, acc);
}

}  // namespace tp
