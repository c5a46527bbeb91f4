// GEMM core for gfx950: C[M,N] = sum_k A(m,k) B(k,n), fp32 accumulation, fused epilogues.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 on LDS-staged, double-buffered 64-deep K tiles.
//   * Each operand is either K-contiguous (element (mn,k) at p[mn*ld + k]) or MN-contiguous
//     (element (mn,k) at p[k*ld + mn]). Both are held in LDS as [R rows][64 k], 128-byte rows,
//     16-byte chunk kc stored at kc ^ ((row ^ row/8) & 7), so every MFMA fragment is one
//     conflict-free 128-bit LDS read per lane:
//       - K-contiguous tiles go from global memory straight into LDS (buffer_load ... lds, no
//         staging registers);
//       - MN-contiguous tiles are fetched into registers (8 k-rows x 8 mn per thread),
//         transposed there with byte permutes and written to LDS. (Keeping them MN-major in LDS
//         and reading with the transposing ds_read_b64_tr_b16 was measured slower.)
//     Nothing is transposed in HBM.
//   * Out-of-range chunks (rows past the edge, k past the end of this split) are fetched at an
//     offset past the buffer's end, which the buffer load returns as 0.
//   * Per-lane global offsets are computed once per output tile; each K tile's fetch is then one
//     load per 16-byte chunk with the K advance in the scalar offset (a ragged last K tile masks
//     its chunks per lane).
//   * The next K tile is fetched into the other LDS stage during the current one (at its start,
//     or behind its first MFMAs, see gemm_tile); fragments of k-step s+1 are read while the
//     MFMAs of k-step s run (order pinned with sched_group_barrier); one barrier per K tile.
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

// NS = LDS stages: 2 (double buffering), or more for configurations whose operands both go
// through DMA, where the loads of tile k + NS - 1 are in flight while tile k is multiplied.
template <int BM_, int BN_, int WGM_, int WGN_, int NS_ = 2>
struct GemmCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 64;
    static constexpr int WGM = WGM_, WGN = WGN_;
    static constexpr int NW = WGM * WGN, NT = 64 * NW;
    static constexpr int WM = BM / WGM, WN = BN / WGN;
    static constexpr int TM = WM / 32, TN = WN / 32;
    static constexpr int NS = NS_;
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int B_BASE = NS * A_BYTES;   // LDS: [A stage 0 .. NS-1 | B stage 0 .. NS-1]
    static constexpr int LDS = NS * STAGE;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(NS >= 2 && LDS <= 160 * 1024, "stages must fit the 160 KB of LDS");
};

// 256x256 and 256x192 with 8 waves (128x64 / 64x96 per wave, two waves per SIMD) and 128x128
// with 4 waves (64x64 per wave, two workgroups per CU): all keep two waves per SIMD to hide
// latency; the larger tiles cut LDS and L2 traffic per MFMA.
typedef GemmCfg<256, 256, 2, 4> Cfg256x256;
typedef GemmCfg<256, 192, 4, 2> Cfg256x192;   // 8 waves, 64x96 per wave: N = 1536 / 3072 / 1152 in whole tiles
typedef GemmCfg<128, 128, 2, 2> Cfg128x128;
// 64x64 with 4 waves of 32x32 and four LDS stages (32 KB each side: two workgroups per CU): for
// the thin remainder of a large GEMM, where few MFMAs per k-step leave the loads exposed
typedef GemmCfg<64, 64, 2, 2, 4> Cfg64x64s4;
// 128x128 with three stages (96 KB: one workgroup per CU) for GEMMs with about one such tile per
// CU, where a single workgroup must hide the loads itself
typedef GemmCfg<128, 128, 2, 2, 3> Cfg128x128s3;

// Buffer resource over [base, base + bytes): loads at offsets >= bytes return 0, which is how
// masked chunks are zero-filled without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Offset of a masked chunk: at or past the end of every buffer (launches keep operands below it)
// and far enough below 2^32 that adding a scalar K offset (< 2^31) cannot wrap.
constexpr int kOOB = 0x7f000000;

typedef __attribute__((address_space(3))) void lds_void;

// Byte offset of 16-byte chunk kc (0..7) of row `row` in a K-contiguous tile (128-byte rows).
__device__ __forceinline__ int lds_off(int row, int kc) {
    return row * 128 + ((kc ^ ((row ^ (row >> 3)) & 7)) << 4);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, int off, char* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, off, 0, 0, 0);
}

// One operand tile of R rows (M or N) x 64 k. load(): global -> LDS by 1 KB DMA instructions,
// lane L of an instruction landing at byte 16*L of its kilobyte. init()/frag(): per-lane
// fragment addresses (4 registers) and the MFMA operand of 32-row group i at 16-deep k-step s.
template <int R, int NT, int L> struct Operand;

template <int R, int NT> struct Operand<R, NT, KCONTIG> {
    static constexpr bool DMA = true;
    static constexpr int BYTES = R * 128;
    static constexpr int IPW = BYTES / 1024 / (NT / 64);
    static_assert(IPW >= 1 && BYTES % (1024 * (NT / 64)) == 0, "tile/threads mismatch");
    int a[4];
    int voff[IPW];   // byte offset of this lane's chunk at k0 = 0, or kOOB for rows past the edge
    int ldsb;        // the wave's first kilobyte in a stage (wave-uniform)
    // Once per tile: per-lane offsets, so each K tile's fetch is one DMA per kilobyte with the K
    // advance in the scalar offset.
    __device__ __forceinline__ void setup(int ld, int mn0, int MN, int tid) {
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
        ldsb = wave * IPW * 1024;
#pragma unroll
        for (int j = 0; j < IPW; ++j) {
            const int c = (wave * IPW + j) * 64 + lane, row = c >> 3;
            const int kc = (c & 7) ^ ((row ^ (row >> 3)) & 7);
            voff[j] = (mn0 + row < MN) ? ((mn0 + row) * ld + kc * 8) * 2 : kOOB;
        }
    }
    // DMA the K tile at k0 (k < K valid; a ragged last tile masks its chunks per lane).
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int k0, int K, int tid, char* lds) const {
        if (k0 + 64 <= K) {
#pragma unroll
            for (int j = 0; j < IPW; ++j) {
                const int vo = voff[j];
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + ldsb + j * 1024), 16, vo, k0 * 2, 0,
                                                         0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < IPW; ++j) {
                const int c = ldsb / 16 + j * 64 + (tid & 63), row = c >> 3;
                const int kc = (c & 7) ^ ((row ^ (row >> 3)) & 7);
                const int vo = (k0 + kc * 8 < K) ? voff[j] : kOOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + ldsb + j * 1024), 16, vo, k0 * 2, 0,
                                                         0);
            }
        }
    }
    // row = first row of the wave's 32-row groups + lane % 32; the swizzle of row + 32i differs
    // from row's by XOR 4 on the chunk, i.e. k-step s <-> s ^ 2 for odd i.
    __device__ __forceinline__ void init(int row, int lane) {
        const int f = (row ^ (row >> 3)) & 7, khalf = lane >> 5;
#pragma unroll
        for (int s = 0; s < 4; ++s) a[s] = row * 128 + (((khalf ^ f) & 1) << 4) + ((s ^ (f >> 1)) << 5);
    }
    __device__ __forceinline__ bf16x8 frag(const char* lds, int i, int s) const {
        return *(const bf16x8*)(lds + a[s ^ ((i & 1) << 1)] + i * 32 * 128);
    }
};

template <int R, int NT> struct Operand<R, NT, MNCONTIG> {
    // Register-staged: each thread fetches KB k-rows x 8 mn (16 bytes per row) and stores them
    // transposed into the K-contiguous, swizzled tile layout of Operand<KCONTIG> (8 or 4 k-values
    // per 16-byte or 8-byte LDS write), whose fragment reads are then used unchanged.
    static constexpr bool DMA = false;
    static constexpr int BYTES = R * 128;
    static constexpr int MC = R / 8;          // 8-wide mn chunks across the tile
    static constexpr int KB = (MC * 16 <= NT) ? 4 : 8;  // k-rows per thread: 4 when the threads suffice
    static constexpr int USED = MC * (64 / KB);         // threads that carry a block
    static constexpr int NLOAD = KB, NSTORE = 8;
    static_assert(USED <= NT, "thread mapping must cover the tile");
    Operand<R, NT, KCONTIG> kc;   // fragment addressing of the K-contiguous layout
    u32x4 v[KB];
    int voff;    // byte offset of this thread's first k-row at k0 = 0, or kOOB
    int ldb;     // row pitch in bytes
    __device__ __forceinline__ void setup(int ld, int mn0, int MN, int tid) {
        const int mc = tid % MC, kg = tid / MC, mn = mn0 + mc * 8;
        voff = (tid < USED && mn < MN) ? (kg * KB * ld + mn) * 2 : kOOB;
        ldb = ld * 2;
    }
    // k-row k0 + kg*KB + j of the tile: the thread's offset plus a scalar (k0 + j) * ld * 2
    __device__ __forceinline__ void fetch(__amdgpu_buffer_rsrc_t rs, int k0, int K, int tid) {
        const bool full = k0 + 64 <= K;
        const int kg = tid / MC;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            const int vo = (full || k0 + kg * KB + j < K) ? voff : kOOB;
            v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, (k0 + j) * ldb, 0);
        }
    }
    __device__ __forceinline__ void store(char* lds, int tid) const {
        if (USED < NT && tid >= USED) return;
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
    __device__ __forceinline__ void init(int row, int lane) { kc.init(row, lane); }
    __device__ __forceinline__ bf16x8 frag(const char* lds, int i, int s) const { return kc.frag(lds, i, s); }
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

// Split-K launches: block id -> (K split, output tile) over tiles x splits units in split-major
// order, each XCD taking a contiguous range of units. An XCD then works on one K range of a
// compact group of tiles, so the operand panels its L2 must hold are a third (for three splits)
// of what a tile-major order spread over all XCDs needs.
__device__ __forceinline__ void map_unit(int bid, int nblocks, int tiles_m, int tiles_n, int& tm, int& tn,
                                         int& split) {
    if ((nblocks & 7) == 0) bid = (bid & 7) * (nblocks >> 3) + (bid >> 3);
    const int tiles = tiles_m * tiles_n;
    split = bid / tiles;
    map_tile(bid - split * tiles, 1, tiles_m, tiles_n, tm, tn);   // nblocks = 1: no second remap
}

// ----------------------------------------------------------------------------------------------
// Epilogues. Each exposes op8(row, col, v[8]) for 8 consecutive columns of one row (col % 8 == 0,
// N and ld multiples of 8, checked at launch) and is applied through apply_staged(): a wave's
// accumulators go to LDS one 32-row strip at a time and come back row-major, so every auxiliary
// load and output store is a 16-byte vector access and a wave's store covers whole row segments.
// (In the MFMA layout a lane holds one column of four rows, which would mean 2-byte accesses.)
// ----------------------------------------------------------------------------------------------
template <class C> struct Staging {
    static constexpr int LD = C::WN + 8;    // floats per slab row: rows r and r + 4 fall in opposite bank halves
    static constexpr int SLAB = 32 * LD;    // floats per wave
    static constexpr int CPR = C::WN / 8;   // 8-column chunks per row
    static constexpr int CHUNKS = 32 * CPR;
    static_assert(SLAB * 4 * C::NW <= C::LDS, "epilogue staging exceeds the tile buffers");
    static_assert(CHUNKS % 64 == 0, "chunks must divide evenly over the wave");
};

template <class C, class Op>
__device__ __forceinline__ void apply_staged(const Op& op, f32x16 (&acc)[C::TM][C::TN], int mw0, int nw0, int lane,
                                             int wave, int M, int N, char* smem) {
    typedef Staging<C> S;
    float* slab = (float*)smem + wave * S::SLAB;
    const int h = lane >> 5, l32 = lane & 31;
    __syncthreads();   // every wave has read its last fragments out of the tile buffers
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) slab[(8 * (v >> 2) + 4 * h + (v & 3)) * S::LD + j * 32 + l32] = acc[i][j][v];
        // the slab is this wave's own and a wave's LDS accesses complete in order: no barrier
        // between writing a strip, reading it back and writing the next
#pragma unroll
        for (int q = 0; q < S::CHUNKS / 64; ++q) {
            const int c = q * 64 + lane, r = c / S::CPR, cc = c - r * S::CPR;
            const float* p = slab + r * S::LD + cc * 8;
            f32x4 lo = *(const f32x4*)p, hi = *(const f32x4*)(p + 4);
            float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const int row = mw0 + i * 32 + r, col = nw0 + cc * 8;
            if (row < M && col < N) op.op8(row, col, v);
        }
    }
}

// apply_staged that also sums, per column, the values the op stores (rounded to its output type
// OutT) over the tile's rows, and writes those sums as row m0 / BM of colpart [tiles_m][N]. After
// a strip's op8 calls each wave writes the stored values back over its slab and its lanes add the
// slab's columns (32 rows, in row order); the WGM waves sharing a column block are then added in
// wave-row order through LDS. Rows past M and columns past N count as zeros.
template <class C, class Op>
__device__ __forceinline__ void apply_staged_colsum(const Op& op, f32x16 (&acc)[C::TM][C::TN], int m0, int n0, int mw0,
                                                    int nw0, int lane, int wave, int M, int N, char* smem,
                                                    float* __restrict__ colpart) {
    typedef Staging<C> S;
    typedef typename Op::OutT OutT;
    constexpr int NCL = (C::WN + 63) / 64;   // slab columns per lane in the column pass
    static_assert(C::WGM * C::BN * 4 <= C::LDS, "column-sum exchange exceeds the tile buffers");
    float* slab = (float*)smem + wave * S::SLAB;
    const int h = lane >> 5, l32 = lane & 31;
    float cs[NCL];
#pragma unroll
    for (int j = 0; j < NCL; ++j) cs[j] = 0.f;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) slab[(8 * (v >> 2) + 4 * h + (v & 3)) * S::LD + j * 32 + l32] = acc[i][j][v];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < S::CHUNKS / 64; ++q) {
            const int c = q * 64 + lane, r = c / S::CPR, cc = c - r * S::CPR;
            float* p = slab + r * S::LD + cc * 8;
            f32x4 lo = *(const f32x4*)p, hi = *(const f32x4*)(p + 4);
            float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const int row = mw0 + i * 32 + r, col = nw0 + cc * 8;
            if (row < M && col < N) {
                op.op8(row, col, v);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = to_f32(from_f32<OutT>(v[e]));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = 0.f;
            }
            // a wave's LDS accesses complete in order: the column pass below reads these values
            *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
            *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
        }
#pragma unroll
        for (int j = 0; j < NCL; ++j) {
            const int col = lane + 64 * j;
            if (col < C::WN) {
#pragma unroll 8
                for (int r = 0; r < 32; ++r) cs[j] += slab[r * S::LD + col];
            }
        }
        __syncthreads();
    }
    const int wm = wave / C::WGN, wn = wave % C::WGN;
    float* red = (float*)smem;   // [WGM][BN]
#pragma unroll
    for (int j = 0; j < NCL; ++j) {
        const int col = lane + 64 * j;
        if (col < C::WN) red[wm * C::BN + wn * C::WN + col] = cs[j];
    }
    __syncthreads();
    for (int c = (int)threadIdx.x; c < C::BN; c += C::NT) {
        float sum = red[c];
#pragma unroll
        for (int w = 1; w < C::WGM; ++w) sum += red[w * C::BN + c];
        if (n0 + c < N) colpart[(size_t)(m0 / C::BM) * N + n0 + c] = sum;
    }
}

// Elementwise form, straight from the MFMA layout (used by the transposed store).
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

#define TP_STAGED_APPLY                                                                                         \
    template <class C>                                                                                          \
    __device__ __forceinline__ void apply(f32x16 (&acc)[C::TM][C::TN], int, int, int mw0, int nw0, int lane,    \
                                          int M, int N, char* smem) const {                                     \
        apply_staged<C>(*this, acc, mw0, nw0, lane, (int)(threadIdx.x >> 6), M, N, smem);                      \
    }

// out[r*ld + c] = v (+ bias[c]) (+ out[r*ld + c] if accumulate)
template <typename T> struct EpiStore {
    static constexpr bool kVec8 = true;
    __device__ __forceinline__ void set_split(int) {}
    T* out; int ld; const T* bias; int accumulate;
    __device__ __forceinline__ void operator()(int r, int c, float v) const {
        if (bias) v += to_f32(bias[c]);
        T* p = out + (size_t)r * ld + c;
        if (accumulate) v += to_f32(*p);
        *p = from_f32<T>(v);
    }
    __device__ __forceinline__ void op8(int r, int c, float (&v)[8]) const {
        T* p = out + (size_t)r * ld + c;
        if (bias) {
            float b[8];
            load8(bias + c, b);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += b[e];
        }
        if (accumulate) {
            float o[8];
            load8(p, o);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += o[e];
        }
        store8(p, v);
    }
    TP_STAGED_APPLY
};

// out[c*ld + r] = v  (transposed store; fp32 logits of the vocab shard)
template <typename T> struct EpiStoreT {
    static constexpr bool kVec8 = false;
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
    static constexpr bool kVec8 = true;
    __device__ __forceinline__ void set_split(int) {}
    T* U; T* Y; int ld; const T* bias;
    __device__ __forceinline__ void operator()(int r, int c, float v) const {
        if (bias) v += to_f32(bias[c]);
        size_t o = (size_t)r * ld + c;
        U[o] = from_f32<T>(v);
        Y[o] = from_f32<T>(gelu_f(v));
    }
    __device__ __forceinline__ void op8(int r, int c, float (&v)[8]) const {
        if (bias) {
            float b[8];
            load8(bias + c, b);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += b[e];
        }
        const size_t o = (size_t)r * ld + c;
        store8(U + o, v);
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = gelu_f(v[e]);
        store8(Y + o, y);
    }
    TP_STAGED_APPLY
};

// dU = v * GeLU'(U); with colpart, also the column sums of the stored dU per tile row
// (apply_staged_colsum)
template <typename T> struct EpiDGelu {
    static constexpr bool kVec8 = true;
    typedef T OutT;
    __device__ __forceinline__ void set_split(int) {}
    T* dU; const T* U; int ld;
    float* colpart = nullptr;
    __device__ __forceinline__ void operator()(int r, int c, float v) const {
        size_t o = (size_t)r * ld + c;
        dU[o] = from_f32<T>(v * gelu_grad_f(to_f32(U[o])));
    }
    __device__ __forceinline__ void op8(int r, int c, float (&v)[8]) const {
        const size_t o = (size_t)r * ld + c;
        float u[8];
        load8(U + o, u);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= gelu_grad_f(u[e]);
        store8(dU + o, v);
    }
    template <class C>
    __device__ __forceinline__ void apply(f32x16 (&acc)[C::TM][C::TN], int m0, int n0, int mw0, int nw0, int lane,
                                          int M, int N, char* smem) const {
        const int wave = (int)(threadIdx.x >> 6);
        if (colpart) apply_staged_colsum<C>(*this, acc, m0, n0, mw0, nw0, lane, wave, M, N, smem, colpart);
        else apply_staged<C>(*this, acc, mw0, nw0, lane, wave, M, N, smem);
    }
};

// Split-K partial: part[split][r*ld + c] = v (fp32). Reduced later in split order.
struct EpiPartial {
    static constexpr bool kVec8 = true;
    float* part; int ld; size_t split_stride;
    int split;
    __device__ __forceinline__ void set_split(int s) { split = s; }
    __device__ __forceinline__ void op8(int r, int c, float (&v)[8]) const {
        store8(part + (size_t)split * split_stride + (size_t)r * ld + c, v);
    }
    TP_STAGED_APPLY
};

// ----------------------------------------------------------------------------------------------
// bf16 MFMA kernel. gridDim.x = output tiles x K splits (each split covers k_per_split), see map_unit.
// LDS: [A stage 0 | A stage 1 | B stage 0 | B stage 1].
// ----------------------------------------------------------------------------------------------
template <class C, int LA, int LB>
struct GemmState {
    Operand<C::BM, C::NT, LA> oa;
    Operand<C::BN, C::NT, LB> ob;
    __amdgpu_buffer_rsrc_t ra, rb;
    int lda, ldb, m0, n0, M, N, kbeg, kend, tid;
    bf16x8 a0[C::TM], b0[C::TN], a1[C::TM], b1[C::TN];
};

template <class C, int LA, int LB, int ST>
__device__ __forceinline__ void read_frags(const GemmState<C, LA, LB>& g, const char* smem, int s, bf16x8 (&af)[C::TM],
                                           bf16x8 (&bf)[C::TN]) {
    const char* As = smem + ST * C::A_BYTES;
    const char* Bs = smem + C::B_BASE + ST * C::B_BYTES;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) af[i] = g.oa.frag(As, i, s);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) bf[j] = g.ob.frag(Bs, j, s);
}

// One k-step of MFMAs over the wave tile; PRIO: issued at raised wave priority (s_setprio 1,
// restored to 0 after).
template <class C, bool PRIO = false>
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[C::TM][C::TN], const bf16x8 (&af)[C::TM],
                                          const bf16x8 (&bf)[C::TN]) {
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
}

// Scheduling-group masks (AMDGPU sched_group_barrier): inside each k-step the next fragments'
// LDS reads issue before this k-step's MFMAs.
constexpr int SG_MFMA = 0x008, SG_DS_READ = 0x100;

// Issue the loads of the K tile at k0: DMA operands go straight into LDS stage `stage`,
// register-staged operands into their registers (written to LDS by store_stage()).
template <class C, int LA, int LB>
__device__ __forceinline__ void load_stage_dma(GemmState<C, LA, LB>& g, char* smem, int stage, int k0) {
    if constexpr (decltype(g.oa)::DMA) g.oa.load(g.ra, k0, g.kend, g.tid, smem + stage * C::A_BYTES);
    if constexpr (decltype(g.ob)::DMA) g.ob.load(g.rb, k0, g.kend, g.tid, smem + C::B_BASE + stage * C::B_BYTES);
}
template <class C, int LA, int LB>
__device__ __forceinline__ void load_stage_reg(GemmState<C, LA, LB>& g, int k0) {
    if constexpr (!decltype(g.oa)::DMA) g.oa.fetch(g.ra, k0, g.kend, g.tid);
    if constexpr (!decltype(g.ob)::DMA) g.ob.fetch(g.rb, k0, g.kend, g.tid);
}
template <class C, int LA, int LB>
__device__ __forceinline__ void load_stage(GemmState<C, LA, LB>& g, char* smem, int stage, int k0) {
    load_stage_dma(g, smem, stage, k0);
    load_stage_reg(g, k0);
}
template <class C, int LA, int LB>
__device__ __forceinline__ void store_stage(const GemmState<C, LA, LB>& g, char* smem, int stage) {
    if constexpr (!decltype(g.oa)::DMA) g.oa.store(smem + stage * C::A_BYTES, g.tid);
    if constexpr (!decltype(g.ob)::DMA) g.ob.store(smem + C::B_BASE + stage * C::B_BYTES, g.tid);
}

constexpr int SG_DS_WRITE = 0x200;

// One K tile held in LDS stage ST (fragments of its k-step 0 already in a0/b0). The next tile
// goes into the other stage, which was last read before the previous barrier: DMA operands at
// the start of this tile, register-staged ones after its third k-step.
template <class C, int LA, int LB, int ST>
__device__ __forceinline__ void gemm_tile(GemmState<C, LA, LB>& g, char* smem, f32x16 (&acc)[C::TM][C::TN], int kt,
                                          int nk) {
    constexpr int NR = C::TM + C::TN, NM = C::TM * C::TN;
    constexpr bool REG = !decltype(g.oa)::DMA || !decltype(g.ob)::DMA;
    constexpr int NDW = (decltype(g.oa)::DMA ? 0 : 8) + (decltype(g.ob)::DMA ? 0 : 8);
    const bool more = kt + 1 < nk;
    // DMA of the next tile: issued behind the first MFMAs (which then start right after the
    // barrier) when a register-staged operand is also in flight; first thing in the tile when
    // both operands go by DMA (measured on MI355X: those tiles need the longer lead; the 256x256
    // vocabulary tiles too since their MFMAs issue at raised priority, 256 -> 248 us)
    constexpr bool LATE = REG;
    // Barrier before the last k-step (see the end of the tile): not for the 256x256 tiles with two
    // register-staged operands (the extra live fragments spill) nor for the 256x192 and 128x128
    // tiles fed only by DMA (measured slower).
    constexpr bool BOTH_REG = !decltype(g.oa)::DMA && !decltype(g.ob)::DMA;
    constexpr bool EARLY_BARRIER = REG ? !(BOTH_REG && C::BM * C::BN >= 256 * 256) : C::BM * C::BN >= 256 * 256;
    // Each k-step's MFMAs issue at raised wave priority, so the two waves sharing a SIMD drift out
    // of phase (one multiplies while the other reads LDS) instead of alternating MFMAs in lockstep
    // (measured on MI355X: the 256x192 forward GEMMs 1-5 us faster each; the weight-gradient
    // tiles with both operands register-staged 1-2 us slower, so not for them). Not in the k-step
    // whose MFMAs are interleaved with the register-staged operand's LDS stores.
    constexpr bool PRIO = !BOTH_REG;
    if (more) load_stage_reg(g, g.kbeg + (kt + 1) * C::BK);
    if constexpr (!LATE) {
        if (more) load_stage_dma(g, smem, ST ^ 1, g.kbeg + (kt + 1) * C::BK);
    }
    read_frags<C, LA, LB, ST>(g, smem, 1, g.a1, g.b1);
    mfma_step<C, PRIO>(acc, g.a0, g.b0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, NR, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, NM, 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (LATE) {
        if (more) load_stage_dma(g, smem, ST ^ 1, g.kbeg + (kt + 1) * C::BK);
    }
    __builtin_amdgcn_sched_barrier(0);
    read_frags<C, LA, LB, ST>(g, smem, 2, g.a0, g.b0);
    mfma_step<C, PRIO>(acc, g.a1, g.b1);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, NR, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, NM, 0);
    __builtin_amdgcn_sched_barrier(0);
    read_frags<C, LA, LB, ST>(g, smem, 3, g.a1, g.b1);
    mfma_step<C, !REG>(acc, g.a0, g.b0);
    if constexpr (REG) {
        if (more) store_stage(g, smem, ST ^ 1);
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, NR, 0);
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, NM / 2, 0);
        __builtin_amdgcn_sched_group_barrier(SG_DS_WRITE, NDW, 0);
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, NM - NM / 2, 0);
    } else {
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, NR, 0);
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, NM, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (EARLY_BARRIER) {
        // The barrier comes before k-step 3's MFMAs, whose fragments are already in registers:
        // the next tile's first fragments then load under those MFMAs instead of after an idle
        // barrier. Before it, this wave's reads of this stage and its writes (DMA, register-staged
        // stores) of the next stage have completed; no memory fence beyond that.
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        read_frags<C, LA, LB, ST ^ 1>(g, smem, 0, g.a0, g.b0);   // unused past the last tile
        mfma_step<C, PRIO>(acc, g.a1, g.b1);
        __builtin_amdgcn_sched_group_barrier(SG_DS_READ, NR, 0);
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, NM, 0);
        __builtin_amdgcn_sched_barrier(0);
    } else {
        mfma_step<C, PRIO>(acc, g.a1, g.b1);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's DMA into the next stage has landed
        __syncthreads();
        if (more) read_frags<C, LA, LB, ST ^ 1>(g, smem, 0, g.a0, g.b0);
    }
}

// NS > 2 (both operands DMA): the tile in stage ST fetches tile kt + NS - 1 into stage
// (ST + NS - 1) % NS, the one read during the previous tile and released by its barrier. The
// fetch is issued even past the end of K (it zero-fills a stage nobody reads), so every wave has
// the same count of DMA instructions in flight and the wait for tile kt + 1 is a fixed vmcnt.
template <class C, int LA, int LB, int ST>
__device__ __forceinline__ void gemm_tile_ms(GemmState<C, LA, LB>& g, char* smem, f32x16 (&acc)[C::TM][C::TN], int kt,
                                             int nk) {
    static_assert(decltype(g.oa)::DMA && decltype(g.ob)::DMA, "multi-stage tiles need DMA operands");
    constexpr int NR = C::TM + C::TN, NM = C::TM * C::TN;
    constexpr int PER_TILE = decltype(g.oa)::IPW + decltype(g.ob)::IPW;   // DMA instructions per wave per tile
    read_frags<C, LA, LB, ST>(g, smem, 1, g.a1, g.b1);
    mfma_step<C>(acc, g.a0, g.b0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, NR, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, NM, 0);
    __builtin_amdgcn_sched_barrier(0);
    // behind the first MFMAs: NS - 1 tiles of lead already cover the load latency
    load_stage_dma(g, smem, (ST + C::NS - 1) % C::NS, g.kbeg + (kt + C::NS - 1) * C::BK);
    __builtin_amdgcn_sched_barrier(0);
    read_frags<C, LA, LB, ST>(g, smem, 2, g.a0, g.b0);
    mfma_step<C>(acc, g.a1, g.b1);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, NR, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, NM, 0);
    __builtin_amdgcn_sched_barrier(0);
    read_frags<C, LA, LB, ST>(g, smem, 3, g.a1, g.b1);
    mfma_step<C>(acc, g.a0, g.b0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, NR, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, NM, 0);
    __builtin_amdgcn_sched_barrier(0);
    // as in gemm_tile: barrier before k-step 3's MFMAs, once this wave's DMA of tile kt + 1 has
    // landed (tiles kt + 2 .. kt + NS - 1 stay in flight: no fence)
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((C::NS - 2) * PER_TILE) : "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags<C, LA, LB, (ST + 1) % C::NS>(g, smem, 0, g.a0, g.b0);   // unused past the last tile
    mfma_step<C>(acc, g.a1, g.b1);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, NR, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, NM, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// NS consecutive tiles, stages 0 .. NS-1.
template <class C, int LA, int LB, int ST>
__device__ __forceinline__ void gemm_tiles_ms_round(GemmState<C, LA, LB>& g, char* smem, f32x16 (&acc)[C::TM][C::TN],
                                                    int kt, int nk) {
    gemm_tile_ms<C, LA, LB, ST>(g, smem, acc, kt + ST, nk);
    if constexpr (ST + 1 < C::NS) gemm_tiles_ms_round<C, LA, LB, ST + 1>(g, smem, acc, kt, nk);
}

// The last nk - kt < NS tiles (kt a multiple of NS).
template <class C, int LA, int LB, int ST>
__device__ __forceinline__ void gemm_tiles_ms_tail(GemmState<C, LA, LB>& g, char* smem, f32x16 (&acc)[C::TM][C::TN],
                                                   int kt, int nk) {
    if constexpr (ST < C::NS - 1) {
        if (kt < nk) {
            gemm_tile_ms<C, LA, LB, ST>(g, smem, acc, kt, nk);
            gemm_tiles_ms_tail<C, LA, LB, ST + 1>(g, smem, acc, kt + 1, nk);
        }
    }
}

// One work unit of the bf16 MFMA GEMM: unit bid of nblocks -> (output tile, K split), see map_unit.
template <class C, int LA, int LB, class Epi>
__device__ __forceinline__ void gemm_unit(const bf16* __restrict__ A, int lda, const bf16* __restrict__ B, int ldb,
                                          int M, int N, int K, int k_per_split, uint32_t a_bytes, uint32_t b_bytes,
                                          const Epi& epi, int bid, int nblocks, char* smem) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WGN, wn = wave % C::WGN;
    const int tiles_m = (M + C::BM - 1) / C::BM, tiles_n = (N + C::BN - 1) / C::BN;
    int tm, tn;
    int split;
    map_unit(bid, nblocks, tiles_m, tiles_n, tm, tn, split);
    Epi ep = epi;
    ep.set_split(split);

    GemmState<C, LA, LB> g;
    g.ra = make_rsrc(A, a_bytes);
    g.rb = make_rsrc(B, b_bytes);
    g.lda = lda; g.ldb = ldb;
    g.m0 = tm * C::BM; g.n0 = tn * C::BN;
    g.M = M; g.N = N;
    g.kbeg = split * k_per_split;
    g.kend = min(K, g.kbeg + k_per_split);
    g.tid = tid;
    g.oa.init(wm * C::WM + (lane & 31), lane);
    g.ob.init(wn * C::WN + (lane & 31), lane);
    g.oa.setup(lda, g.m0, M, tid);
    g.ob.setup(ldb, g.n0, N, tid);

    f32x16 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int nk = g.kend > g.kbeg ? (g.kend - g.kbeg + C::BK - 1) / C::BK : 0;
    if constexpr (C::NS == 2) {
        if (nk > 0) {
            load_stage(g, smem, 0, g.kbeg);
            store_stage(g, smem, 0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (nk > 0) read_frags<C, LA, LB, 0>(g, smem, 0, g.a0, g.b0);
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            gemm_tile<C, LA, LB, 0>(g, smem, acc, kt, nk);
            gemm_tile<C, LA, LB, 1>(g, smem, acc, kt + 1, nk);
        }
        if (kt < nk) gemm_tile<C, LA, LB, 0>(g, smem, acc, kt, nk);
    } else if (nk > 0) {
        constexpr int PER_TILE = decltype(g.oa)::IPW + decltype(g.ob)::IPW;
#pragma unroll
        for (int s = 0; s < C::NS - 1; ++s) load_stage(g, smem, s, g.kbeg + s * C::BK);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((C::NS - 2) * PER_TILE) : "memory");
        __builtin_amdgcn_s_barrier();
        read_frags<C, LA, LB, 0>(g, smem, 0, g.a0, g.b0);
        int kt = 0;
        for (; kt + C::NS <= nk; kt += C::NS) gemm_tiles_ms_round<C, LA, LB, 0>(g, smem, acc, kt, nk);
        gemm_tiles_ms_tail<C, LA, LB, 0>(g, smem, acc, kt, nk);
        // the zero-fill DMAs issued past the end of K land before the epilogue reuses the LDS
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
    ep.template apply<C>(acc, g.m0, g.n0, g.m0 + wm * C::WM, g.n0 + wn * C::WN, lane, M, N, smem);
}

template <class C, int LA, int LB, class Epi>
__global__ __launch_bounds__(C::NT, 1) void gemm_bf16_kernel(const bf16* __restrict__ A, int lda,
                                                             const bf16* __restrict__ B, int ldb,
                                                             int M, int N, int K, int k_per_split,
                                                             uint32_t a_bytes, uint32_t b_bytes, Epi epi) {
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
    gemm_unit<C, LA, LB, Epi>(A, lda, B, ldb, M, N, K, k_per_split, a_bytes, b_bytes, epi, (int)blockIdx.x,
                              (int)gridDim.x, smem);
}

// Operands and epilogue of one GEMM of a paired launch.
template <class Epi> struct GemmArgs {
    const bf16* A; int lda; const bf16* B; int ldb;
    int M, N, K, k_per_split;
    uint32_t a_bytes, b_bytes;
    Epi epi;
};

// Two independent GEMMs with the same tile configuration in one launch: blocks [0, n1) are the
// first GEMM's units, the rest the second's (each mapped as in its own launch). For two GEMMs
// that each leave most of the chip idle, so that their units share the CUs instead of running
// one after the other.
template <class C, int LA1, int LB1, class E1, int LA2, int LB2, class E2>
__global__ __launch_bounds__(C::NT, 1) void gemm_bf16_pair_kernel(GemmArgs<E1> p, GemmArgs<E2> q, int n1) {
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
    const int bid = (int)blockIdx.x;
    if (bid < n1)
        gemm_unit<C, LA1, LB1, E1>(p.A, p.lda, p.B, p.ldb, p.M, p.N, p.K, p.k_per_split, p.a_bytes, p.b_bytes, p.epi,
                                   bid, n1, smem);
    else
        gemm_unit<C, LA2, LB2, E2>(q.A, q.lda, q.B, q.ldb, q.M, q.N, q.K, q.k_per_split, q.a_bytes, q.b_bytes, q.epi,
                                   bid - n1, (int)gridDim.x - n1, smem);
}

// ----------------------------------------------------------------------------------------------
// fp32 SIMT kernel: TS x TS tile (64 or 32), BK = 16, 256 threads, (TS/16)^2 outputs per thread.
// The next K step's operand elements are fetched into registers while the current one is
// multiplied from LDS, so a step waits on global memory only once at the start.
// ----------------------------------------------------------------------------------------------
template <int TS, int LA, int LB, class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int lda,
                                                       const float* __restrict__ B, int ldb,
                                                       int M, int N, int K, int k_per_split, Epi epi) {
    static_assert(TS == 64 || TS == 32, "tile size");
    constexpr int R = TS / 16;   // outputs per thread per dimension, and elements per operand per step
    __shared__ float As[16][TS + 4];
    __shared__ float Bs[16][TS + 4];
    const int tid = threadIdx.x;
    const int tiles_n = (N + TS - 1) / TS;
    const int m0 = (blockIdx.x / tiles_n) * TS, n0 = (blockIdx.x % tiles_n) * TS;
    const int kbeg = blockIdx.y * k_per_split, kend = min(K, kbeg + k_per_split);
    Epi ep = epi;
    ep.set_split(blockIdx.y);
    const int ty = tid / 16, tx = tid % 16;
    // element i of this thread's share of a TS x 16 operand slab: (mn, k)
    auto coord = [&](int layout, int i, int& mn, int& k) {
        const int e = tid + i * 256;
        if (layout == KCONTIG) { mn = e / 16; k = e % 16; } else { k = e / TS; mn = e % TS; }
    };
    float ra[R], rb[R];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            int mn, k;
            coord(LA, i, mn, k);
            const int gm = m0 + mn, gk = k0 + k;
            ra[i] = (gm < M && gk < kend) ? ((LA == KCONTIG) ? A[(size_t)gm * lda + gk] : A[(size_t)gk * lda + gm]) : 0.f;
            coord(LB, i, mn, k);
            const int gn = n0 + mn, gkb = k0 + k;
            rb[i] = (gn < N && gkb < kend) ? ((LB == KCONTIG) ? B[(size_t)gn * ldb + gkb] : B[(size_t)gkb * ldb + gn])
                                           : 0.f;
        }
    };
    float acc[R][R] = {};
    if (kbeg < kend) fetch(kbeg);
    for (int k0 = kbeg; k0 < kend; k0 += 16) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            int mn, k;
            coord(LA, i, mn, k);
            As[k][mn] = ra[i];
            coord(LB, i, mn, k);
            Bs[k][mn] = rb[i];
        }
        __syncthreads();
        if (k0 + 16 < kend) fetch(k0 + 16);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            float a[R], b[R];
#pragma unroll
            for (int i = 0; i < R; ++i) a[i] = As[k][ty * R + i];
#pragma unroll
            for (int j = 0; j < R; ++j) b[j] = Bs[k][tx * R + j];
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
                for (int j = 0; j < R; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < R; ++j) {
            int r = m0 + ty * R + i, c = n0 + tx * R + j;
            if (r < M && c < N) ep(r, c, acc[i][j]);
        }
}

// Split-K reduction: out = epi(sum_{s=0}^{splits-1} part[s][r*N + c]) in split order, 8 columns
// per thread (N % 8 == 0), in blocks [0, nsk). Blocks past nsk run a column-sum job carried by the
// launch (rowsum_block over its column blocks), so that a small reduction whose inputs are ready
// needs no launch of its own.
template <class Epi>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits,
                                                            size_t split_stride, int M, int N, Epi epi, ColSumJob cj,
                                                            int nsk) {
    if ((int)blockIdx.x >= nsk) {
        rowsum_block<bf16>(cj.part, (bf16*)cj.out, cj.nb, cj.n, cj.accumulate, (int)blockIdx.x - nsk);
        return;
    }
    const size_t idx = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (idx >= (size_t)M * N) return;
    const int r = (int)(idx / N), c = (int)(idx % N);
    float acc[8];
    load8(part + idx, acc);
    for (int s = 1; s < splits; ++s) {
        float v[8];
        load8(part + (size_t)s * split_stride + idx, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += v[e];
    }
    epi.op8(r, c, acc);
}

}  // namespace tp
