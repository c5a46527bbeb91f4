// Causal multi-head attention for one rank's heads on gfx950, forward and backward.
//
// Per (sequence, head): S = Q K^T / sqrt(d), masked, P = softmax(S), O = P V, saved lse.
// Head width D (64, 96, 128 or 192) is handled as D/16 k-steps of 16 (scores) and D/32 tiles of 32
// (outputs); D = 96 is the 8.3B shape's.
//
// Orientation. The kernels compute S^T = K Q^T so that an MFMA accumulator lane holds ONE query
// (column = lane % 32) and 16 keys in registers: the softmax row reductions are in-lane plus one
// exchange with lane ^ 32, and the fp32 probabilities already sit in the MFMA B-operand layout
// for O^T = V^T P^T. The k-order inside a lane's 8-element operand is a free choice as long as
// both operands use the same one; the kernels use the accumulator's own row order
// (keys 16s + 4*(lane/32) + 0..3 and 16s + 8 + 4*(lane/32) + 0..3), so P is converted to bf16
// in place, and V^T (likewise K^T, Q^T, dO^T in the backward) is read in that order from the
// row-major V tile with gfx950's transposing LDS load: no tile is ever transposed in memory.
// Softmax runs in the log2 domain in fp32 (scores pre-scaled by log2(e)/sqrt(d)).
//
// Work split. A block has four waves and owns 64 rows (queries in the forward and dQ kernels, keys
// in the dK/dV kernel): waves 0/1 and 2/3 each cover the 64 rows as two 32-row groups. In the
// forward and dQ kernels the two pairs take alternate 64-wide key tiles; in the dK/dV kernel they
// take the two 32-query halves of each query tile (one tile per step keeps its staging registers
// within the two-waves-per-SIMD budget). The pairs' partial results are merged through LDS at the
// end in a fixed order. Blocks are launched heaviest first (most visible tiles under the causal
// mask). Up to D = 96 the kernels are held to 256 registers per lane (two waves per SIMD). Loop
// tiles are staged through registers: the next step's global loads are in flight while the
// current step's tiles are used.
//
// Backward: D = rowsum(dO * O); the dK/dV kernel owns 64 keys per block, loops over query tiles,
// recomputes P from lse and forms dS = P (dP - D); it also stores dS (bf16, the values its dK
// product uses) as one 64 x 64 block per (key tile, query tile) pair it visits, each block in the
// order the waves' accumulators hold it, so every store instruction writes a whole kilobyte. The
// dQ kernel owns 64 queries per block, turns those blocks into [key][query] LDS tiles as it
// stages them and computes dQ = dS K: no second pass over S, P and dP. No atomics: every output
// element is written by exactly one lane.
//
// Dropout on the attention weights (DROP = true; "Megatron-LM ..." paper digest, §3.4: drawn per
// rank): the forward draws each lane's keep bits with Philox (rng.h; the element mapping puts a
// lane's 16 keys of a 32-key tile in two calls), applies P~ = P * keep * scale before P V while
// the row sums l use the undropped P, and stores the bits as a query-major bitmap, one 32-bit word
// per (query, 32-key tile). The backward reads the bits instead of drawing again: dV = P~^T dO,
// dP = (dO V^T) * keep * scale, dS = P (dP - D) with D = rowsum(dO * O) unchanged. The dK/dV
// kernel (one key and 16 queries per lane) stages the query tile's words in LDS with lse and D;
// the dQ kernel reads dS and so needs no bits.
#pragma once
#include "common.h"
#include "rng.h"

namespace tp {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int ATT_B = 64;        // queries per block (fwd, dQ) / keys per block (dK dV), rows per tile
constexpr int ATT_NT = 256;      // 4 waves: two 32-row groups x two loop-tile parities

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// LDS tiles are row-major [64][D] bf16 with the 16-byte chunk index XOR-swizzled by a function of
// the row's low four bits, chosen per width so that three access patterns are free of bank
// conflicts (64 banks of 4 bytes; 128-bit accesses served 16 lanes at a time, 64-bit ones 32): the
// 128-bit read of 8 consecutive columns by 32 consecutive rows (MFMA operand with K along the
// columns), the transposing 64-bit read of 4-row x 16-column blocks (MFMA operand with K along the
// rows), and row-major 16-byte stores of whole rows. Width 96 (192-byte rows): bits 2, 3 of the
// row. Widths 64 and 192: bits 1, 2 and 1^3. Width 128: bits 0, 1, 0^2 and 1^3. (Row strides
// that are multiples of 256 bytes, or of 128, put rows r and r + 2 on the same banks; the extra
// terms separate them.) The XOR stays inside an aligned group of 4, 8 or 16 chunks, so it never
// leaves the row.
template <int D>
__device__ __forceinline__ int att_swz(int row) {
    const int b0 = row & 1, b1 = (row >> 1) & 1, b2 = (row >> 2) & 1, b3 = (row >> 3) & 1;
    if constexpr (D == 128) return b0 | (b1 << 1) | ((b0 ^ b2) << 2) | ((b1 ^ b3) << 3);
    else if constexpr (D == 64 || D == 192) return b1 | (b2 << 1) | ((b1 ^ b3) << 2);
    else return (row >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int att_off(int row, int col) {
    static_assert(D == 64 || D == 96 || D == 128 || D == 192, "tile width without a swizzle");
    return row * D + ((((col >> 3) ^ att_swz<D>(row)) << 3) | (col & 7));
}

// Register-staged copy of rows [r0, r0 + ROWS) x D of a strided bf16 matrix into consecutive LDS
// tiles (row r lands in tile r / 64; att_off is valid across them). Loads go through a buffer
// resource covering exactly the sequence's `valid` rows (att_rsrc): a row index clamped to `valid`
// starts at or past the resource's end (the row stride is at least D), so rows >= valid read 0
// with no compare or branch per load.
template <int D, int ROWS = 2 * ATT_B>
struct AttTileRegs {
    static constexpr int CPR = D / 8, N = ROWS * CPR / ATT_NT;
    static_assert((ROWS * CPR) % ATT_NT == 0, "tile/threads mismatch");
    u32x4 v[N];
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int ld, int r0, int valid, int tid) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int c = tid + i * ATT_NT, row = c / CPR, dc = c % CPR;
            const int off = (min(r0 + row, valid) * ld + dc * 8) * 2;
            v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        }
    }
    __device__ __forceinline__ void store(bf16* tiles, int tid) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            int c = tid + i * ATT_NT, row = c / CPR, dc = c % CPR;
            *(u32x4*)(tiles + att_off<D>(row, dc * 8)) = v[i];
        }
    }
};

// Buffer resource over a sequence's s rows x D columns of a strided matrix starting at p (row
// stride ld): exactly the bytes from the first row's start to the last row's end.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t att_rsrc(const bf16* p, int ld, int s) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(p), (short)0, (int)(((size_t)(s - 1) * ld + D) * 2),
                                             0x00020000);
}

// Copy of rows [r0, r0 + 64) x D of a strided bf16 matrix into one LDS tile (rows >= valid
// read 0); used once per block for the block's own rows, which then serve as MFMA operands
// straight from LDS instead of occupying registers.
template <int D>
__device__ __forceinline__ void load_tile(const bf16* __restrict__ src, int ld, int r0, int valid, bf16* tile, int tid) {
    AttTileRegs<D, ATT_B> r;   // every load issued before the first store
    r.load(att_rsrc<D>(src, ld, valid), ld, r0, valid, tid);
    r.store(tile, tid);
}

// MFMA operand with the tile's rows as M and its columns as K: rows row0 + lane%32, columns
// col0 + 8*(lane/32) .. +7.
template <int D>
__device__ __forceinline__ bf16x8 frag_rows(const bf16* tile, int row0, int col0, int lane) {
    return *(const bf16x8*)(tile + att_off<D>(row0 + (lane & 31), col0 + 8 * (lane >> 5)));
}

// MFMA operand with the tile's columns as M and its rows as K, read with the transposing LDS load,
// in the accumulator's k-order: lane l gets column m0 + l%32 and rows k0 + 4h + 0..3 and
// k0 + 8 + 4h + 0..3 (h = l/32). Within a 16-lane group the hardware hands lane i the (i%4)-th
// element of the 8 bytes addressed by lane 4e + i/4, e = 0..3; so source lane s addresses
// row (s/4), columns 4*(s%4) .. +3 of the group's 4x16 block.
template <int D>
__device__ __forceinline__ bf16x8 frag_cols(const bf16* tile, int k0, int m0, int lane) {
    const int h = lane >> 5, g = (lane >> 4) & 1, s = lane & 15;
    const int row = k0 + 4 * h + (s >> 2), col = m0 + 16 * g + 4 * (s & 3);
    s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + att_off<D>(row, col)));
    s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + att_off<D>(row + 8, col)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 2^x with the hardware instruction: results below 2^-126 flush to zero, which only drops
// probabilities that are negligible against the row's maximum (and maps -inf to 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 pack8(const f32x16& a, int base) {
    u32x4 u;
    u[0] = pack_bf16x2(a[base + 0], a[base + 1]);
    u[1] = pack_bf16x2(a[base + 2], a[base + 3]);
    u[2] = pack_bf16x2(a[base + 4], a[base + 5]);
    u[3] = pack_bf16x2(a[base + 6], a[base + 7]);
    return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int v = 0; v < 16; ++v) z[v] = 0.f;
    return z;
}

// Exchange of per-lane fp32 values between the two parities of a row group (LDS, lane-fastest).
template <int NV>
__device__ __forceinline__ void xch_put(float* xch, int group, int j, int lane, float v) {
    xch[(group * NV + j) * 64 + lane] = v;
}
template <int NV>
__device__ __forceinline__ float xch_get(const float* xch, int group, int j, int lane) {
    return xch[(group * NV + j) * 64 + lane];
}

// ---------------------------------------------------------------------------------------------
// Forward. grid = (b * heads_t, query tiles), query tile qt = last - blockIdx.y (heavy first).
// Wave w: row group g = w & 1 (queries qt*64 + 32g ..), key-tile parity kp = w >> 1.
// ---------------------------------------------------------------------------------------------
template <int D, bool DROP>
__global__ __launch_bounds__(ATT_NT) __attribute__((amdgpu_waves_per_eu(D <= 96 ? 2 : 1)))
void attn_fwd_kernel(const bf16* __restrict__ QKV, int ld, int h_t, int s, int heads_t, float scale_log2,
                     int causal, bf16* __restrict__ O, int ldo, float* __restrict__ lse, DropParams dp) {
    __shared__ __attribute__((aligned(16))) bf16 smem[4 * ATT_B * D];   // K tiles [2] | V tiles [2]
    __shared__ __attribute__((aligned(16))) bf16 Qs[ATT_B * D];          // the block's queries
    bf16* Kb = smem;
    bf16* Vb = smem + 2 * ATT_B * D;
    const int head = blockIdx.x % heads_t, bi = blockIdx.x / heads_t, qt = gridDim.y - 1 - blockIdx.y;
    // the wave index through readfirstlane: everything derived from it (row group, loop parity,
    // masks) is known uniform, so those branches are scalar instead of per-lane selects
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), h = lane >> 5,
              l32 = lane & 31;
    const int grp = wave & 1, kp = wave >> 1;
    const size_t tok0 = (size_t)bi * s;
    const bf16* Qp = QKV + tok0 * ld + head * D;
    const bf16* Kp = QKV + tok0 * ld + h_t + head * D;
    const bf16* Vp = QKV + tok0 * ld + 2 * h_t + head * D;
    const int q0w = qt * ATT_B + grp * 32;
    const int myq = q0w + l32;

    const int kv_end = causal ? min(s, (qt + 1) * ATT_B) : s;
    const int ntiles = (kv_end + ATT_B - 1) / ATT_B;
    const int niter = (ntiles + 1) / 2;
    AttTileRegs<D> kr, vr;
    const auto krs = att_rsrc<D>(Kp, ld, s), vrs = att_rsrc<D>(Vp, ld, s);
    // the first step's K/V loads and the block's Q tile are in flight together
    if (niter > 0) {
        kr.load(krs, ld, 0, s, tid);
        vr.load(vrs, ld, 0, s, tid);
    }
    load_tile<D>(Qp, ld, qt * ATT_B, s, Qs, tid);
    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] = zero16();
    float m_i = -INFINITY, l_i = 0.f;
    if (niter > 0) {
        kr.store(Kb, tid);
        vr.store(Vb, tid);
    }
    __syncthreads();
    for (int it = 0; it < niter; ++it) {
        const bool more = it + 1 < niter;
        if (more) {
            kr.load(krs, ld, (it + 1) * 2 * ATT_B, s, tid);
            vr.load(vrs, ld, (it + 1) * 2 * ATT_B, s, tid);
        }
        const int kt = 2 * it + kp, k0 = kt * ATT_B;
        if (kt < ntiles && !(causal && k0 > q0w + 31)) {   // some key of this tile is visible to this wave
            const bf16* K = Kb + kp * ATT_B * D;
            const bf16* V = Vb + kp * ATT_B * D;
            const bool need_mask = (causal && k0 + ATT_B - 1 > q0w) || (k0 + ATT_B > s);
            f32x16 st[2];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                st[sub] = zero16();
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks)
                    st[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<D>(K, sub * 32, ks * 16, lane),
                                                                      frag_rows<D>(Qs, grp * 32, ks * 16, lane),
                                                                      st[sub], 0, 0, 0);
            }
            if (need_mask) {   // uniform: tiles with every key visible skip the block
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int key = k0 + sub * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                        const bool masked = (causal && key > myq) || key >= s;
                        st[sub][v] = masked ? -INFINITY : st[sub][v];
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, st[sub][v]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_i, mx * scale_log2);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_i - m_use);
            float rs = 0.f;
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    float p = fast_exp2(fmaf(st[sub][v], scale_log2, -m_use));
                    st[sub][v] = p;
                    rs += p;
                }
            rs += __shfl_xor(rs, 32);
            l_i = l_i * alpha + rs;
            m_i = m_new;
            if constexpr (DROP) {
                const int n32 = (s + 31) >> 5;
                const uint64_t row = ((uint64_t)bi * dp.heads + dp.head0 + head) * s + myq;
#pragma unroll
                for (int sub = 0; sub < 2; ++sub) {
                    const int kt32 = (k0 >> 5) + sub;
                    const uint64_t call = ((row * n32 + kt32) * 2 + h) * 2;
                    const uint32_t bits = keep8(call, dp) | (keep8(call + 1, dp) << 8);
                    uint32_t w = 0;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const uint32_t kb = (bits >> v) & 1u;
                        st[sub][v] = kb ? st[sub][v] * dp.scale : 0.0f;
                        w |= kb << (8 * (v >> 2) + 4 * h + (v & 3));
                    }
                    w |= __shfl_xor(w, 32);
                    if (h == 0 && myq < s && kt32 < n32) dp.mask[((size_t)(bi * heads_t + head) * s + myq) * n32 + kt32] = w;
                }
            }
            // rescale only when some lane's running max moved (alpha == 1 leaves o unchanged)
            if (__builtin_amdgcn_read_exec() && __any(alpha != 1.0f)) {
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
            }
#pragma unroll
            for (int ks = 0; ks < ATT_B / 16; ++ks) {
                bf16x8 pb = pack8(st[ks >> 1], 8 * (ks & 1));
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols<D>(V, 16 * ks, dt * 32, lane), pb, o[dt],
                                                                    0, 0, 0);
            }
        }
        __syncthreads();   // both tiles consumed
        if (more) {
            kr.store(Kb, tid);
            vr.store(Vb, tid);
        }
        __syncthreads();
    }
    // merge the odd-tile partial (m, l, o) into the even-tile one: m = max, rescale both, add
    constexpr int NV = D / 2 + 2;
    float* xch = (float*)smem;
    static_assert(2 * NV * 64 * 4 <= 4 * ATT_B * D * 2, "exchange exceeds the tile buffers");
    if (kp == 1) {
        xch_put<NV>(xch, grp, 0, lane, m_i);
        xch_put<NV>(xch, grp, 1, lane, l_i);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) xch_put<NV>(xch, grp, 2 + dt * 16 + v, lane, o[dt][v]);
    }
    __syncthreads();
    if (kp == 0 && myq < s) {
        const float m_o = xch_get<NV>(xch, grp, 0, lane), l_o = xch_get<NV>(xch, grp, 1, lane);
        const float m = fmaxf(m_i, m_o);
        const float m_use = (m == -INFINITY) ? 0.f : m;
        const float a = fast_exp2(m_i - m_use), c = fast_exp2(m_o - m_use);
        const float l = l_i * a + l_o * c;
        const float inv = 1.0f / l;
        bf16* op = O + (tok0 + myq) * ldo + head * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) o[dt][v] = (o[dt][v] * a + xch_get<NV>(xch, grp, 2 + dt * 16 + v, lane) * c) * inv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int d = dt * 32 + 8 * i + 4 * h;
                *(u32x2*)(op + d) = u32x2{pack_bf16x2(o[dt][4 * i], o[dt][4 * i + 1]),
                                          pack_bf16x2(o[dt][4 * i + 2], o[dt][4 * i + 3])};
            }
        }
        if (h == 0) lse[((size_t)bi * heads_t + head) * s + myq] = (m + log2f(l)) * kLn2;
    }
}

// ---------------------------------------------------------------------------------------------
// D[b, head, q] = sum_d dO[q, head*D + d] * O[q, head*D + d]   (fp32)
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dot_kernel(const bf16* __restrict__ dO, const bf16* __restrict__ O,
                                                           int ld, int b, int s, int heads_t, float* __restrict__ Dv) {
    // four lanes per (token, head) row, each taking every fourth 16-byte chunk of it: a wave's
    // load covers 64 contiguous bytes of each of 16 rows; the four partial sums meet by shuffles
    static_assert(D % 32 == 0, "head width must be a multiple of 32");
    const size_t idx = ((size_t)blockIdx.x * 256 + threadIdx.x) >> 2;
    const int part = threadIdx.x & 3;
    const size_t total = (size_t)b * s * heads_t;
    const bool live = idx < total;
    float acc = 0.f;
    const int head = live ? (int)(idx % heads_t) : 0;
    const size_t tok = live ? idx / heads_t : 0;
    if (live) {
        const bf16* a = dO + tok * ld + head * D;
        const bf16* c = O + tok * ld + head * D;
#pragma unroll
        for (int k = part * 8; k < D; k += 32) {
            bf16x8 x = *(const bf16x8*)(a + k), y = *(const bf16x8*)(c + k);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += (float)x[e] * (float)y[e];
        }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    if (live && part == 0) {
        const int bi = (int)(tok / s), pos = (int)(tok % s);
        Dv[((size_t)bi * heads_t + head) * s + pos] = acc;
    }
}

// Column sums over a block's 64 rows (tokens) of D columns held in MFMA accumulator layout by two
// waves (rows 32g + lane % 32, column dt*32 + 8(v/4) + 4(lane/32) + v%4 of acc[dt][v]): the values
// as rounded to bf16 (zeros for rows past the sequence) go through an fp32 LDS buffer [64][D + 4]
// and D threads add their column's rows in order; out[d] = sum. Called by all threads of the block
// after the buffer's previous contents are no longer needed by any wave.
template <int D, int NDT>
__device__ __forceinline__ void tile_colsum(const f32x16 (&acc)[NDT], bool holder, bool valid, int row, int lane, int tid,
                                            float* buf, float* __restrict__ out) {
    constexpr int LDC = D + 4;
    const int h = lane >> 5;
    __syncthreads();
    if (holder) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = valid ? (float)(bf16)acc[dt][4 * i + e] : 0.f;
                *(f32x4*)(buf + row * LDC + dt * 32 + 8 * i + 4 * h) = w;
            }
    }
    __syncthreads();
    for (int d = tid; d < D; d += ATT_NT) {
        float sum = 0.f;
#pragma unroll 8
        for (int r = 0; r < ATT_B; ++r) sum += buf[r * LDC + d];
        out[d] = sum;
    }
}

// dS blocks of one (sequence, head): one per (key tile kt, query tile qt) pair with a visible key,
// i.e. qt >= kt under the causal mask (ordered by kt, then qt), every pair otherwise.
__host__ __device__ __forceinline__ int ds_pairs(int nq, int causal) { return causal ? nq * (nq + 1) / 2 : nq * nq; }
__device__ __forceinline__ int ds_pair(int kt, int qt, int nq, int causal) {
    return causal ? kt * nq - kt * (kt - 1) / 2 + (qt - kt) : kt * nq + qt;
}

// ---------------------------------------------------------------------------------------------
// dK, dV. grid = (b * heads_t, key tiles), key tile kt = blockIdx.y (heavy first under the causal
// mask). Wave w: key group g = w & 1 (keys kt*64 + 32g ..), query half q = w >> 1 of each query
// tile; the waves loop over the query tiles that can see their keys, one tile (Q, dO, lse, D) per
// step, and the two query halves' dK, dV are added at the end.
//   S = Q K^T, P = exp2(S*c - lse2), dP = dO V^T, dS = P (dP - D)      (query rows x own keys)
//   dV^T += dO^T P,  dK^T += Q^T dS                                     (transposing reads)
// ---------------------------------------------------------------------------------------------
template <int D, bool DROP>
__global__ __launch_bounds__(ATT_NT) __attribute__((amdgpu_waves_per_eu(D <= 96 ? 2 : 1)))
void attn_bwd_dkdv_kernel(const bf16* __restrict__ QKV, int ld, int h_t, int s, int heads_t,
                          const bf16* __restrict__ dO, int ld_do, const float* __restrict__ lse,
                          const float* __restrict__ Dv, float scale_log2, float scale, int causal,
                          bf16* __restrict__ dQKV, int ld_dq, bf16* __restrict__ dSb, float* __restrict__ colpart,
                          DropParams dp) {
    __shared__ __attribute__((aligned(16))) bf16 smem[4 * ATT_B * D];   // Q tile | dO tile | K | V
    __shared__ float lse_s[ATT_B], D_s[ATT_B];
    __shared__ uint32_t mk_s[ATT_B][2];   // dropout keep words of the query tile x the block's two key groups
    bf16* Qb = smem;
    bf16* Gb = smem + ATT_B * D;
    bf16* KVs = smem + 2 * ATT_B * D;
    const int head = blockIdx.x % heads_t, bi = blockIdx.x / heads_t, kt = blockIdx.y;
    // the wave index through readfirstlane: everything derived from it (row group, loop parity,
    // masks) is known uniform, so those branches are scalar instead of per-lane selects
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), h = lane >> 5,
              l32 = lane & 31;
    const int grp = wave & 1, qh = wave >> 1;
    const size_t tok0 = (size_t)bi * s;
    const bf16* Qp = QKV + tok0 * ld + head * D;
    const bf16* Kp = QKV + tok0 * ld + h_t + head * D;
    const bf16* Vp = QKV + tok0 * ld + 2 * h_t + head * D;
    const bf16* dOp = dO + tok0 * ld_do + head * D;
    const float* lsep = lse + ((size_t)bi * heads_t + head) * s;
    const float* Dp = Dv + ((size_t)bi * heads_t + head) * s;
    const int kw0 = kt * ATT_B + grp * 32;
    const int mykey = kw0 + l32;

    const bf16* Ks = KVs;
    const bf16* Vs = KVs + ATT_B * D;
    const int nqt = (s + ATT_B - 1) / ATT_B;
    const int qt0 = causal ? kt : 0;
    AttTileRegs<D, ATT_B> qr, gr;
    const auto qrs = att_rsrc<D>(Qp, ld, s), grs = att_rsrc<D>(dOp, ld_do, s);
    float lse_r = INFINITY, d_r = 0.f;
    uint32_t mk_r = 0;
    const int n32 = (s + 31) >> 5;
    auto fetch = [&](int q0) {
        qr.load(qrs, ld, q0, s, tid);
        gr.load(grs, ld_do, q0, s, tid);
        if (tid < ATT_B) {
            int q = q0 + tid;
            lse_r = (q < s) ? lsep[q] * kLog2e : INFINITY;
            d_r = (q < s) ? Dp[q] : 0.f;
        }
        if constexpr (DROP) {
            if (tid < 2 * ATT_B) {
                const int q = q0 + (tid >> 1), kt32 = 2 * kt + (tid & 1);
                mk_r = (q < s && kt32 < n32) ? dp.mask[((size_t)(bi * heads_t + head) * s + q) * n32 + kt32] : 0u;
            }
        }
    };
    auto stash = [&]() {
        qr.store(Qb, tid);
        gr.store(Gb, tid);
        if (tid < ATT_B) { lse_s[tid] = lse_r; D_s[tid] = d_r; }
        if constexpr (DROP) {
            if (tid < 2 * ATT_B) mk_s[tid >> 1][tid & 1] = mk_r;
        }
    };
    // the first query tile's loads and the block's K/V tiles are in flight together
    if (qt0 < nqt) fetch(qt0 * ATT_B);
    load_tile<D>(Kp, ld, kt * ATT_B, s, KVs, tid);
    load_tile<D>(Vp, ld, kt * ATT_B, s, KVs + ATT_B * D, tid);
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) { dk[dt] = zero16(); dv[dt] = zero16(); }
    if (qt0 < nqt) stash();
    __syncthreads();
    // this wave's two 1 KB chunks (kk = 0, 1) of dS block (kt, qt), in the accumulator's own order
    bf16* dsw = dSb + ((size_t)(bi * heads_t + head) * ds_pairs(nqt, causal) + ds_pair(kt, qt0, nqt, causal)) * (ATT_B * ATT_B) +
                (grp * 2 + qh) * 2 * 512 + lane * 8;
    for (int qt = qt0; qt < nqt; ++qt, dsw += ATT_B * ATT_B) {
        const bool more = qt + 1 < nqt;
        if (more) fetch((qt + 1) * ATT_B);
        const int q0 = qt * ATT_B;
        const int qs0 = q0 + qh * 32;
        u32x4 dsv[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};   // this step's dS, stored at its end
        if (causal && qs0 + 31 < kw0) {   // no query of this half sees a key of this wave: dS = 0
        } else {
            const bool need_mask = (causal && qs0 < kw0 + 31) || (qs0 + 32 > s) || (kw0 + 32 > s);
            f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<D>(Qb, qh * 32, ks * 16, lane),
                                                               frag_rows<D>(Ks, grp * 32, ks * 16, lane), sacc, 0, 0, 0);
                dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<D>(Gb, qh * 32, ks * 16, lane),
                                                                frag_rows<D>(Vs, grp * 32, ks * 16, lane), dpacc, 0, 0, 0);
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int qi = qh * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                sacc[v] = fast_exp2(fmaf(sacc[v], scale_log2, -lse_s[qi]));
            }
            if (need_mask) {   // uniform: one skipped block on the tiles that need no mask
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int q = q0 + qh * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                    const bool masked = (causal && mykey > q) || mykey >= s;
                    sacc[v] = masked ? 0.f : sacc[v];
                }
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int qi = qh * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                const float pv = sacc[v];
                if constexpr (DROP) {
                    const bool kb = (mk_s[qi][grp] >> l32) & 1u;
                    sacc[v] = kb ? pv * dp.scale : 0.0f;
                    dpacc[v] = pv * ((kb ? dpacc[v] * dp.scale : 0.0f) - D_s[qi]);
                } else {
                    sacc[v] = pv;
                    dpacc[v] = pv * (dpacc[v] - D_s[qi]);
                }
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 pb = pack8(sacc, 8 * kk), dsb = pack8(dpacc, 8 * kk);
                dsv[kk] = __builtin_bit_cast(u32x4, dsb);
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols<D>(Gb, qh * 32 + 16 * kk, dt * 32, lane),
                                                                     pb, dv[dt], 0, 0, 0);
                    dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols<D>(Qb, qh * 32 + 16 * kk, dt * 32, lane),
                                                                     dsb, dk[dt], 0, 0, 0);
                }
            }
        }
        __syncthreads();
        if (more) stash();
        __syncthreads();
        // dS for the dQ kernel, issued after the stash's wait for the next tile's loads so that the
        // stores drain during the next step instead of holding up that wait
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) *(u32x4*)(dsw + 512 * kk) = dsv[kk];
    }
    // merge: the second query half's waves hand dK, dV to the first half's wave of the same key
    // group, through the tile buffers (in two rounds, dK then dV, when both do not fit at once)
    float* xch = (float*)smem;
    constexpr int NH = D / 2;   // floats per lane per accumulator set
    constexpr bool ONE_ROUND = 2 * (2 * NH) * 64 * 4 <= 4 * ATT_B * D * 2;
    static_assert(2 * NH * 64 * 4 <= 4 * ATT_B * D * 2, "exchange exceeds the tile buffers");
    if constexpr (ONE_ROUND) {
        if (qh == 1) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    xch_put<2 * NH>(xch, grp, dt * 16 + v, lane, dk[dt][v]);
                    xch_put<2 * NH>(xch, grp, NH + dt * 16 + v, lane, dv[dt][v]);
                }
        }
        __syncthreads();
        if (qh == 0) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    dk[dt][v] += xch_get<2 * NH>(xch, grp, dt * 16 + v, lane);
                    dv[dt][v] += xch_get<2 * NH>(xch, grp, NH + dt * 16 + v, lane);
                }
        }
    } else {
        if (qh == 1) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int v = 0; v < 16; ++v) xch_put<NH>(xch, grp, dt * 16 + v, lane, dk[dt][v]);
        }
        __syncthreads();
        if (qh == 0) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int v = 0; v < 16; ++v) dk[dt][v] += xch_get<NH>(xch, grp, dt * 16 + v, lane);
        }
        __syncthreads();
        if (qh == 1) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int v = 0; v < 16; ++v) xch_put<NH>(xch, grp, dt * 16 + v, lane, dv[dt][v]);
        }
        __syncthreads();
        if (qh == 0) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int v = 0; v < 16; ++v) dv[dt][v] += xch_get<NH>(xch, grp, dt * 16 + v, lane);
        }
    }
    if (qh == 0) {
        bf16* kp_ = dQKV + (tok0 + mykey) * ld_dq + h_t + head * D;
        bf16* vp_ = dQKV + (tok0 + mykey) * ld_dq + 2 * h_t + head * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) dk[dt][v] *= scale;
            if (mykey < s) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    int d = dt * 32 + 8 * i + 4 * h;
                    *(u32x2*)(kp_ + d) = u32x2{pack_bf16x2(dk[dt][4 * i], dk[dt][4 * i + 1]),
                                               pack_bf16x2(dk[dt][4 * i + 2], dk[dt][4 * i + 3])};
                    *(u32x2*)(vp_ + d) = u32x2{pack_bf16x2(dv[dt][4 * i], dv[dt][4 * i + 1]),
                                               pack_bf16x2(dv[dt][4 * i + 2], dv[dt][4 * i + 3])};
                }
            }
        }
    }
    static_assert(ATT_B * (D + 4) * 4 <= sizeof(smem), "column-sum buffer exceeds the tile buffers");
    if (colpart) {
        float* cp = colpart + (size_t)(bi * nqt + kt) * (3 * h_t) + head * D;
        tile_colsum<D, D / 32>(dk, qh == 0, mykey < s, grp * 32 + l32, lane, tid, (float*)smem, cp + h_t);
        tile_colsum<D, D / 32>(dv, qh == 0, mykey < s, grp * 32 + l32, lane, tid, (float*)smem, cp + 2 * h_t);
    }
}

// ---------------------------------------------------------------------------------------------
// dQ = scale * dS K from the dK/dV kernel's dS blocks. grid = (b * heads_t, query tiles), qt = last
// - blockIdx.y (heavy first). Wave w: row group g = w & 1 (32 queries), key-tile parity kp = w >> 1;
// per step the block stages two key tiles and their dS blocks (register-staged, the next pair's
// loads in flight while the current pair is multiplied):
//   dQ^T (D x 32 queries) += K^T (D x 64 keys) dS^T (64 keys x 32 queries)
// both operands read with the transposing LDS load from the row-major K tile and the [key][query]
// dS block, in the same k order. The two parities' sums are added at the end.
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(ATT_NT) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void attn_bwd_dq_kernel(const bf16* __restrict__ QKV, int ld, int h_t, int s, int heads_t,
                        const bf16* __restrict__ dSb, float scale, int causal, bf16* __restrict__ dQKV, int ld_dq,
                        float* __restrict__ colpart) {
    __shared__ __attribute__((aligned(16))) bf16 sm[2 * ATT_B * D + 2 * ATT_B * ATT_B];
    bf16* Kb = sm;                      // key tiles of parity 0 | 1
    bf16* Sb = sm + 2 * ATT_B * D;      // their dS blocks
    const int head = blockIdx.x % heads_t, bi = blockIdx.x / heads_t, qt = gridDim.y - 1 - blockIdx.y;
    // the wave index through readfirstlane: everything derived from it (row group, loop parity,
    // masks) is known uniform, so those branches are scalar instead of per-lane selects
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), h = lane >> 5,
              l32 = lane & 31;
    const int grp = wave & 1, kp = wave >> 1;
    const size_t tok0 = (size_t)bi * s;
    const bf16* Kp = QKV + tok0 * ld + h_t + head * D;
    const int nq = (s + ATT_B - 1) / ATT_B;
    const bf16* dSh = dSb + (size_t)(bi * heads_t + head) * ds_pairs(nq, causal) * (ATT_B * ATT_B);
    const int myq = qt * ATT_B + grp * 32 + l32;
    f32x16 dq[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) dq[dt] = zero16();

    const int ntiles = causal ? qt + 1 : nq;
    const int niter = (ntiles + 1) / 2;
    AttTileRegs<D> kr;
    const auto krs = att_rsrc<D>(Kp, ld, s);
    // The dS blocks of key tiles 2it, 2it + 1, four 16-byte chunks per thread (a block past the last
    // key tile reads zeros). Chunk c = ((g*2 + qh)*2 + kk)*64 + 32h + k of a block holds key 32g + k
    // and queries 32qh + 16kk + 4h + 0..3 and + 8 .. + 11 (the dK/dV kernel's accumulator order);
    // it goes to the [key][query] tile as two 8-byte pieces. Pass u = 4j + wave covers block u/8,
    // key group (u/4)%2, keys 8(u%4) .. + 7; lane = key%8 + 8 (h + 2qh + 4kk), so a wave reads
    // whole 128-byte lines and the 8-byte LDS writes of each half-wave fall on distinct banks.
    u32x4 sr[4];
    auto ds_coords = [&](int j, int& blk, int& key, int& q0, int& c) {
        const int u = 4 * j + wave, g = (u >> 2) & 1, k = (u & 3) * 8 + (lane & 7), cb = lane >> 3;
        const int hh = cb & 1, qh = (cb >> 1) & 1, kk = cb >> 2;
        blk = u >> 3;
        key = g * 32 + k;
        q0 = qh * 32 + 16 * kk + 4 * hh;
        c = ((g * 2 + qh) * 2 + kk) * 64 + 32 * hh + k;
    };
    auto fetch_ds = [&](int it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int blk, key, q0, c;
            ds_coords(j, blk, key, q0, c);
            const int kt = 2 * it + blk;
            sr[j] = kt < ntiles ? *(const u32x4*)(dSh + (size_t)ds_pair(kt, qt, nq, causal) * (ATT_B * ATT_B) + c * 8)
                                : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto stash_ds = [&]() {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int blk, key, q0, c;
            ds_coords(j, blk, key, q0, c);
            bf16* t = Sb + blk * ATT_B * ATT_B;
            *(u32x2*)(t + att_off<ATT_B>(key, q0)) = u32x2{sr[j][0], sr[j][1]};
            *(u32x2*)(t + att_off<ATT_B>(key, q0 + 8)) = u32x2{sr[j][2], sr[j][3]};
        }
    };
    if (niter > 0) {
        kr.load(krs, ld, 0, s, tid);
        fetch_ds(0);
        kr.store(Kb, tid);
        stash_ds();
    }
    __syncthreads();
    for (int it = 0; it < niter; ++it) {
        const bool more = it + 1 < niter;
        if (more) {
            kr.load(krs, ld, (it + 1) * 2 * ATT_B, s, tid);
            fetch_ds(it + 1);
        }
        if (2 * it + kp < ntiles) {
            const bf16* K = Kb + kp * ATT_B * D;
            const bf16* S = Sb + kp * ATT_B * ATT_B;
#pragma unroll
            for (int ks = 0; ks < ATT_B / 16; ++ks) {
                const bf16x8 dsf = frag_cols<ATT_B>(S, 16 * ks, grp * 32, lane);
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
                    dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols<D>(K, 16 * ks, dt * 32, lane), dsf, dq[dt],
                                                                     0, 0, 0);
            }
        }
        __syncthreads();
        if (more) {
            kr.store(Kb, tid);
            stash_ds();
        }
        __syncthreads();
    }
    constexpr int NV = D / 2;
    float* xch = (float*)Kb;
    static_assert(2 * NV * 64 * 4 <= 2 * ATT_B * D * 2, "exchange exceeds the tile buffers");
    if (kp == 1) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) xch_put<NV>(xch, grp, dt * 16 + v, lane, dq[dt][v]);
    }
    __syncthreads();
    if (kp == 0) {
        bf16* qp_ = dQKV + (tok0 + myq) * ld_dq + head * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) dq[dt][v] = (dq[dt][v] + xch_get<NV>(xch, grp, dt * 16 + v, lane)) * scale;
            if (myq < s) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    int d = dt * 32 + 8 * i + 4 * h;
                    *(u32x2*)(qp_ + d) = u32x2{pack_bf16x2(dq[dt][4 * i], dq[dt][4 * i + 1]),
                                               pack_bf16x2(dq[dt][4 * i + 2], dq[dt][4 * i + 3])};
                }
            }
        }
    }
    static_assert(ATT_B * (D + 4) * 4 <= sizeof(sm), "column-sum buffer exceeds the tile buffers");
    if (colpart) tile_colsum<D, D / 32>(dq, kp == 0, myq < s, grp * 32 + l32, lane, tid, (float*)sm,
                                        colpart + (size_t)(bi * nq + qt) * (3 * h_t) + head * D);
}

}  // namespace tp
