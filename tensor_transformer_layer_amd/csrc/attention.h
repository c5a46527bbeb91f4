// Causal multi-head attention for one rank's heads on gfx950, forward and backward.
//
// Per (sequence, head): S = Q K^T / sqrt(d), masked, P = softmax(S), O = P V, saved lse.
// Head width D = 96 is handled as 6 k-steps of 16 (scores) and 3 tiles of 32 (outputs).
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
// Backward: D = rowsum(dO * O); dK/dV kernel owns 64 keys per block and loops over query tiles;
// dQ kernel owns 64 queries per block and loops over key tiles. Both recompute P from lse.
// No atomics: every output element is written by exactly one lane.
#pragma once
#include "common.h"

namespace tp {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int ATT_B = 64;        // queries per block (fwd, dQ) / keys per block (dK dV), rows per tile
constexpr int ATT_NT = 128;      // 2 waves, 32 rows each

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// LDS tiles are row-major [64][D] bf16 with the 16-byte chunk index XOR-swizzled by
// (row >> 2) & 3. Two access patterns are conflict-free on it: a 128-bit read of 8 consecutive
// columns by 16 consecutive rows (MFMA operand with K along the columns), and the transposing
// 64-bit read of a 4-row x 16-column block per 16-lane group (MFMA operand with K along the rows).
template <int D>
__device__ __forceinline__ int att_off(int row, int col) {
    return row * D + ((((col >> 3) ^ ((row >> 2) & 3)) << 3) | (col & 7));
}

// Register-staged copy of rows [r0, r0+64) x D of a strided bf16 matrix (rows >= valid read 0).
template <int D>
struct AttTileRegs {
    static constexpr int CPR = D / 8, N = ATT_B * CPR / ATT_NT;
    static_assert((ATT_B * CPR) % ATT_NT == 0, "tile/threads mismatch");
    u32x4 v[N];
    __device__ __forceinline__ void load(const bf16* __restrict__ src, int ld, int r0, int valid, int tid) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            int c = tid + i * ATT_NT, row = c / CPR, dc = c % CPR;
            v[i] = (r0 + row < valid) ? *(const u32x4*)(src + (size_t)(r0 + row) * ld + dc * 8) : u32x4{0, 0, 0, 0};
        }
    }
    __device__ __forceinline__ void store(bf16* tile, int tid) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            int c = tid + i * ATT_NT, row = c / CPR, dc = c % CPR;
            *(u32x4*)(tile + att_off<D>(row, dc * 8)) = v[i];
        }
    }
};

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

// ---------------------------------------------------------------------------------------------
// Forward. grid = (ceil(s/64) query tiles, heads_t, b); heavy (late) query tiles first.
// K and V tiles are double-buffered; the next tile's global loads are in flight during the
// current tile's MFMAs. Only tiles that cross the diagonal (or the sequence end) are masked.
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(ATT_NT) void attn_fwd_kernel(const bf16* __restrict__ QKV, int ld, int h_t, int s,
                                                          int heads_t, float scale_log2, int causal,
                                                          bf16* __restrict__ O, int ldo, float* __restrict__ lse) {
    __shared__ __attribute__((aligned(16))) bf16 Kb[2][ATT_B * D];
    __shared__ __attribute__((aligned(16))) bf16 Vb[2][ATT_B * D];
    const int qt = gridDim.x - 1 - blockIdx.x, head = blockIdx.y, bi = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const size_t tok0 = (size_t)bi * s;
    const bf16* Qp = QKV + tok0 * ld + head * D;
    const bf16* Kp = QKV + tok0 * ld + h_t + head * D;
    const bf16* Vp = QKV + tok0 * ld + 2 * h_t + head * D;
    const int q0w = qt * ATT_B + wave * 32;
    const int myq = q0w + l32;

    bf16x8 qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        u32x4 v = u32x4{0, 0, 0, 0};
        if (myq < s) v = *(const u32x4*)(Qp + (size_t)myq * ld + ks * 16 + 8 * h);
        qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] = zero16();
    float m_i = -INFINITY, l_i = 0.f;

    const int kv_end = causal ? min(s, (qt + 1) * ATT_B) : s;
    const int ntiles = (kv_end + ATT_B - 1) / ATT_B;
    AttTileRegs<D> kr, vr;
    if (ntiles > 0) {
        kr.load(Kp, ld, 0, s, tid);
        vr.load(Vp, ld, 0, s, tid);
        kr.store(Kb[0], tid);
        vr.store(Vb[0], tid);
    }
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
        const int k0 = kt * ATT_B, buf = kt & 1;
        const bool more = kt + 1 < ntiles;
        if (more) {
            kr.load(Kp, ld, k0 + ATT_B, s, tid);
            vr.load(Vp, ld, k0 + ATT_B, s, tid);
        }
        if (!(causal && k0 > q0w + 31)) {   // some key of this tile is visible to this wave
            const bf16* K = Kb[buf];
            const bf16* V = Vb[buf];
            const bool need_mask = (causal && k0 + ATT_B - 1 > q0w) || (k0 + ATT_B > s);
            f32x16 st[2];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                st[sub] = zero16();
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks)
                    st[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<D>(K, sub * 32, ks * 16, lane), qf[ks],
                                                                      st[sub], 0, 0, 0);
            }
            if (need_mask) {
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        int key = k0 + sub * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                        if ((causal && key > myq) || key >= s) st[sub][v] = -INFINITY;
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
            const float alpha = exp2f(m_i - m_use);
            float rs = 0.f;
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    float p = exp2f(fmaf(st[sub][v], scale_log2, -m_use));
                    st[sub][v] = p;
                    rs += p;
                }
            rs += __shfl_xor(rs, 32);
            l_i = l_i * alpha + rs;
            m_i = m_new;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
#pragma unroll
            for (int ks = 0; ks < ATT_B / 16; ++ks) {
                bf16x8 pb = pack8(st[ks >> 1], 8 * (ks & 1));
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols<D>(V, 16 * ks, dt * 32, lane), pb, o[dt],
                                                                    0, 0, 0);
            }
        }
        if (more) {   // the other buffer was last read before the previous barrier
            kr.store(Kb[buf ^ 1], tid);
            vr.store(Vb[buf ^ 1], tid);
        }
        __syncthreads();
    }
    if (myq < s) {
        const float inv = 1.0f / l_i;
        bf16* op = O + (tok0 + myq) * ldo + head * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int d = dt * 32 + 8 * i + 4 * h;
                u32x2 w = u32x2{pack_bf16x2(o[dt][4 * i] * inv, o[dt][4 * i + 1] * inv),
                                pack_bf16x2(o[dt][4 * i + 2] * inv, o[dt][4 * i + 3] * inv)};
                *(u32x2*)(op + d) = w;
            }
        if (h == 0) lse[((size_t)bi * heads_t + head) * s + myq] = (m_i + log2f(l_i)) * kLn2;
    }
}

// ---------------------------------------------------------------------------------------------
// D[b, head, q] = sum_d dO[q, head*D + d] * O[q, head*D + d]   (fp32)
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dot_kernel(const bf16* __restrict__ dO, const bf16* __restrict__ O,
                                                           int ld, int b, int s, int heads_t, float* __restrict__ Dv) {
    size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    size_t total = (size_t)b * s * heads_t;
    if (idx >= total) return;
    int head = (int)(idx % heads_t);
    size_t tok = idx / heads_t;
    const bf16* a = dO + tok * ld + head * D;
    const bf16* c = O + tok * ld + head * D;
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < D; k += 8) {
        bf16x8 x = *(const bf16x8*)(a + k), y = *(const bf16x8*)(c + k);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)x[e] * (float)y[e];
    }
    int bi = (int)(tok / s), pos = (int)(tok % s);
    Dv[((size_t)bi * heads_t + head) * s + pos] = acc;
}

// ---------------------------------------------------------------------------------------------
// dK, dV. grid = (ceil(s/64) key tiles, heads_t, b). Wave w owns keys kt*64 + 32w .. +31 and loops
// over the query tiles that can see them; Q and dO tiles (and lse, D) are double-buffered.
//   S = Q K^T, P = exp2(S*c - lse2), dP = dO V^T, dS = P (dP - D)      (query rows x own keys)
//   dV^T += dO^T P,  dK^T += Q^T dS                                     (transposing reads)
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(ATT_NT) void attn_bwd_dkdv_kernel(const bf16* __restrict__ QKV, int ld, int h_t, int s,
                                                               int heads_t, const bf16* __restrict__ dO, int ld_do,
                                                               const float* __restrict__ lse,
                                                               const float* __restrict__ Dv, float scale_log2,
                                                               float scale, int causal, bf16* __restrict__ dQKV,
                                                               int ld_dq) {
    __shared__ __attribute__((aligned(16))) bf16 Qb[2][ATT_B * D];
    __shared__ __attribute__((aligned(16))) bf16 Gb[2][ATT_B * D];
    __shared__ float lse_s[2][ATT_B], D_s[2][ATT_B];
    const int kt = blockIdx.x, head = blockIdx.y, bi = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const size_t tok0 = (size_t)bi * s;
    const bf16* Qp = QKV + tok0 * ld + head * D;
    const bf16* Kp = QKV + tok0 * ld + h_t + head * D;
    const bf16* Vp = QKV + tok0 * ld + 2 * h_t + head * D;
    const bf16* dOp = dO + tok0 * ld_do + head * D;
    const float* lsep = lse + ((size_t)bi * heads_t + head) * s;
    const float* Dp = Dv + ((size_t)bi * heads_t + head) * s;
    const int kw0 = kt * ATT_B + wave * 32;
    const int mykey = kw0 + l32;

    bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        u32x4 a = u32x4{0, 0, 0, 0}, c = u32x4{0, 0, 0, 0};
        if (mykey < s) {
            a = *(const u32x4*)(Kp + (size_t)mykey * ld + ks * 16 + 8 * h);
            c = *(const u32x4*)(Vp + (size_t)mykey * ld + ks * 16 + 8 * h);
        }
        kf[ks] = __builtin_bit_cast(bf16x8, a);
        vf[ks] = __builtin_bit_cast(bf16x8, c);
    }
    f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) { dk[dt] = zero16(); dv[dt] = zero16(); }

    const int nqt = (s + ATT_B - 1) / ATT_B;
    const int qt0 = causal ? kt : 0;
    AttTileRegs<D> qr, gr;
    float lse_r = INFINITY, d_r = 0.f;
    auto fetch = [&](int qt) {
        const int q0 = qt * ATT_B;
        qr.load(Qp, ld, q0, s, tid);
        gr.load(dOp, ld_do, q0, s, tid);
        if (tid < ATT_B) {
            int q = q0 + tid;
            lse_r = (q < s) ? lsep[q] * kLog2e : INFINITY;
            d_r = (q < s) ? Dp[q] : 0.f;
        }
    };
    auto stash = [&](int buf) {
        qr.store(Qb[buf], tid);
        gr.store(Gb[buf], tid);
        if (tid < ATT_B) { lse_s[buf][tid] = lse_r; D_s[buf][tid] = d_r; }
    };
    if (qt0 < nqt) { fetch(qt0); stash(0); }
    __syncthreads();
    for (int qt = qt0; qt < nqt; ++qt) {
        const int q0 = qt * ATT_B, buf = (qt - qt0) & 1;
        const bool more = qt + 1 < nqt;
        if (more) fetch(qt + 1);
        const bf16* Q = Qb[buf];
        const bf16* Gt = Gb[buf];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int qs0 = q0 + sub * 32;
            if (causal && qs0 + 31 < kw0) continue;  // every query of this half precedes every key of this wave
            const bool need_mask = (causal && qs0 < kw0 + 31) || (qs0 + 32 > s) || (kw0 + 32 > s);
            f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<D>(Q, sub * 32, ks * 16, lane), kf[ks], sacc, 0, 0, 0);
                dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<D>(Gt, sub * 32, ks * 16, lane), vf[ks], dpacc, 0, 0, 0);
            }
            f32x16 p, ds;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                int qi = sub * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                float pv = exp2f(fmaf(sacc[v], scale_log2, -lse_s[buf][qi]));
                if (need_mask) {
                    int q = q0 + qi;
                    if ((causal && mykey > q) || mykey >= s) pv = 0.f;
                }
                p[v] = pv;
                ds[v] = pv * (dpacc[v] - D_s[buf][qi]);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 pb = pack8(p, 8 * kk), dsb = pack8(ds, 8 * kk);
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols<D>(Gt, sub * 32 + 16 * kk, dt * 32, lane), pb,
                                                                     dv[dt], 0, 0, 0);
                    dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols<D>(Q, sub * 32 + 16 * kk, dt * 32, lane), dsb,
                                                                     dk[dt], 0, 0, 0);
                }
            }
        }
        if (more) stash(buf ^ 1);
        __syncthreads();
    }
    if (mykey < s) {
        bf16* kp = dQKV + (tok0 + mykey) * ld_dq + h_t + head * D;
        bf16* vp = dQKV + (tok0 + mykey) * ld_dq + 2 * h_t + head * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int d = dt * 32 + 8 * i + 4 * h;
                *(u32x2*)(kp + d) = u32x2{pack_bf16x2(dk[dt][4 * i] * scale, dk[dt][4 * i + 1] * scale),
                                          pack_bf16x2(dk[dt][4 * i + 2] * scale, dk[dt][4 * i + 3] * scale)};
                *(u32x2*)(vp + d) = u32x2{pack_bf16x2(dv[dt][4 * i], dv[dt][4 * i + 1]),
                                          pack_bf16x2(dv[dt][4 * i + 2], dv[dt][4 * i + 3])};
            }
    }
}

// ---------------------------------------------------------------------------------------------
// dQ. grid = (ceil(s/64) query tiles, heads_t, b); heavy tiles first. Wave w owns 32 queries and
// loops over the key tiles they can see; K and V tiles are double-buffered.
//   S^T = K Q^T, P^T = exp2(S^T*c - lse2), dP^T = V dO^T, dS^T = P^T (dP^T - D); dQ^T += K^T dS^T
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(ATT_NT) void attn_bwd_dq_kernel(const bf16* __restrict__ QKV, int ld, int h_t, int s,
                                                             int heads_t, const bf16* __restrict__ dO, int ld_do,
                                                             const float* __restrict__ lse,
                                                             const float* __restrict__ Dv, float scale_log2,
                                                             float scale, int causal, bf16* __restrict__ dQKV,
                                                             int ld_dq) {
    __shared__ __attribute__((aligned(16))) bf16 Kb[2][ATT_B * D];
    __shared__ __attribute__((aligned(16))) bf16 Vb[2][ATT_B * D];
    const int qt = gridDim.x - 1 - blockIdx.x, head = blockIdx.y, bi = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const size_t tok0 = (size_t)bi * s;
    const bf16* Qp = QKV + tok0 * ld + head * D;
    const bf16* Kp = QKV + tok0 * ld + h_t + head * D;
    const bf16* Vp = QKV + tok0 * ld + 2 * h_t + head * D;
    const bf16* dOp = dO + tok0 * ld_do + head * D;
    const int q0w = qt * ATT_B + wave * 32;
    const int myq = q0w + l32;
    const float lse2 = (myq < s) ? lse[((size_t)bi * heads_t + head) * s + myq] * kLog2e : INFINITY;
    const float Dq = (myq < s) ? Dv[((size_t)bi * heads_t + head) * s + myq] : 0.f;

    bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        u32x4 a = u32x4{0, 0, 0, 0}, c = u32x4{0, 0, 0, 0};
        if (myq < s) {
            a = *(const u32x4*)(Qp + (size_t)myq * ld + ks * 16 + 8 * h);
            c = *(const u32x4*)(dOp + (size_t)myq * ld_do + ks * 16 + 8 * h);
        }
        qf[ks] = __builtin_bit_cast(bf16x8, a);
        gf[ks] = __builtin_bit_cast(bf16x8, c);
    }
    f32x16 dq[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) dq[dt] = zero16();

    const int kv_end = causal ? min(s, (qt + 1) * ATT_B) : s;
    const int ntiles = (kv_end + ATT_B - 1) / ATT_B;
    AttTileRegs<D> kr, vr;
    if (ntiles > 0) {
        kr.load(Kp, ld, 0, s, tid);
        vr.load(Vp, ld, 0, s, tid);
        kr.store(Kb[0], tid);
        vr.store(Vb[0], tid);
    }
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
        const int k0 = kt * ATT_B, buf = kt & 1;
        const bool more = kt + 1 < ntiles;
        if (more) {
            kr.load(Kp, ld, k0 + ATT_B, s, tid);
            vr.load(Vp, ld, k0 + ATT_B, s, tid);
        }
        const bf16* K = Kb[buf];
        const bf16* V = Vb[buf];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int ks0 = k0 + sub * 32;
            if (causal && ks0 > q0w + 31) continue;
            const bool need_mask = (causal && ks0 + 31 > q0w) || (ks0 + 32 > s);
            f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<D>(K, sub * 32, ks * 16, lane), qf[ks], sacc, 0, 0, 0);
                dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_rows<D>(V, sub * 32, ks * 16, lane), gf[ks], dpacc, 0, 0, 0);
            }
            f32x16 ds;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float pv = exp2f(fmaf(sacc[v], scale_log2, -lse2));
                if (need_mask) {
                    int key = ks0 + 8 * (v >> 2) + 4 * h + (v & 3);
                    if ((causal && key > myq) || key >= s) pv = 0.f;
                }
                ds[v] = pv * (dpacc[v] - Dq);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 dsb = pack8(ds, 8 * kk);
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
                    dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_cols<D>(K, sub * 32 + 16 * kk, dt * 32, lane), dsb,
                                                                     dq[dt], 0, 0, 0);
            }
        }
        if (more) {
            kr.store(Kb[buf ^ 1], tid);
            vr.store(Vb[buf ^ 1], tid);
        }
        __syncthreads();
    }
    if (myq < s) {
        bf16* qp = dQKV + (tok0 + myq) * ld_dq + head * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int d = dt * 32 + 8 * i + 4 * h;
                *(u32x2*)(qp + d) = u32x2{pack_bf16x2(dq[dt][4 * i] * scale, dq[dt][4 * i + 1] * scale),
                                          pack_bf16x2(dq[dt][4 * i + 2] * scale, dq[dt][4 * i + 3] * scale)};
            }
    }
}

}  // namespace tp
