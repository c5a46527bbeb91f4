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
// in place and V^T is read from LDS in that order.
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
constexpr int ATT_B = 64;        // queries per block (fwd, dQ) / keys per block (dK dV)
constexpr int ATT_NT = 128;      // 2 waves, 32 rows each
constexpr int ATT_PAD_RM = 8;    // row-major tile padding (elements): 208-byte rows for D = 96
constexpr int ATT_PAD_T = 4;     // transposed tile padding: 136-byte rows

// Copy rows [r0, r0+64) x D of a strided bf16 matrix into LDS, zero-filling rows >= rows_valid.
// rm: row-major copy [64][D + ATT_PAD_RM]; tr: transposed copy [D][64 + ATT_PAD_T]. Either may be null.
template <int D>
__device__ __forceinline__ void att_load_tile(const bf16* __restrict__ src, int ld, int r0, int rows_valid,
                                              bf16 (*rm)[D + ATT_PAD_RM], bf16 (*tr)[ATT_B + ATT_PAD_T], int tid) {
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int TOTAL = ATT_B * CPR;
    for (int c = tid; c < TOTAL; c += ATT_NT) {
        int row = c / CPR, dc = c % CPR;
        u32x4 v = u32x4{0, 0, 0, 0};
        if (r0 + row < rows_valid) v = *(const u32x4*)(src + (size_t)(r0 + row) * ld + dc * 8);
        if (rm) *(u32x4*)&rm[row][dc * 8] = v;
        if (tr) {
            bf16x8 e = __builtin_bit_cast(bf16x8, v);
#pragma unroll
            for (int k = 0; k < 8; ++k) tr[dc * 8 + k][row] = e[k];
        }
    }
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& a, int base) {
    u32x4 u;
    u[0] = pack_bf16x2(a[base + 0], a[base + 1]);
    u[1] = pack_bf16x2(a[base + 2], a[base + 3]);
    u[2] = pack_bf16x2(a[base + 4], a[base + 5]);
    u[3] = pack_bf16x2(a[base + 6], a[base + 7]);
    return __builtin_bit_cast(bf16x8, u);
}

// A-operand fragment from a transposed LDS tile in the accumulator's k-order:
// row `row`, columns c0 + 4h + 0..3 and c0 + 8 + 4h + 0..3.
template <int W>
__device__ __forceinline__ bf16x8 frag_tr(const bf16 (*tr)[W], int row, int c0, int h) {
    u32x2 lo = *(const u32x2*)&tr[row][c0 + 4 * h];
    u32x2 hi = *(const u32x2*)&tr[row][c0 + 8 + 4 * h];
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int v = 0; v < 16; ++v) z[v] = 0.f;
    return z;
}

// ---------------------------------------------------------------------------------------------
// Forward. grid = (ceil(s/64) query tiles, heads_t, b); heavy (late) query tiles first.
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(ATT_NT) void attn_fwd_kernel(const bf16* __restrict__ QKV, int ld, int h_t, int s,
                                                          int heads_t, float scale_log2, int causal,
                                                          bf16* __restrict__ O, int ldo, float* __restrict__ lse) {
    __shared__ __attribute__((aligned(16))) bf16 Ks[ATT_B][D + ATT_PAD_RM];
    __shared__ __attribute__((aligned(16))) bf16 Vt[D][ATT_B + ATT_PAD_T];
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
    for (int kt = 0; kt < ntiles; ++kt) {
        const int k0 = kt * ATT_B;
        __syncthreads();
        att_load_tile<D>(Kp, ld, k0, s, Ks, nullptr, tid);
        att_load_tile<D>(Vp, ld, k0, s, nullptr, Vt, tid);
        __syncthreads();
        if (causal && k0 > q0w + 31) continue;  // every key of this tile is after every query of this wave

        f32x16 st[2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            st[sub] = zero16();
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                bf16x8 a = *(const bf16x8*)&Ks[sub * 32 + l32][ks * 16 + 8 * h];
                st[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], st[sub], 0, 0, 0);
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                int key = k0 + sub * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                float x = st[sub][v] * scale_log2;
                if ((causal && key > myq) || key >= s) x = -INFINITY;
                st[sub][v] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_i, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_i - m_use);
        float rs = 0.f;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float p = exp2f(st[sub][v] - m_use);
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
            for (int dt = 0; dt < D / 32; ++dt) {
                bf16x8 a = frag_tr<ATT_B + ATT_PAD_T>(Vt, dt * 32 + l32, 16 * ks, h);
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[dt], 0, 0, 0);
            }
        }
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
        if (h == 0) lse[((size_t)bi * heads_t + head) * s + myq] = (m_i + __log2f(l_i)) * kLn2;
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
// dK, dV. grid = (ceil(s/64) key tiles, heads_t, b). Wave w owns keys kt*64 + 32w .. +31.
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(ATT_NT) void attn_bwd_dkdv_kernel(const bf16* __restrict__ QKV, int ld, int h_t, int s,
                                                               int heads_t, const bf16* __restrict__ dO, int ld_do,
                                                               const float* __restrict__ lse,
                                                               const float* __restrict__ Dv, float scale_log2,
                                                               float scale, int causal, bf16* __restrict__ dQKV,
                                                               int ld_dq) {
    __shared__ __attribute__((aligned(16))) bf16 Qs[ATT_B][D + ATT_PAD_RM];
    __shared__ __attribute__((aligned(16))) bf16 dOs[ATT_B][D + ATT_PAD_RM];
    __shared__ __attribute__((aligned(16))) bf16 Qt[D][ATT_B + ATT_PAD_T];
    __shared__ __attribute__((aligned(16))) bf16 dOt[D][ATT_B + ATT_PAD_T];
    __shared__ float lse_s[ATT_B], D_s[ATT_B];
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
    for (int qt = causal ? kt : 0; qt < nqt; ++qt) {
        const int q0 = qt * ATT_B;
        __syncthreads();
        att_load_tile<D>(Qp, ld, q0, s, Qs, Qt, tid);
        att_load_tile<D>(dOp, ld_do, q0, s, dOs, dOt, tid);
        if (tid < ATT_B) {
            int q = q0 + tid;
            lse_s[tid] = (q < s) ? lsep[q] * kLog2e : INFINITY;
            D_s[tid] = (q < s) ? Dp[q] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int qs0 = q0 + sub * 32;
            if (causal && qs0 + 31 < kw0) continue;  // every query of this half precedes every key of this wave
            f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                bf16x8 a = *(const bf16x8*)&Qs[sub * 32 + l32][ks * 16 + 8 * h];
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[ks], sacc, 0, 0, 0);
                bf16x8 g = *(const bf16x8*)&dOs[sub * 32 + l32][ks * 16 + 8 * h];
                dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(g, vf[ks], dpacc, 0, 0, 0);
            }
            f32x16 p, ds;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                int qi = sub * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                int q = q0 + qi;
                float pv = exp2f(sacc[v] * scale_log2 - lse_s[qi]);
                if ((causal && mykey > q) || mykey >= s) pv = 0.f;
                p[v] = pv;
                ds[v] = pv * (dpacc[v] - D_s[qi]);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 pb = pack8(p, 8 * kk), dsb = pack8(ds, 8 * kk);
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    bf16x8 ag = frag_tr<ATT_B + ATT_PAD_T>(dOt, dt * 32 + l32, sub * 32 + 16 * kk, h);
                    dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag, pb, dv[dt], 0, 0, 0);
                    bf16x8 aq = frag_tr<ATT_B + ATT_PAD_T>(Qt, dt * 32 + l32, sub * 32 + 16 * kk, h);
                    dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, dsb, dk[dt], 0, 0, 0);
                }
            }
        }
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
// dQ. grid = (ceil(s/64) query tiles, heads_t, b); heavy tiles first. Wave w owns 32 queries.
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(ATT_NT) void attn_bwd_dq_kernel(const bf16* __restrict__ QKV, int ld, int h_t, int s,
                                                             int heads_t, const bf16* __restrict__ dO, int ld_do,
                                                             const float* __restrict__ lse,
                                                             const float* __restrict__ Dv, float scale_log2,
                                                             float scale, int causal, bf16* __restrict__ dQKV,
                                                             int ld_dq) {
    __shared__ __attribute__((aligned(16))) bf16 Ks[ATT_B][D + ATT_PAD_RM];
    __shared__ __attribute__((aligned(16))) bf16 Vs[ATT_B][D + ATT_PAD_RM];
    __shared__ __attribute__((aligned(16))) bf16 Kt[D][ATT_B + ATT_PAD_T];
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
    for (int kt = 0; kt < ntiles; ++kt) {
        const int k0 = kt * ATT_B;
        __syncthreads();
        att_load_tile<D>(Kp, ld, k0, s, Ks, Kt, tid);
        att_load_tile<D>(Vp, ld, k0, s, Vs, nullptr, tid);
        __syncthreads();
        if (causal && k0 > q0w + 31) continue;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            if (causal && k0 + sub * 32 > q0w + 31) continue;
            f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                bf16x8 a = *(const bf16x8*)&Ks[sub * 32 + l32][ks * 16 + 8 * h];
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc, 0, 0, 0);
                bf16x8 c = *(const bf16x8*)&Vs[sub * 32 + l32][ks * 16 + 8 * h];
                dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c, gf[ks], dpacc, 0, 0, 0);
            }
            f32x16 ds;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                int key = k0 + sub * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                float pv = exp2f(sacc[v] * scale_log2 - lse2);
                if ((causal && key > myq) || key >= s) pv = 0.f;
                ds[v] = pv * (dpacc[v] - Dq);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 dsb = pack8(ds, 8 * kk);
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    bf16x8 a = frag_tr<ATT_B + ATT_PAD_T>(Kt, dt * 32 + l32, sub * 32 + 16 * kk, h);
                    dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb, dq[dt], 0, 0, 0);
                }
            }
        }
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
