// Vocabulary-parallel fused logits GEMM + cross-entropy statistics for gfx950.
//
// The GEMM computes the transposed logits C[v][n] = E_r[v] . X[n] (vocab rows on M, tokens on N),
// so an MFMA accumulator lane holds ONE token and 16 vocabulary rows: the per-token max, argmax,
// sum of exponentials and target pick-out are in-lane, then one exchange with lane ^ 32, then a
// merge of the block's wave rows through LDS. Each output tile writes one 16-byte partial per
// token; logits never reach memory. The merge of a token's tiles (in tile order) and of the ranks
// into the loss are in xent.hip.
#pragma once
#include <climits>
#include "common.h"
#include "gemm.h"

namespace tp {

struct XentPartial {
    float mx;   // max logit over the tile's valid rows (-inf if none)
    float se;   // sum of exp(logit - mx) over the tile's valid rows
    float tv;   // target logit if the target row is in the tile, else 0
    int am;     // local row of mx, lowest on ties (INT_MAX if none)
};

__device__ __forceinline__ void xent_better(float& mx, int& am, float omx, int oam) {
    if (omx > mx || (omx == mx && oam < am)) { mx = omx; am = oam; }
}

// Merge two (max, sumexp) pairs.
__device__ __forceinline__ void xent_merge_se(float& mx, float& se, float omx, float ose) {
    if (omx == -INFINITY) return;
    if (mx == -INFINITY) { mx = omx; se = ose; return; }
    float m = fmaxf(mx, omx);
    se = se * expf(mx - m) + ose * expf(omx - m);
    mx = m;
}

struct EpiXent {
    static constexpr bool kVec8 = false;
    XentPartial* part;        // [tiles_m][N]
    const int32_t* targets;   // [N] global ids
    int col0;                 // global id of local row 0 (r * V_t)
    int Vreal;
    int mask;                 // 1: rows with col0 + row >= Vreal are -inf
    int row0;                 // added to the reported argmax row (launches over a slice of the shard's rows)
    __device__ __forceinline__ void set_split(int) {}

    template <class C>
    __device__ __forceinline__ void apply(f32x16 (&acc)[C::TM][C::TN], int m0, int n0, int mw0, int nw0, int lane,
                                          int M, int N, char* smem) const {
        XentPartial* red = (XentPartial*)smem;   // [WGM][BN]; the main loop ended on a barrier
        const int h = lane >> 5, l32 = lane & 31;
        const int wm = (mw0 - m0) / C::WM;
        // a wave whose rows are all inside M and unmasked skips the per-row validity tests; a
        // lane visits its rows in increasing order, so a strict > keeps the lowest row on ties
        const bool full = (mw0 + C::WM <= M) && (!mask || col0 + mw0 + C::WM <= Vreal);
        constexpr float kL2e = 1.4426950408889634f;
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int nloc = (nw0 - n0) + j * 32 + l32;
            const int n = n0 + nloc;
            const int trow = (n < N) ? targets[n] - col0 : -1;
            float mx = -INFINITY, tv = 0.f;
            int am = INT_MAX;
            if (full) {
#pragma unroll
                for (int i = 0; i < C::TM; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int row = mw0 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                        const float x = acc[i][j][v];
                        if (x > mx) { mx = x; am = row; }
                        tv = (row == trow) ? x : tv;
                    }
            } else {
#pragma unroll
                for (int i = 0; i < C::TM; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int row = mw0 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                        const bool valid = row < M && (!mask || col0 + row < Vreal);
                        const float x = acc[i][j][v];
                        if (valid && x > mx) { mx = x; am = row; }
                        if (row == trow && row < M) tv = x;
                    }
            }
            xent_better(mx, am, __shfl_xor(mx, 32), __shfl_xor(am, 32));
            tv += __shfl_xor(tv, 32);
            float se = 0.f;
            if (mx != -INFINITY) {
                const float nb = -mx * kL2e;
#pragma unroll
                for (int i = 0; i < C::TM; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int row = mw0 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                        const bool valid = full || (row < M && (!mask || col0 + row < Vreal));
                        // hardware exp2: terms below 2^-126 of the max flush to zero
                        if (valid) se += __builtin_amdgcn_exp2f(fmaf(acc[i][j][v], kL2e, nb));
                    }
            }
            se += __shfl_xor(se, 32);
            if (h == 0) red[wm * C::BN + nloc] = XentPartial{mx, se, tv, am};
        }
        __syncthreads();
        const int tm = m0 / C::BM;
        for (int nl = threadIdx.x; nl < C::BN; nl += C::NT) {
            int n = n0 + nl;
            if (n >= N) continue;
            XentPartial p = red[nl];
#pragma unroll
            for (int w = 1; w < C::WGM; ++w) {
                XentPartial q = red[w * C::BN + nl];
                float mx = p.mx;
                int am = p.am;
                xent_better(mx, am, q.mx, q.am);
                xent_merge_se(p.mx, p.se, q.mx, q.se);
                p.am = am;
                p.tv += q.tv;
            }
            if (p.am != INT_MAX) p.am += row0;
            part[(size_t)tm * N + n] = p;
        }
    }
};

// ---------------------------------------------------------------------------------------------
// Logits gradient of the vocabulary-parallel cross-entropy (the backward of the fused logits). The
// GEMM recomputes C[v][n] = E_r[v] . X[n]; the epilogue turns each logit into
//     dl = dloss_n * (exp(y - M_n) / S_n - [v == target_n]),     0 on masked padding rows,
// with the merged (all-rank) per-token max M and sum S, and stores it twice in bf16: token-major
// DT[n][v] straight from the accumulator layout (a lane holds 4 consecutive vocabulary rows of
// one token: 8-byte stores) and vocab-major D[v][n] through the staged row-major epilogue. The two
// copies feed dX_r = DT E_r and dE_r = D X, both with a K-contiguous A operand.
// ---------------------------------------------------------------------------------------------
struct EpiXentGrad {
    static constexpr bool kVec8 = false;
    bf16* D; int ldd;          // [Vt][ldd], ldd >= N, multiple of 8
    bf16* DT; int ldt;         // [N][ldt], ldt = Vt
    const float* Mx; const float* Sx; const float* g; const int32_t* targets;
    int col0, Vreal, mask;
    __device__ __forceinline__ void set_split(int) {}

    struct StoreRows {   // op8 for the staged pass: 8 consecutive tokens of one vocabulary row
        bf16* out; int ld;
        __device__ __forceinline__ void op8(int r, int c, float (&v)[8]) const { store8(out + (size_t)r * ld + c, v); }
    };

    template <class C>
    __device__ __forceinline__ void apply(f32x16 (&acc)[C::TM][C::TN], int m0, int n0, int mw0, int nw0, int lane,
                                          int M, int N, char* smem) const {
        const int h = lane >> 5, l32 = lane & 31;
        constexpr float kL2e = 1.4426950408889634f;
        const bool full = (mw0 + C::WM <= M) && (!mask || col0 + mw0 + C::WM <= Vreal);
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int n = nw0 + j * 32 + l32;
            const bool vn = n < N;
            const float nb = vn ? -Mx[n] * kL2e : 0.f;
            const float inv = vn ? 1.0f / Sx[n] : 0.f;
            const float gn = vn ? g[n] : 0.f;
            const int trow = vn ? targets[n] - col0 : -1;
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = mw0 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                    float p = __builtin_amdgcn_exp2f(fmaf(acc[i][j][v], kL2e, nb)) * inv;
                    if (!full && mask && col0 + row >= Vreal) p = 0.f;
                    acc[i][j][v] = gn * (p - (row == trow ? 1.0f : 0.0f));
                }
            if (vn) {
                bf16* dt = DT + (size_t)n * ldt;
#pragma unroll
                for (int i = 0; i < C::TM; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int row = mw0 + i * 32 + 8 * q + 4 * h;
                        if (row < M)
                            *(u32x2*)(dt + row) = u32x2{pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                                        pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
                    }
            }
        }
        apply_staged<C>(StoreRows{D, ldd}, acc, mw0, nw0, lane, (int)(threadIdx.x >> 6), M, N, smem);
    }
};

}  // namespace tp
