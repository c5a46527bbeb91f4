// Vocabulary-parallel input embedding ("Megatron-LM ..." paper digest, §3.4, Input Embedding
// Parallelism): rank r holds rows r*Vt .. (r+1)*Vt - 1 of the table; its partial output is the
// looked-up row for tokens it owns and a zero row for every other token (g sums the partials).
//
// Forward: one thread per 8 columns of a token row, a 16-byte copy or a 16-byte zero store.
// Backward, deterministic (no float atomics): dE_r[v] = sum over the tokens i with ids[i] = r*Vt + v
// of dX[i], in token order. A stable counting sort over chunks of 128 tokens, then ordered sums:
//   1. emb_rank_kernel (one workgroup per chunk): each owned token's rank among the earlier tokens
//      of its chunk with the same id, and the chunk's count per table row, written by the last
//      such token (the chunk histogram H[chunk][v], zero elsewhere).
//   2. emb_prefix_kernel (one thread per table row): the exclusive prefix of H over chunks, in
//      place, and the row totals; emb_scan_kernel (one workgroup): their exclusive scan over rows,
//      the segment starts.
//   3. emb_place_kernel: token i goes to start[v] + H[chunk][v] + rank_i.
//   4. emb_segsum_kernel (one workgroup per table row and 2048-column slice): sums the segment's
//      dX rows in token order in fp32 and writes (or adds to) dE_r's row; rows without tokens get
//      zeros (or are left as they are when accumulating).
#include <algorithm>

#include "launch.h"
#include "common.h"

namespace tp {

template <typename T>
__global__ __launch_bounds__(256) void emb_fwd_kernel(int N, int h, int Vt, int r, const int32_t* __restrict__ ids,
                                                      const T* __restrict__ E, T* __restrict__ out) {
    const int cpr = h >> 3;
    const long q = (long)blockIdx.x * 256 + threadIdx.x;
    if (q >= (long)N * cpr) return;
    const int tok = (int)(q / cpr), c = (int)(q - (long)tok * cpr) * 8;
    const long local = (long)ids[tok] - (long)r * Vt;
    float f[8];
    if (local >= 0 && local < Vt) {
        load8(E + (size_t)local * h + c, f);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = 0.0f;
    }
    store8(out + (size_t)tok * h + c, f);
}

constexpr int EMB_CHUNK = 128;

// local table row of token i on rank r, or -1
__device__ __forceinline__ int emb_local(const int32_t* ids, int i, int N, long base, int Vt) {
    if (i >= N) return -1;
    const long l = (long)ids[i] - base;
    return (l >= 0 && l < Vt) ? (int)l : -1;
}

__global__ __launch_bounds__(EMB_CHUNK) void emb_rank_kernel(int N, int Vt, int r, const int32_t* __restrict__ ids,
                                                             int* __restrict__ H, int* __restrict__ rank) {
    __shared__ int chunk[EMB_CHUNK];
    const int tid = threadIdx.x, i = blockIdx.x * EMB_CHUNK + tid;
    int* Hb = H + (size_t)blockIdx.x * Vt;
    for (int v = tid; v < Vt; v += EMB_CHUNK) Hb[v] = 0;
    const int l = emb_local(ids, i, N, (long)r * Vt, Vt);
    chunk[tid] = l;
    __syncthreads();   // also orders the zero stores before the count stores below
    if (l < 0) return;
    int before = 0, after = 0;
    for (int j = 0; j < EMB_CHUNK; ++j) {
        const int same = chunk[j] == l;
        before += (j < tid) & same;
        after += (j > tid) & same;
    }
    rank[i] = before;
    if (after == 0) Hb[l] = before + 1;
}

// One thread per table row (coalesced over rows): the exclusive prefix of H[., v] over chunks, in
// place, and the row total into start[v].
__global__ __launch_bounds__(256) void emb_prefix_kernel(int nchunks, int Vt, int* __restrict__ H,
                                                         int* __restrict__ start) {
    const int v = blockIdx.x * 256 + threadIdx.x;
    if (v >= Vt) return;
    int acc = 0;
    // 16 independent loads in flight, then the running sum over them
    for (int b0 = 0; b0 < nchunks; b0 += 16) {
        int c[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) c[j] = (b0 + j < nchunks) ? H[(size_t)(b0 + j) * Vt + v] : 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (b0 + j < nchunks) H[(size_t)(b0 + j) * Vt + v] = acc;
            acc += c[j];
        }
    }
    start[v] = acc;
}

// One workgroup of 1024 threads: exclusive scan of the row totals in start[0..Vt) (contiguous runs
// per thread, then a block scan of the run sums); start[Vt] = all owned tokens.
__global__ __launch_bounds__(1024) void emb_scan_kernel(int Vt, int* __restrict__ start) {
    __shared__ int wsum[16];
    const int tid = threadIdx.x;
    const int per = (Vt + 1023) / 1024;
    const int lo = min(Vt, tid * per), hi = min(Vt, lo + per);
    int run = 0;
    for (int v = lo; v < hi; ++v) run += start[v];
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if ((tid & 63) >= o) incl += y;
    }
    if ((tid & 63) == 63) wsum[tid >> 6] = incl;
    __syncthreads();
    int acc = incl - run;
    for (int w = 0; w < (tid >> 6); ++w) acc += wsum[w];
    for (int v = lo; v < hi; ++v) {
        const int c = start[v];
        start[v] = acc;
        acc += c;
    }
    if (tid == 1023) start[Vt] = acc;
}

__global__ __launch_bounds__(EMB_CHUNK) void emb_place_kernel(int N, int Vt, int r, const int32_t* __restrict__ ids,
                                                              const int* __restrict__ H, const int* __restrict__ rank,
                                                              const int* __restrict__ start, int* __restrict__ order) {
    const int i = blockIdx.x * EMB_CHUNK + threadIdx.x;
    const int l = emb_local(ids, i, N, (long)r * Vt, Vt);
    if (l < 0) return;
    order[start[l] + H[(size_t)blockIdx.x * Vt + l] + rank[i]] = i;
}

template <typename T>
__global__ __launch_bounds__(256) void emb_segsum_kernel(int h, const int* __restrict__ start,
                                                         const int* __restrict__ order, const T* __restrict__ dX,
                                                         T* __restrict__ dE, int accumulate) {
    const int v = blockIdx.x;
    const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
    if (c >= h) return;
    const int s0 = start[v], s1 = start[v + 1];
    if (s0 == s1 && accumulate) return;
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = s0; j < s1; ++j) {
        float g[8];
        load8(dX + (size_t)order[j] * h + c, g);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] += g[e];
    }
    T* dst = dE + (size_t)v * h + c;
    if (accumulate) {
        float o[8];
        load8(dst, o);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] += o[e];
    }
    store8(dst, a);
}

hipError_t embedding_fwd(int dt, int N, int h, int Vt, int r, const int32_t* ids, const void* E_r, void* out,
                         hipStream_t st) {
    const long n = (long)N * (h / 8);
    if (n == 0) return hipSuccess;
    dim3 grid((unsigned)((n + 255) / 256));
    if (dt == 1)
        hipLaunchKernelGGL(emb_fwd_kernel<bf16>, grid, dim3(256), 0, st, N, h, Vt, r, ids, (const bf16*)E_r, (bf16*)out);
    else
        hipLaunchKernelGGL(emb_fwd_kernel<float>, grid, dim3(256), 0, st, N, h, Vt, r, ids, (const float*)E_r,
                           (float*)out);
    return hipGetLastError();
}

static size_t al256(size_t b) { return (b + 255) / 256 * 256; }

// ws: H [nchunks][Vt], rank [N], start [Vt + 1], order [N] (ints)
size_t embedding_bwd_ws_bytes(int N, int Vt) {
    const size_t nch = (size_t)std::max(1, (N + EMB_CHUNK - 1) / EMB_CHUNK), n = (size_t)std::max(N, 1);
    return al256(nch * Vt * sizeof(int)) + 2 * al256(n * sizeof(int)) + al256((size_t)(Vt + 1) * sizeof(int));
}

hipError_t embedding_bwd(int dt, int N, int h, int Vt, int r, const int32_t* ids, const void* dX, void* dE_r,
                         int accumulate, void* ws, hipStream_t st) {
    if (Vt <= 0) return hipErrorInvalidValue;
    const int nch = std::max(1, (N + EMB_CHUNK - 1) / EMB_CHUNK);
    const size_t n = (size_t)std::max(N, 1);
    char* w = (char*)ws;
    int* H = (int*)w;
    w += al256((size_t)nch * Vt * sizeof(int));
    int* rank = (int*)w;
    w += al256(n * sizeof(int));
    int* order = (int*)w;
    w += al256(n * sizeof(int));
    int* start = (int*)w;
    hipLaunchKernelGGL(emb_rank_kernel, dim3(nch), dim3(EMB_CHUNK), 0, st, N, Vt, r, ids, H, rank);
    hipLaunchKernelGGL(emb_prefix_kernel, dim3((Vt + 255) / 256), dim3(256), 0, st, nch, Vt, H, start);
    hipLaunchKernelGGL(emb_scan_kernel, dim3(1), dim3(1024), 0, st, Vt, start);
    if (N > 0)
        hipLaunchKernelGGL(emb_place_kernel, dim3(nch), dim3(EMB_CHUNK), 0, st, N, Vt, r, ids, H, rank, start, order);
    dim3 grid((unsigned)Vt, (unsigned)((h + 2047) / 2048));
    if (dt == 1)
        hipLaunchKernelGGL(emb_segsum_kernel<bf16>, grid, dim3(256), 0, st, h, start, order, (const bf16*)dX, (bf16*)dE_r,
                           accumulate);
    else
        hipLaunchKernelGGL(emb_segsum_kernel<float>, grid, dim3(256), 0, st, h, start, order, (const float*)dX,
                           (float*)dE_r, accumulate);
    return hipGetLastError();
}

}  // namespace tp
