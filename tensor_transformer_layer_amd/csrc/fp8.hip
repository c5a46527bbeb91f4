// Per-tensor fp8 (OCP E4M3) quantisation: amax, power-of-two scale, conversion, and an
// optional transposed copy of the codes (the K-contiguous layout a weight-gradient GEMM needs).
//
// Scheme (the library's own; the pages train in 16-bit floating point, "Megatron-LM, annotated",
// §4.2, and define no 8-bit format):
//   amax = max |x|; e = the largest integer with amax * 2^e <= 448 (0 for amax = 0 or not finite),
//   clamped to [-126, 126]; code = E4M3(x * 2^e), round to nearest even, saturating at +-448;
//   the caller gets descale = 2^-e, so x ~ dec(code) * descale.
// x * 2^e is exact in fp32, so the conversion is the only rounding.
//
// Two launches: amax_partial_kernel (grid-stride, one max per block; max is exact and
// order-free, so the result does not depend on the partition) and fp8_cast_kernel (every block
// folds the <= 512 partials, derives e, converts a 64 x 128 tile; block (0,0) writes amax and
// descale).
#include <algorithm>

#include "launch.h"
#include "common.h"

namespace tp {

constexpr int Q_PARTS = 512;          // amax partials (blocks of the first launch)
constexpr int Q_TR = 64, Q_TC = 128;  // cast tile: rows x columns

template <typename T>
__global__ __launch_bounds__(256) void amax_partial_kernel(int rows, int cols, const T* __restrict__ x, int ldx,
                                                           float* __restrict__ part) {
    const int cpr = cols >> 3;   // 8-element chunks per row; rows * cpr < 2^31 (checked on the host)
    const int total = rows * cpr;
    const int stride = gridDim.x * 256;
    float m = 0.0f;
    int q = blockIdx.x * 256 + threadIdx.x;
    for (; q < total - 3 * stride; q += 4 * stride) {
        float v[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int qq = q + u * stride;
            const int r = qq / cpr, c = (qq - r * cpr) * 8;
            load8(x + (size_t)r * ldx + c, v[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[u][e]));
    }
    for (; q < total; q += stride) {
        const int r = q / cpr, c = (q - r * cpr) * 8;
        float v[8];
        load8(x + (size_t)r * ldx + c, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// e of the header for a non-negative fp32 amax, from its bits: amax = f * 2^p with f in [0.5, 1);
// amax * 2^e <= 448 = 0.875 * 2^9 holds for e = 9 - p when f <= 0.875, else for e = 8 - p, and
// fails for e + 1 in both cases.
__device__ __forceinline__ int fp8_scale_exp(float amax) {
    const uint32_t u = __float_as_uint(amax);
    const int ef = (int)((u >> 23) & 0xff);
    if (amax == 0.0f || ef == 0xff) return 0;
    if (ef == 0) return 126;   // subnormal amax: e would exceed the clamp
    const int p = ef - 126;
    const int e = ((u & 0x7fffffu) <= 0x600000u) ? 9 - p : 8 - p;
    return max(-126, min(126, e));
}

__device__ __forceinline__ float sat448(float v) { return v > 448.0f ? 448.0f : (v < -448.0f ? -448.0f : v); }

// four floats -> four E4M3 codes, first value in the lowest byte
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
    return (uint32_t)w;
}

template <typename T>
__global__ __launch_bounds__(256) void fp8_cast_kernel(int rows, int cols, const T* __restrict__ x, int ldx,
                                                       const float* __restrict__ part, int nparts,
                                                       uint8_t* __restrict__ codes, int ldc,
                                                       uint8_t* __restrict__ codes_t, int ldt,
                                                       float* __restrict__ amax_out, float* __restrict__ descale_out) {
    __shared__ float red[4];
    __shared__ uint32_t tile[Q_TR][Q_TC / 4 + 1];   // codes of the tile, row-major, padded
    const int tid = threadIdx.x;
    float m = 0.0f;
    for (int i = tid; i < nparts; i += 256) m = fmaxf(m, part[i]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int e = fp8_scale_exp(m);
    const float s = __uint_as_float((uint32_t)(127 + e) << 23);
    if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
        if (amax_out) *amax_out = m;
        *descale_out = __uint_as_float((uint32_t)(127 - e) << 23);
    }
    const int r0 = blockIdx.y * Q_TR, c0 = blockIdx.x * Q_TC;
    // 64 rows x 16 chunks of 8 = 1024 chunks, 4 per thread
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int q = tid + j * 256, lr = q >> 4, lc = (q & 15) * 8;
        const int r = r0 + lr, c = c0 + lc;
        uint32_t lo = 0, hi = 0;
        if (r < rows && c < cols) {
            float v[8];
            load8(x + (size_t)r * ldx + c, v);
            lo = cvt4_e4m3(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
            hi = cvt4_e4m3(v[4] * s, v[5] * s, v[6] * s, v[7] * s);
            if (codes) *(u32x2*)(codes + (size_t)r * ldc + c) = u32x2{lo, hi};
        }
        if (codes_t) {
            tile[lr][lc >> 2] = lo;
            tile[lr][(lc >> 2) + 1] = hi;
        }
    }
    if (!codes_t) return;
    __syncthreads();
    // transposed: 128 columns x 4 groups of 16 rows; each thread one 16-byte run of one column
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int q = tid + j * 256, lc = q >> 2, lr0 = (q & 3) * 16;
        const int c = c0 + lc, r = r0 + lr0;
        if (c >= cols || r >= rows) continue;
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t b = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) b |= ((tile[lr0 + 4 * i + k][lc >> 2] >> (8 * (lc & 3))) & 0xffu) << (8 * k);
            w[i] = b;
        }
        uint8_t* dst = codes_t + (size_t)c * ldt + r;
        if (r + 16 <= rows) {
            *(u32x4*)dst = u32x4{w[0], w[1], w[2], w[3]};
        } else {
            for (int i = 0; i < rows - r; ++i) dst[i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
        }
    }
}

size_t fp8_quantize_ws_bytes() { return Q_PARTS * sizeof(float); }

hipError_t fp8_quantize(int dt, int rows, int cols, const void* x, int ldx, uint8_t* codes, int ldc,
                        uint8_t* codes_t, int ldt, float* amax, float* descale, float* ws, hipStream_t st) {
    const long chunks = (long)rows * (cols / 8);
    const int nparts = (int)std::max(1L, std::min((long)Q_PARTS, (chunks + 1023) / 1024));
    dim3 grid(std::max(1, (cols + Q_TC - 1) / Q_TC), std::max(1, (rows + Q_TR - 1) / Q_TR));
    if (dt == 1) {
        hipLaunchKernelGGL(amax_partial_kernel<bf16>, dim3(nparts), dim3(256), 0, st, rows, cols, (const bf16*)x, ldx, ws);
        hipLaunchKernelGGL(fp8_cast_kernel<bf16>, grid, dim3(256), 0, st, rows, cols, (const bf16*)x, ldx, ws, nparts,
                           codes, ldc, codes_t, ldt, amax, descale);
    } else {
        hipLaunchKernelGGL(amax_partial_kernel<float>, dim3(nparts), dim3(256), 0, st, rows, cols, (const float*)x, ldx, ws);
        hipLaunchKernelGGL(fp8_cast_kernel<float>, grid, dim3(256), 0, st, rows, cols, (const float*)x, ldx, ws, nparts,
                           codes, ldc, codes_t, ldt, amax, descale);
    }
    return hipGetLastError();
}

}  // namespace tp
