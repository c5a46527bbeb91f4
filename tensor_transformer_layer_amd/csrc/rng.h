// Counter-based random numbers for dropout: Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011), written from the paper's definition.
//
// Streams and element mapping (shared with the tests' reference, which replays them on the CPU):
//   key = (seed low 32 bits, seed high 32 bits); counter = (call low, call high, 0, stream);
//   one call -> eight 16-bit uniforms, u[j] = (word j/2 >> 16 (j%2)) & 0xffff;
//   keep iff u >= thr, thr = round(p * 65536); kept values are scaled by 65536 / (65536 - thr).
//   Residual sites over [rows, n]: element (row, c) is slot c % 8 of call row * n/8 + c/8, so the
//   8 consecutive columns a thread owns are exactly one call.
//   Attention, element (sequence b, global head hg, query q, key k), n32 = ceil(s / 32): slot
//   ((k % 16) / 8) * 4 + k % 4 of call ((((b heads + hg) s + q) n32 + k / 32) 2 + (k % 8) / 4) 2
//   + (k % 32) / 16: one lane's 16 keys of a 32-key tile are two whole calls.
#pragma once
#include <stdint.h>

#include "common.h"

namespace tp {

// Dropout parameters as the kernels take them (the C ABI's tp_dropout, with p turned into its
// threshold and scale on the host).
struct DropParams {
    uint32_t thr;       // 0 = no dropout
    float scale;        // 65536 / (65536 - thr)
    uint32_t seed_lo, seed_hi, stream;
    int head0, heads;   // attention: global index of the rank's first head, heads of all ranks
    uint32_t* mask;     // attention keep bits [b][heads_t][s][ceil(s/32)]: bit j of word (.., q, kt) keeps key 32 kt + j
};

// Ten rounds on the counter c with key (k0, k1).
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t hi0 = __umulhi(0xD2511F53u, c[0]), lo0 = 0xD2511F53u * c[0];
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c[2]), lo1 = 0xCD9E8D57u * c[2];
        const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
    }
}

// Keep bits of the eight elements of one call: bit j = (u[j] >= thr).
__device__ __forceinline__ uint32_t keep8(uint64_t call, const DropParams& d) {
    uint32_t c[4] = {(uint32_t)call, (uint32_t)(call >> 32), 0u, d.stream};
    philox4x32_10(c, d.seed_lo, d.seed_hi);
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t u = (c[j >> 1] >> (16 * (j & 1))) & 0xffffu;
        bits |= (u >= d.thr ? 1u : 0u) << j;
    }
    return bits;
}

// v[e] = keep ? v[e] * scale : 0 for the eight elements of one call.
__device__ __forceinline__ void apply_keep8(float (&v)[8], uint32_t bits, float scale) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = ((bits >> e) & 1u) ? v[e] * scale : 0.0f;
}

}  // namespace tp
