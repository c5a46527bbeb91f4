// Reference outputs of rocRAND's Philox4x32-10 (its header implementation, compiled for the host)
// for the oracle's RNG pin. Usage: rocrand_philox_ref SEED SUBSEQUENCE OFFSET N -> N lines of four
// 32-bit words (hex). rocRAND keys Philox with the seed and starts the counter at
// (OFFSET / 4, 0, SUBSEQUENCE low, SUBSEQUENCE high).
#include <rocrand/rocrand_kernel.h>

#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
    if (argc != 5) return 2;
    const unsigned long long seed = strtoull(argv[1], nullptr, 0), sub = strtoull(argv[2], nullptr, 0),
                             off = strtoull(argv[3], nullptr, 0);
    const int n = atoi(argv[4]);
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, sub, off, &st);
    for (int i = 0; i < n; ++i) {
        const uint4 v = rocrand4(&st);
        printf("%08x %08x %08x %08x\n", v.x, v.y, v.z, v.w);
    }
    return 0;
}
