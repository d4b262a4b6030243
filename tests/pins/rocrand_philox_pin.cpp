// Host-side reference for the Philox4x32-10 pin: evaluates rocRAND's
// header-only philox4x32_10_engine (an implementation independent of both the
// oracle and the HIP library) at explicit (counter, key) points.
// stdin: lines "c0 c1 c2 c3 k0 k1" (decimal); stdout: four words per line.
// The engine's seed is the 64-bit key; its subsequence index fills counter
// words 2..3 and its offset (4 outputs per counter step) fills words 0..1.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdint>

int main() {
    unsigned long long c0, c1, c2, c3, k0, k1;
    while (std::scanf("%llu %llu %llu %llu %llu %llu", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        const unsigned long long seed = k0 | (k1 << 32);
        const unsigned long long subseq = c2 | (c3 << 32);
        const unsigned long long offset = 4ull * (c0 | (c1 << 32));
        rocrand_device::philox4x32_10_engine eng(seed, subseq, offset);
        const uint4 r = eng.next4();
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
