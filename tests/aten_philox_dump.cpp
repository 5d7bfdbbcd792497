// Test-only cross-check of the oracle's Philox4x32-10: evaluates ATen's
// header-only Philox engine (an independent implementation of the same
// published generator) at counters read from stdin.
// Input lines: key_lo key_hi c0 c1 c2 c3  -> output line: x0 x1 x2 x3
// ATen's engine takes seed = key, subsequence = (c3:c2), offset = (c1:c0).
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdint>

int main() {
    unsigned long long k0, k1, c0, c1, c2, c3;
    while (std::scanf("%llu %llu %llu %llu %llu %llu", &k0, &k1, &c0, &c1, &c2, &c3) == 6) {
        uint64_t seed = (k1 << 32) | k0;
        uint64_t subseq = (c3 << 32) | c2;
        uint64_t offset = (c1 << 32) | c0;
        at::philox_engine eng(seed, subseq, offset);
        uint32_t x0 = eng(), x1 = eng(), x2 = eng(), x3 = eng();
        std::printf("%u %u %u %u\n", x0, x1, x2, x3);
    }
    return 0;
}
