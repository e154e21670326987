// Host-only check of the library's invariant-divisor division (FastDiv):
// compares fdiv(n, make_fastdiv(d)) with n / d.  Exhaustive for small d and
// n, sampled with edge values up to 2^31 - 1 otherwise.  No HIP calls.
#include <cstdio>
#include <cstdint>
#include <random>

#include "internal.h"

int main()
{
    using namespace cnv;
    long long checked = 0;
    for (uint32_t d = 1; d <= 2048; ++d) {
        FastDiv f = make_fastdiv(d);
        for (uint32_t n = 0; n < 70000; ++n, ++checked)
            if (fdiv(n, f) != n / d) { std::printf("FAIL d=%u n=%u\n", d, n); return 1; }
    }
    std::mt19937_64 rng(7);
    const uint32_t top = 0x7FFFFFFFu;
    for (int it = 0; it < 20000; ++it) {
        uint32_t d = (uint32_t)(rng() % top) + 1;
        if (it % 3 == 0) d = (uint32_t)(rng() % 100000) + 1;
        FastDiv f = make_fastdiv(d);
        uint32_t edges[6] = {top, top - 1, d - 1, d, d + 1 <= top ? d + 1 : d, (uint32_t)(rng() % top)};
        for (uint32_t n : edges) {
            if (n > top) continue;
            ++checked;
            if (fdiv(n, f) != n / d) { std::printf("FAIL d=%u n=%u\n", d, n); return 1; }
        }
        for (int k = 0; k < 200; ++k) {
            uint32_t n = (uint32_t)(rng() % ((uint64_t)top + 1));
            ++checked;
            if (fdiv(n, f) != n / d) { std::printf("FAIL d=%u n=%u\n", d, n); return 1; }
        }
    }
    std::printf("ok %lld\n", checked);
    return 0;
}
