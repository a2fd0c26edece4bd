// Host check of the launch-constant division used by the kernels
// (make_fastdiv / fdiv in ctconv_internal.h): exhaustive over small divisors
// and numerators, plus random divisors and the largest numerators below 2^31.
#include <cstdio>
#include <random>

#include "ctconv_internal.h"

int main() {
    using ctconv::FastDiv;
    using ctconv::fdiv;
    using ctconv::make_fastdiv;
    long bad = 0, total = 0;
    auto check = [&](uint32_t n, uint32_t d, const FastDiv& f) {
        ++total;
        if (fdiv(n, f) != n / d) {
            if (bad < 5) printf("mismatch n=%u d=%u got %u\n", n, d, fdiv(n, f));
            ++bad;
        }
    };
    std::mt19937_64 g(12345);
    for (uint32_t d = 1; d <= 2048; ++d) {
        const FastDiv f = make_fastdiv(d);
        for (uint32_t n = 0; n < 8192; ++n) check(n, d, f);
        for (int i = 0; i < 256; ++i) check((uint32_t)(g() & 0x7fffffffu), d, f);
        check(0x7fffffffu, d, f);
        check(0x7fffffffu / d * d, d, f);
        if (0x7fffffffu / d * d > 0) check(0x7fffffffu / d * d - 1, d, f);
    }
    for (int i = 0; i < 20000; ++i) {
        uint32_t d = (uint32_t)(g() % 0x7fffffffu) + 1u;
        if (i % 3 == 0) d = 1u << (g() % 31);
        const FastDiv f = make_fastdiv(d);
        for (int k = 0; k < 64; ++k) check((uint32_t)(g() & 0x7fffffffu), d, f);
        check(0x7fffffffu, d, f);
        const uint32_t m = 0x7fffffffu / d * d;
        check(m, d, f);
        if (m > 0) check(m - 1, d, f);
    }
    printf("%ld of %ld wrong\n", bad, total);
    return bad != 0;
}
