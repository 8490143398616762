// Host-side check of the kernels' division by launch-time multipliers
// (FastDiv in kernel_common.h): fdiv(n, make_fastdiv(d)) == n / d for every
// dividend in [0, 2^31) tried, over all divisors up to 4096, the powers of
// two and their neighbours, and random divisors. Built with hipcc (the
// header includes the HIP runtime) and run by tests/test_fastdiv.py.
#include <cstdio>
#include <cstdint>
#include <random>

#include "kernel_common.h"

int main() {
    std::mt19937_64 rng(12345);
    long checked = 0, bad = 0;
    auto check = [&](int n, int d, const attn::FastDiv& f) {
        ++checked;
        if (attn::fdiv(n, f) != n / d) {
            if (bad < 5) std::printf("mismatch: %d / %d -> %d\n", n, d, attn::fdiv(n, f));
            ++bad;
        }
    };
    auto edges = [&](int d, const attn::FastDiv& f) {
        const int hi = 0x7fffffff;
        for (int n : {0, 1, d - 1, d, d + 1, hi, hi - 1, hi - d, hi / d * d, hi / d * d - 1}) if (n >= 0) check(n, d, f);
        for (int k = 1; k < 64; ++k) {             // multiples of d and their neighbours
            const int64_t m = (int64_t)d * (int64_t)(rng() % (hi / d + 1));
            for (int64_t n : {m - 1, m, m + 1}) if (n >= 0 && n <= hi) check((int)n, d, f);
        }
    };
    for (int d = 1; d <= 4096; ++d) {
        const attn::FastDiv f = attn::make_fastdiv(d);
        for (int n = 0; n < 8192; ++n) check(n, d, f);
        edges(d, f);
    }
    for (int l = 0; l < 31; ++l)
        for (int64_t d : {(int64_t)1 << l, ((int64_t)1 << l) - 1, ((int64_t)1 << l) + 1})
            if (d >= 1 && d <= 0x7fffffff) edges((int)d, attn::make_fastdiv((int)d));
    for (int i = 0; i < 200000; ++i) {
        const int d = (int)(rng() % 0x7fffffff) + 1, n = (int)(rng() & 0x7fffffff);
        check(n, d, attn::make_fastdiv(d));
    }
    std::printf("checked %ld, mismatches %ld\n", checked, bad);
    return bad != 0;
}
