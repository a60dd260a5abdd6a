// Host check of lnr_fastdiv.h: divu32(n, make_divu32(d)) == n / d on edge and random values
// for many divisors, and exhaustively over every 32-bit n for two divisors. Prints the number
// of mismatches (0 expected) and exits non-zero on any.
#include <stdio.h>
#include <stdint.h>

#include <random>
#include <vector>

#include "lnr_fastdiv.h"

int main() {
    using namespace lnr;
    std::vector<uint32_t> divisors;
    for (uint32_t d = 1; d <= 4096; ++d) divisors.push_back(d);
    for (int k = 12; k < 32; ++k) {
        const uint32_t p = 1u << k;
        for (uint32_t d : {p - 1, p, p + 1, p + 3 * (p >> 2)}) divisors.push_back(d);
    }
    for (uint32_t d : {641u, 6700417u, 0x7FFFFFFFu, 0x80000001u, 0xFFFFFFFEu, 0xFFFFFFFFu,
                       16384u * 8u, 8u * 256u, 16u * 512u, 8u * 2048u})
        divisors.push_back(d);
    std::mt19937_64 rng(12345);
    uint64_t bad = 0, checked = 0;
    for (uint32_t d : divisors) {
        const DivU32 f = make_divu32(d);
        std::vector<uint32_t> ns = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 2 * d, 0x7FFFFFFFu,
                                    0x80000000u, 0xFFFFFFFEu, 0xFFFFFFFFu};
        const uint32_t qmax = 0xFFFFFFFFu / d;
        for (uint32_t q : {qmax, qmax - 1, qmax / 2}) {
            const uint64_t b = static_cast<uint64_t>(q) * d;
            for (int64_t o = -2; o <= 2; ++o) {
                const int64_t n = static_cast<int64_t>(b) + o;
                if (n >= 0 && n <= 0xFFFFFFFFll) ns.push_back(static_cast<uint32_t>(n));
            }
        }
        for (int i = 0; i < 2000; ++i) ns.push_back(static_cast<uint32_t>(rng()));
        for (uint32_t n : ns) {
            ++checked;
            if (divu32(n, f) != n / d) {
                if (bad < 10) printf("mismatch: n=%u d=%u got %u want %u\n", n, d, divu32(n, f), n / d);
                ++bad;
            }
        }
    }
    for (uint32_t d : {1000003u}) {
        const DivU32 f = make_divu32(d);
        uint32_t n = 0;
        do {
            ++checked;
            if (divu32(n, f) != n / d) ++bad;
        } while (++n != 0);
    }
    printf("checked %llu, mismatches %llu\n", (unsigned long long)checked, (unsigned long long)bad);
    return bad == 0 ? 0 : 1;
}
