// lnr_fastdiv.h -- unsigned 32-bit division by a divisor fixed for a whole launch, as one
// multiply-high, two shifts and two adds (5 VALU operations) instead of the ~25 of a general
// division. Method: T. Granlund and P. L. Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994, section 4 (Figure 4.1, unsigned division with N = 32):
//
//   l  = ceil(log2 d),  m' = floor(2^32 * (2^l - d) / d) + 1,
//   sh1 = min(l, 1),  sh2 = max(l - 1, 0),
//   t1 = mulhi(m', n),  q = (t1 + ((n - t1) >> sh1)) >> sh2      for every 0 <= n < 2^32.
//
// The host computes (m', sh1, sh2) once per launch; kernels take the struct by value.
// Plain C++ on the host side so that the magic numbers can be checked without a GPU.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define LNR_HD __host__ __device__
#else
#define LNR_HD
#endif

namespace lnr {

struct DivU32 {
    uint32_t d;    // the divisor, >= 1
    uint32_t m;    // m' above
    uint32_t sh1;  // 0 or 1
    uint32_t sh2;  // 0 .. 31
};

inline DivU32 make_divu32(uint32_t d) {
    uint32_t l = 0;
    while (l < 32 && (uint64_t{1} << l) < d) ++l;  // l = ceil(log2 d); d >= 1
    const uint64_t two_l = uint64_t{1} << l;
    const uint64_t m = ((two_l - d) << 32) / d + 1;  // (2^l - d) < 2^31, so no overflow
    return DivU32{d, static_cast<uint32_t>(m), l < 1 ? l : 1u, l > 0 ? l - 1 : 0u};
}

LNR_HD inline uint32_t divu32(uint32_t n, const DivU32 &f) {
    const uint32_t t1 = static_cast<uint32_t>((static_cast<uint64_t>(f.m) * n) >> 32);
    return (t1 + ((n - t1) >> f.sh1)) >> f.sh2;
}

}  // namespace lnr
