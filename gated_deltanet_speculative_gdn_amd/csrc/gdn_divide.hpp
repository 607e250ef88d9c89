// gdn_divide.hpp -- unsigned 32-bit division by a divisor that is fixed for a
// whole launch (the head count, the row count), without a division
// instruction sequence in every workgroup's prologue.
//
// Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication" (PLDI 1994), the round-up method for N = 32 bits: with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1 (which fits in 32
// bits), q = floor(x / d) = (t + ((x - t) >> s1)) >> s2, t = (m * x) >> 32,
// s1 = min(l, 1), s2 = max(l - 1, 0), for every 32-bit x and every d >= 1.
// Plain C++ so the host computes the constants and a host test checks them.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define GDN_HOST_DEVICE __host__ __device__
#else
#define GDN_HOST_DEVICE
#endif

namespace gdn {

struct Divider {
    uint32_t m, s1, s2;
};

// d == 0 is taken as 1 (a launch with no heads or rows divides nothing).
inline Divider make_divider(uint32_t d)
{
    if (d == 0) d = 1;
    uint32_t l = 0;
    while (l < 32 && (uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((((uint64_t(1) << l) - d) << 32) / d) + 1;
    return Divider{(uint32_t)m, l > 0 ? 1u : 0u, l > 0 ? l - 1 : 0u};
}

GDN_HOST_DEVICE inline uint32_t udiv(uint32_t x, Divider v)
{
    const uint32_t t = (uint32_t)(((uint64_t)v.m * x) >> 32);
    return (t + ((x - t) >> v.s1)) >> v.s2;
}

}  // namespace gdn
