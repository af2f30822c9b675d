// Division of 32-bit unsigned integers by a run-time invariant divisor with
// one multiply-high, a subtract, an add and two shifts (Granlund and
// Montgomery, "Division by invariant integers using multiplication", PLDI
// 1994, the round-up method for N-bit dividends).  The host computes the
// multiplier once per launch; the kernels split their flat tile index into
// (batch, token, block) without a hardware divide.
//
// Plain C++ so that the host test can compile it with g++.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define QKR_HD __host__ __device__
#else
#define QKR_HD
#endif

namespace qkr {

struct FastDiv {
    uint32_t d;    // divisor (>= 1)
    uint32_t m;    // multiplier
    uint32_t sh;   // the two shifts: s1 in bits 0..7, s2 in bits 8..15
};

// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1, s1 = min(l, 1),
// s2 = l - s1.  The shifts are packed on the host so that a kernel spends no
// instruction on choosing s1.
inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t l = 0;
    while (((uint64_t)1 << l) < d)
        ++l;
    const uint32_t s1 = l < 1u ? l : 1u;
    FastDiv f{d, 0u, s1 | ((l - s1) << 8)};
    f.m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
    return f;
}

QKR_HD inline uint32_t mulhi32(uint32_t a, uint32_t b) { return (uint32_t)(((uint64_t)a * b) >> 32); }

// n / f.d for every 32-bit n:  t = mulhi(m, n);  q = (t + ((n - t) >> s1)) >> s2.
// For d >= 2 that is the paper's (t + ((n - t) >> 1)) >> (l - 1); for d = 1
// (l = 0, m = 1) t is 0 and q = n.  No branch, so a kernel can fetch every
// divisor field in one batch.  Both shifts are at most 31; the masks are the
// ones the shift instructions apply anyway.
QKR_HD inline uint32_t fast_div(uint32_t n, const FastDiv& f)
{
    const uint32_t t = mulhi32(f.m, n);
    return (t + ((n - t) >> (f.sh & 31u))) >> ((f.sh >> 8) & 31u);
}

}  // namespace qkr
