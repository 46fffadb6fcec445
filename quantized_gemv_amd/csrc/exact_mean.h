// exact_mean.h -- correctly rounded mean of |x| over fp32 values.
//
// Used for the ternary absmean scale gamma and the per-row sign-backbone
// scale alpha: both are the mean absolute weight, and this computes the fp32
// nearest to that exact real number (ties to even), independent of the order
// in which the contributions were accumulated.  Plain C++ so that the same
// code also builds for the host.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define QG_HD __host__ __device__
#else
#define QG_HD
#endif

namespace qg {

// ------------------------------------------------------------------ exact mean of |x|
// |x| of a finite fp32 equals mant * 2^(shift - 149) with mant < 2^24 and
// shift = max(biased exponent, 1) - 1 in [0, 253].  Summing mant per shift
// (a "binade histogram") in 64-bit integers is exact and independent of the
// order of the additions.
QG_HD inline void abs_binade(float x, uint32_t& shift, uint32_t& mant) {
    uint32_t b;
    __builtin_memcpy(&b, &x, 4);
    b &= 0x7FFFFFFFu;
    uint32_t e = b >> 23;
    mant = (b & 0x7FFFFFu) | (e ? 0x800000u : 0u);
    shift = (e ? e : 1u) - 1u;
}

// Given hist[shift] = sum of mant over the binade `shift` (256 entries) and
// the element count (< 2^40), return the fp32 nearest to
// (sum_shift hist[shift] * 2^shift) * 2^-149 / count, ties to even.
// Multi-precision integer arithmetic with 16-bit limbs; the quotient carries
// 64 extra fractional bits, and the remainder feeds the sticky bit.
QG_HD inline float round_mean_from_binades(const uint64_t* hist, uint64_t count) {
    constexpr int NL = 28;  // 448 bits: covers 2^(253 + 64 + 64) with margin
    uint32_t L[NL];
    for (int i = 0; i < NL; ++i) L[i] = 0;
    for (int sh = 0; sh < 256; ++sh) {
        const uint64_t v = hist[sh];
        if (!v) continue;
        const int pos = sh + 64;
        const int li = pos >> 4, off = pos & 15;
        uint64_t carry = 0;
        for (int i = 0; li + i < NL; ++i) {
            const int bit = 16 * i - off;  // limb li+i takes bits [bit, bit+16) of v
            uint32_t piece;
            if (bit >= 64) piece = 0;
            else if (bit >= 0) piece = (uint32_t)((v >> bit) & 0xFFFFu);
            else piece = (uint32_t)((v << (-bit)) & 0xFFFFu);
            if (bit >= 64 && carry == 0) break;
            const uint64_t t = (uint64_t)L[li + i] + piece + carry;
            L[li + i] = (uint32_t)(t & 0xFFFFu);
            carry = t >> 16;
        }
    }
    uint32_t Q[NL];
    uint64_t rem = 0;
    for (int i = NL - 1; i >= 0; --i) {
        const uint64_t cur = (rem << 16) | L[i];
        Q[i] = (uint32_t)(cur / count);
        rem = cur % count;
    }
    int top = -1;
    for (int i = NL - 1; i >= 0; --i) {
        if (Q[i]) {
            top = i * 16 + (31 - __builtin_clz(Q[i]));
            break;
        }
    }
    if (top < 0) return 0.0f;  // below 2^-213: nearest fp32 is 0
    int shift = top + 1 - 24;
    if (shift < 64) shift = 64;  // subnormal quantum 2^-149 == 2^64 quotient units
    uint32_t mant = 0;
    for (int b = shift + 23; b >= shift; --b) {
        const uint32_t bitv = (b < NL * 16) ? ((Q[b >> 4] >> (b & 15)) & 1u) : 0u;
        mant = (mant << 1) | bitv;
    }
    const uint32_t guard = (Q[(shift - 1) >> 4] >> ((shift - 1) & 15)) & 1u;
    bool sticky = rem != 0;
    for (int b = shift - 2; b >= 0 && !sticky; --b) sticky = ((Q[b >> 4] >> (b & 15)) & 1u) != 0;
    if (guard && (sticky || (mant & 1u))) mant += 1u;
    // value = mant * 2^(shift - 64 - 149); exact in fp32 by construction
    return __builtin_ldexpf((float)mant, shift - 64 - 149);
}

}  // namespace qg
