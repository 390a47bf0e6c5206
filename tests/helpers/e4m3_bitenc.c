/*
 * Test helper: an independent E4M3FN encoder written with integer arithmetic on the
 * binary32 bit pattern (round to nearest, ties to even, saturate at 448), and an
 * exhaustive sweep that compares it with an encoder passed in by pointer (the oracle's).
 * Test code only.
 */
#include <stdint.h>
#include <string.h>

static uint8_t bitenc(uint32_t u)
{
    uint32_t sign = (u >> 31) << 7;
    uint32_t a = u & 0x7FFFFFFFu;
    if (a >= 0x43E00000u)                    /* |y| >= 448.0f (and +-inf) */
        return (uint8_t)(sign | 0x7E);
    int32_t E = (int32_t)(a >> 23);
    uint32_t M = a & 0x7FFFFFu;
    if (E == 0)                              /* fp32 subnormal: far below 2^-10 */
        return (uint8_t)sign;
    int32_t e = E - 127;
    uint32_t sig = M | 0x800000u;            /* 24-bit significand */
    uint32_t q, rem, half, sh;
    if (e >= -6) {
        /* normal E4M3: keep 3 mantissa bits, round away the low 20 */
        sh = 20;
        q = (((uint32_t)(e + 7)) << 3) | (M >> 20);
        rem = M & 0xFFFFFu;
    } else {
        /* subnormal E4M3: count of 2^-9 quanta = sig * 2^(e-14) */
        sh = (uint32_t)(14 - e);            /* >= 21 */
        if (sh >= 32)
            return (uint8_t)sign;            /* < 2^-10 / 2: rounds to zero */
        q = sig >> sh;
        rem = sig & ((1u << sh) - 1u);
    }
    half = 1u << (sh - 1);
    if (rem > half || (rem == half && (q & 1u)))
        q += 1;                              /* carry may move into the exponent: correct */
    return (uint8_t)(sign | q);
}

uint8_t helper_bitenc(float y)
{
    uint32_t u;
    memcpy(&u, &y, sizeof u);
    return bitenc(u);
}

typedef uint8_t (*enc_fn)(float);

/* Compare over bit patterns [lo, hi) (hi up to 2^32), skipping NaNs.  Returns the number
 * of mismatches and stores the first one in *first. */
uint64_t helper_sweep(enc_fn other, uint64_t lo, uint64_t hi, uint64_t *first)
{
    uint64_t bad = 0;
    *first = (uint64_t)-1;
    for (uint64_t p = lo; p < hi; ++p) {
        uint32_t u = (uint32_t)p;
        if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu))
            continue;
        float y;
        memcpy(&y, &u, sizeof y);
        if (bitenc(u) != other(y)) {
            if (!bad)
                *first = p;
            ++bad;
        }
    }
    return bad;
}
