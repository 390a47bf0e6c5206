/* Test-side check of the division the NVFP4 coder uses instead of one IEEE divide per
 * element: with r = fl32(1/D) (correctly rounded), q = fl32(x*r) and the negated remainder
 * e = fma(q, D, -x), y = fma(-e, r, q) should be fl32(x/D) (Markstein's theorem) wherever
 * the remainder is exact -- not where x is so small that it underflows, but there the
 * quotient is far below the first E2M1 boundary.  For `nd` pseudo-random D in
 * [2^-100, 2^100] and every bf16 x this counts: the x with 1/8 <= |x/D| <= 16 (every E2M1
 * boundary lies inside) whose y is not the correctly rounded quotient; the x with
 * |x/D| <= 16 (the coder only sees |x| < 9*D, whatever the magnitude) whose y gives another
 * E2M1 code than the correctly rounded quotient; and, among those, the x whose y has the
 * wrong sign.  Built with -ffp-contract=off: one IEEE binary32 operation
 * per C operation. */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static uint64_t next(uint64_t* s)   /* splitmix64 */
{
    uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* E2M1 code of y, nearest-even, saturating at 6 (written independently of the GPU code):
 * the grid 0, .5, 1, 1.5, 2, 3, 4, 6 and the midpoints between neighbours */
static unsigned e2m1(float y)
{
    static const float grid[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    const float a = fabsf(y);
    unsigned best = 0;
    for (unsigned c = 1; c < 8; ++c) {
        const float mid = 0.5f * (grid[c - 1] + grid[c]);
        if (a > mid || (a == mid && (c & 1) == 0))
            best = c;
    }
    return best | ((u_of(y) >> 28) & 8u);
}

uint64_t markstein_sweep(uint64_t nd, uint64_t seed, uint64_t* code_errors,
                         uint64_t* sign_errors, uint64_t* checked)
{
    uint64_t bad = 0, cbad = 0, sbad = 0, n = 0, s = seed;
    for (uint64_t d = 0; d < nd; ++d) {
        const uint64_t z = next(&s);
        const int ex = (int)(z % 201) - 100;                   /* exponent -100 .. 100 */
        const uint32_t man = (uint32_t)(z >> 32) & 0x7FFFFFu;
        const float D = f_of(((uint32_t)(ex + 127) << 23) | man);
        const float r = 1.0f / D;
        for (uint32_t b = 0; b < 65536; ++b) {
            if (((b >> 7) & 0xFF) == 0xFF)
                continue;                                      /* inf / NaN */
            const float x = f_of(b << 16);
            const float q = x * r;
            const float e = fmaf(q, D, -x);
            const float y = fmaf(-e, r, q);
            const float ref = x / D;
            const float a = fabsf(ref);
            if (a > 16.0f)
                continue;                              /* the coder sees |x| < 9*D only */
            if ((u_of(y) >> 31) != (b >> 15))
                ++sbad;
            if (e2m1(y) != e2m1(ref))
                ++cbad;
            if (a >= 0.125f && a <= 16.0f) {
                ++n;
                if (u_of(y) != u_of(ref))
                    ++bad;
            }
        }
    }
    *code_errors = cbad;
    *sign_errors = sbad;
    *checked = n;
    return bad;
}
