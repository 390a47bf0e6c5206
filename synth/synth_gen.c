/*
 * synth_gen.c -- seeded synthetic bf16 inputs for the quantizers and the GEMM.
 *
 * Input generation only: nothing here quantizes, scales or multiplies matrices.  Both the
 * HIP library's tests/benchmark and the CPU oracle consume the arrays this produces.
 *
 * Random numbers: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
 * as easy as 1, 2, 3", SC'11), a counter-based generator: output = f(counter, key) with
 * no state, so any element can be generated independently on any host or thread.
 *   key     = (seed, stream)            stream: 0 = A/X values, 1 = B/W values,
 *                                               2 = outlier mask, 3 = row magnitudes
 *   counter = (i mod 2^32, i div 2^32, 0, 0)   i = flat element (or row) index
 * Normals: Box-Muller in fp64 from two 53-bit uniforms.  Every product (sigma, outlier
 * factor, row magnitude) is taken in fp64, then rounded once to bf16, nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static void philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

static void draw(uint64_t seed, uint32_t stream, uint64_t i, uint32_t out[4])
{
    uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(i >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, stream};
    philox4x32_10(ctr, key, out);
}

/* 53-bit uniform in [0,1) from two words */
static double u53(uint32_t a, uint32_t b)
{
    uint64_t v = ((uint64_t)(a >> 5) << 26) | (uint64_t)(b >> 6);
    return (double)v * 0x1.0p-53;
}

/* one standard normal per index (Box-Muller, cosine branch) */
static double normal_at(uint64_t seed, uint32_t stream, uint64_t i)
{
    uint32_t w[4];
    draw(seed, stream, i, w);
    double u1 = 1.0 - u53(w[0], w[1]); /* (0,1] */
    double u2 = u53(w[2], w[3]);       /* [0,1) */
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

double synth_uniform_at(uint64_t seed, uint32_t stream, uint64_t i)
{
    uint32_t w[4];
    draw(seed, stream, i, w);
    return u53(w[0], w[1]);
}

void synth_philox_block(uint64_t seed, uint32_t stream, uint64_t i, uint32_t *out4)
{
    draw(seed, stream, i, out4);
}

/* fp64 -> bf16 bits, one rounding to nearest, ties to even (bf16: 8 significant bits,
 * exponent range of binary32, subnormal quantum 2^-133). */
uint16_t synth_f64_to_bf16(double d)
{
    float f;
    uint32_t u;
    if (isnan(d))
        return 0x7FC0;
    double a = fabs(d);
    double r;
    if (a == 0.0) {
        r = 0.0;
    } else {
        int e;
        frexp(a, &e);                  /* a = m * 2^e, m in [0.5,1) */
        int qexp = e - 8;              /* quantum for 8 significant bits */
        if (qexp < -133)
            qexp = -133;               /* bf16 subnormal quantum */
        r = ldexp(rint(ldexp(a, -qexp)), qexp); /* rint: nearest, ties to even */
        if (r >= 0x1.0p128)
            r = INFINITY;
    }
    f = (float)r; /* exact: r has <= 8 significant bits within binary32 range */
    memcpy(&u, &f, sizeof u);
    u >>= 16;
    if (signbit(d))
        u |= 0x8000;
    return (uint16_t)u;
}

/*
 * Fill rows r0 <= r < r1 of a [rows, cols] row-major bf16 matrix:
 *   v = sigma * z(seed, stream, i)                    i = r*cols + c
 *   if outlier_p > 0 and U(seed, 2 + outlier_stream_offset, i) < outlier_p: v *= outlier_factor
 *   if row_log_mag: v *= 10^(row_log_lo + (row_log_hi - row_log_lo) * U(seed, 3, r))
 * Returns the number of outliers placed in these rows.
 */
int64_t synth_matrix_bf16(uint16_t *out, int64_t rows, int64_t cols, uint64_t seed,
                          uint32_t stream, double sigma, double outlier_p, double outlier_factor,
                          uint32_t outlier_stream, int row_log_mag, double row_log_lo,
                          double row_log_hi, int64_t r0, int64_t r1)
{
    int64_t outliers = 0;
    if (r0 < 0 || r1 > rows || r0 > r1)
        return -1;
    for (int64_t r = r0; r < r1; ++r) {
        double rowmag = 1.0;
        if (row_log_mag) {
            double u = synth_uniform_at(seed, 3u, (uint64_t)r);
            rowmag = pow(10.0, row_log_lo + (row_log_hi - row_log_lo) * u);
        }
        for (int64_t c = 0; c < cols; ++c) {
            uint64_t i = (uint64_t)(r * cols + c);
            double v = sigma * normal_at(seed, stream, i);
            if (outlier_p > 0.0 && synth_uniform_at(seed, outlier_stream, i) < outlier_p) {
                v *= outlier_factor;
                ++outliers;
            }
            if (row_log_mag)
                v *= rowmag;
            out[r * cols + c] = synth_f64_to_bf16(v);
        }
    }
    return outliers;
}
