/*
 * fgq_oracle.c -- plain, slow, scalar CPU oracle for fine-grained FP8 quantization
 * and the block-scaled FP8 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call this code: only the
 * tests, the smoke check and the benchmark's CPU-baseline leg use it.  It shares no code,
 * header, table or constant with the HIP library.
 *
 * Method source: the page "Fine-Grained FP8/FP4 Quantization":
 *   - section "Scaling Granularities": one FP32 scale per 1x128 row tile of an activation
 *     and one per 128x128 block of a weight;
 *   - section "DeepGEMM: Tile-wise and Block-wise Scaling": scale tensor shapes
 *     scale_A [M, K/128] and scale_B [K/128, N/128] (row-major), and the GEMM that, for
 *     every 128-wide K chunk, multiplies the FP8 partial by scale_A[m,kb]*scale_B[kb,nb]
 *     and accumulates;
 *   - table "UE8M0 vs E4M3 Scale Formats": the E4M3 range ends at 448.
 * Readings where the page is silent (each listed in the design notes):
 *   - the stored scale is the dequantization scale s = amax / 448 (fp32, IEEE divide);
 *   - codes are E4M3 of the correctly rounded fp32 quotient x / s, rounded to nearest,
 *     ties to even, saturating at +-448 (OCP OFP8 "E4M3FN" variant: bias 7, no infinities,
 *     S.1111.111 is NaN);
 *   - an all-zero tile gets s = 0 and signed-zero codes;
 *   - the GEMM reference is dequantize-then-matmul in fp64 and overwrites C.
 *
 * Build: gcc -O2 -std=gnu99 -fPIC -shared -ffp-contract=off -fno-fast-math
 * (no contraction, no fast math: every float operation below is one IEEE binary32 or
 * binary64 operation with round-to-nearest-even, as written).
 */
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------------------ */
/* E4M3 (OCP OFP8 E4M3FN): decode is the closed form of the format definition.          */
/* ------------------------------------------------------------------------------------ */

/* Value of one E4M3FN code as a double; NaN for S.1111.111. */
double oracle_e4m3_decode(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);            /* subnormal: (m/8) * 2^(1-7) */
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);   /* normal: (1+m/8) * 2^(e-7) */
    return sign ? -mag : mag;
}

/* The 127 non-negative finite magnitudes, indexed by code 0x00..0x7E (increasing). */
static double e4m3_mag[127];

/* filled once when the library is loaded, before any thread can call the encoder */
__attribute__((constructor)) static void e4m3_init(void)
{
    for (int c = 0; c < 127; ++c)
        e4m3_mag[c] = oracle_e4m3_decode((uint8_t)c);
}

/*
 * Encode one fp32 value: round to the nearest E4M3FN value, ties to the code whose
 * mantissa LSB (= code LSB) is 0, saturating at 448.  Written as a nearest-value search
 * over the sorted table of representable magnitudes.  NaN input is out of contract.
 */
uint8_t oracle_e4m3_encode(float y)
{
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs((double)y);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    /* largest code lo with mag[lo] <= a (binary search over the increasing table) */
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (e4m3_mag[mid] <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    if (e4m3_mag[lo] == a)
        return (uint8_t)(sign | lo);
    /* a lies strictly between mag[lo] and mag[lo+1]; compare 2a with their sum (exact) */
    double twice = 2.0 * a;
    double sum = e4m3_mag[lo] + e4m3_mag[lo + 1];
    int pick;
    if (twice < sum)
        pick = lo;
    else if (twice > sum)
        pick = lo + 1;
    else
        pick = (lo % 2 == 0) ? lo : lo + 1; /* tie: even mantissa */
    return (uint8_t)(sign | pick);
}

/* bf16 bits -> fp32 (exact: the 16 bits are the high half of the binary32 pattern). */
static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Quantize one group of n values (given by index list) sharing one scale. */
static float quantize_group(const uint16_t *x, const int64_t *idx, int64_t n, uint8_t *q)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float v = fabsf(bf16_to_f32(x[idx[i]]));
        if (v > amax)
            amax = v;
    }
    float s = amax / 448.0f;
    for (int64_t i = 0; i < n; ++i) {
        float v = bf16_to_f32(x[idx[i]]);
        if (s == 0.0f)
            q[idx[i]] = signbit(v) ? 0x80 : 0x00;
        else
            q[idx[i]] = oracle_e4m3_encode(v / s);
    }
    return s;
}

/*
 * Activation quantization, 1x128 tiles along K (rows m0 <= m < m1 only, so callers may
 * split rows across threads).  X: bf16 bits [M,K] row-major.  Xq: codes [M,K].
 * sX: fp32 [M, K/128], sX[m*(K/128)+kb] is the scale of X[m, 128kb .. 128kb+127].
 * Requires K % 128 == 0.  Returns 0, or -1 on a bad shape.
 */
int oracle_quantize_act_1x128(const uint16_t *X, uint8_t *Xq, float *sX, int64_t M, int64_t K,
                              int64_t m0, int64_t m1)
{
    if (M < 0 || K < 0 || K % 128 != 0 || m0 < 0 || m1 > M || m0 > m1)
        return -1;
    int64_t KB = K / 128;
    int64_t idx[128];
    for (int64_t m = m0; m < m1; ++m) {
        for (int64_t kb = 0; kb < KB; ++kb) {
            for (int64_t j = 0; j < 128; ++j)
                idx[j] = m * K + kb * 128 + j;
            sX[m * KB + kb] = quantize_group(X, idx, 128, Xq);
        }
    }
    return 0;
}

/*
 * Weight quantization, 128x128 blocks (block rows kb0 <= kb < kb1 only).
 * W: bf16 bits [K,N] row-major.  Wq: codes [K,N].  sW: fp32 [K/128, N/128],
 * sW[kb*(N/128)+nb] is the scale of W[128kb .. 128kb+127][128nb .. 128nb+127].
 * Requires K % 128 == 0 and N % 128 == 0.  Returns 0, or -1 on a bad shape.
 */
int oracle_quantize_weight_128x128(const uint16_t *W, uint8_t *Wq, float *sW, int64_t K,
                                   int64_t N, int64_t kb0, int64_t kb1)
{
    if (K < 0 || N < 0 || K % 128 != 0 || N % 128 != 0 || kb0 < 0 || kb1 > K / 128 || kb0 > kb1)
        return -1;
    int64_t NB = N / 128;
    static __thread int64_t idx[128 * 128];
    for (int64_t kb = kb0; kb < kb1; ++kb) {
        for (int64_t nb = 0; nb < NB; ++nb) {
            int64_t t = 0;
            for (int64_t r = 0; r < 128; ++r)
                for (int64_t c = 0; c < 128; ++c)
                    idx[t++] = (kb * 128 + r) * N + nb * 128 + c;
            sW[kb * NB + nb] = quantize_group(W, idx, 128 * 128, Wq);
        }
    }
    return 0;
}

/*
 * Block-scaled GEMM reference, rows m0 <= m < m1.
 * a[m,k] = dec(Aq[m,k]) * sA[m, k/128],  b[k,n] = dec(Bq[k,n]) * sB[k/128, n/128]  (fp64)
 * C[m,n] = sum_k a[m,k] b[k,n]   and   S[m,n] = sum_k |a[m,k] b[k,n]|   (fp64, k ascending).
 * Aq [M,K], Bq [K,N] row-major codes; C, S [M,N] row-major (S may be NULL).
 */
int oracle_gemm_f64(const uint8_t *Aq, const float *sA, const uint8_t *Bq, const float *sB,
                    int64_t M, int64_t N, int64_t K, double *C, double *S, int64_t m0, int64_t m1)
{
    if (M < 0 || N < 0 || K < 0 || K % 128 != 0 || N % 128 != 0 || m0 < 0 || m1 > M || m0 > m1)
        return -1;
    int64_t KB = K / 128, NB = N / 128;
    double dec[256];
    for (int c = 0; c < 256; ++c)
        dec[c] = oracle_e4m3_decode((uint8_t)c);
    for (int64_t m = m0; m < m1; ++m) {
        double *crow = C + m * N;
        double *srow = S ? S + m * N : 0;
        for (int64_t n = 0; n < N; ++n) {
            crow[n] = 0.0;
            if (srow)
                srow[n] = 0.0;
        }
        for (int64_t k = 0; k < K; ++k) {
            double a = dec[Aq[m * K + k]] * (double)sA[m * KB + k / 128];
            const uint8_t *brow = Bq + k * N;
            const float *sbrow = sB + (k / 128) * NB;
            for (int64_t n = 0; n < N; ++n) {
                double p = a * (dec[brow[n]] * (double)sbrow[n / 128]);
                crow[n] += p;
                if (srow)
                    srow[n] += fabs(p);
            }
        }
    }
    return 0;
}

/*
 * The same reference for an explicit list of output elements (rows[i], cols[i]), each
 * computed on its own as one dot product over k (ascending) -- for spot checks of
 * outputs too large to form whole.
 */
int oracle_gemm_f64_at(const uint8_t *Aq, const float *sA, const uint8_t *Bq, const float *sB,
                       int64_t M, int64_t N, int64_t K, const int64_t *rows, const int64_t *cols,
                       int64_t count, double *C, double *S)
{
    if (M < 0 || N < 0 || K < 0 || K % 128 != 0 || N % 128 != 0)
        return -1;
    int64_t KB = K / 128, NB = N / 128;
    double dec[256];
    for (int c = 0; c < 256; ++c)
        dec[c] = oracle_e4m3_decode((uint8_t)c);
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = rows[i], n = cols[i];
        if (m < 0 || m >= M || n < 0 || n >= N)
            return -1;
        double c = 0.0, s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = dec[Aq[m * K + k]] * (double)sA[m * KB + k / 128];
            double p = a * (dec[Bq[k * N + n]] * (double)sB[(k / 128) * NB + n / 128]);
            c += p;
            s += fabs(p);
        }
        C[i] = c;
        if (S)
            S[i] = s;
    }
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* UE8M0 power-of-two scales (page "Fine-Grained FP8/FP4 Quantization", section           */
/* "Blackwell: Native Block Scaling": an unsigned 8-bit exponent e encodes 2^(e-127); and */
/* table "UE8M0 vs E4M3 Scale Formats").  The page gives the format, not the rule that    */
/* picks e from a group; the reading used here: the smallest power of two that lets the  */
/* group's amax reach at most 448 (so no code saturates), i.e. the smallest e in 0..254   */
/* with 448 * 2^(e-127) >= amax, e = 0 when even 2^-127 is more than enough (tiny or      */
/* all-zero groups).  Same 1x128 / 128x128 groups and code rule as the fp32-scale path:   */
/* code = ENC(fl32(x / s)) with s = 2^(e-127).  e = 255 is not produced (NaN in the OCP   */
/* microscaling definition of E8M0).                                                      */
/* ------------------------------------------------------------------------------------ */

/* Value of one UE8M0 scale byte (NaN for 255). */
double oracle_ue8m0_decode(uint8_t e)
{
    if (e == 255)
        return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* The exponent byte of a group with the given amax: walk e upward; 448 * 2^(e-127) is
 * exact in binary64, so every comparison is exact. */
static uint8_t ue8m0_exponent(double amax)
{
    int e = 0;
    while (e < 254 && 448.0 * ldexp(1.0, e - 127) < amax)
        ++e;
    return (uint8_t)e;
}

/* Quantize one group (index list) with a UE8M0 scale; returns the exponent byte. */
static uint8_t quantize_group_ue8m0(const uint16_t *x, const int64_t *idx, int64_t n,
                                    uint8_t *q)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float v = fabsf(bf16_to_f32(x[idx[i]]));
        if (v > amax)
            amax = v;
    }
    uint8_t e = ue8m0_exponent((double)amax);
    float s = (float)oracle_ue8m0_decode(e);   /* exact: 2^-127 .. 2^127 are binary32 values */
    for (int64_t i = 0; i < n; ++i)
        q[idx[i]] = oracle_e4m3_encode(bf16_to_f32(x[idx[i]]) / s);
    return e;
}

/* 1x128 activation quantization with UE8M0 scales: sX is uint8 [M, K/128]. */
int oracle_quantize_act_1x128_ue8m0(const uint16_t *X, uint8_t *Xq, uint8_t *sX, int64_t M,
                                    int64_t K, int64_t m0, int64_t m1)
{
    if (M < 0 || K < 0 || K % 128 != 0 || m0 < 0 || m1 > M || m0 > m1)
        return -1;
    int64_t KB = K / 128;
    int64_t idx[128];
    for (int64_t m = m0; m < m1; ++m)
        for (int64_t kb = 0; kb < KB; ++kb) {
            for (int64_t j = 0; j < 128; ++j)
                idx[j] = m * K + kb * 128 + j;
            sX[m * KB + kb] = quantize_group_ue8m0(X, idx, 128, Xq);
        }
    return 0;
}

/* 128x128 weight quantization with UE8M0 scales: sW is uint8 [K/128, N/128]. */
int oracle_quantize_weight_128x128_ue8m0(const uint16_t *W, uint8_t *Wq, uint8_t *sW,
                                         int64_t K, int64_t N, int64_t kb0, int64_t kb1)
{
    if (K < 0 || N < 0 || K % 128 != 0 || N % 128 != 0 || kb0 < 0 || kb1 > K / 128 || kb0 > kb1)
        return -1;
    int64_t NB = N / 128;
    static __thread int64_t idx[128 * 128];
    for (int64_t kb = kb0; kb < kb1; ++kb)
        for (int64_t nb = 0; nb < NB; ++nb) {
            int64_t t = 0;
            for (int64_t r = 0; r < 128; ++r)
                for (int64_t c = 0; c < 128; ++c)
                    idx[t++] = (kb * 128 + r) * N + nb * 128 + c;
            sW[kb * NB + nb] = quantize_group_ue8m0(W, idx, 128 * 128, Wq);
        }
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* NVFP4 two-level scaling (page "Fine-Grained FP8/FP4 Quantization", section "NVFP4     */
/* Two-Level Scaling"): E2M1 codes (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), one E4M3     */
/* block scale per 16 consecutive elements along K ([M, K/16] for A), one FP32 global    */
/* scale per tensor, dequantized as global * block * e2m1.  The page gives the format and */
/* the dequantization only; the readings used here to pick the scales:                   */
/*   g  = fl32(amax_tensor / 2688)          (2688 = 448 * 6: the largest block scale is  */
/*                                           448 and the largest code 6)                 */
/*   sb = ENC_E4M3(fl32(amax_block / fl32(6 * g)))   (saturating, nearest-even)          */
/*   D  = fl32(DEC_E4M3(sb) * g)            the block's dequantization multiplier        */
/*   code = ENC_E2M1(fl32(x / D))           nearest, ties to the even code, saturating   */
/*                                           at 6; signed zero when D == 0               */
/* Both operands of the GEMM are row-major [rows, K] with the blocks along K (the weight */
/* is stored as its [N, K] transpose), two codes per byte, element 2i in the low nibble. */
/* ------------------------------------------------------------------------------------ */

static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Value of one E2M1 code (low 4 bits: sign bit 3, magnitude code 0..7). */
double oracle_e2m1_decode(uint8_t code)
{
    double v = E2M1_MAG[code & 7];
    return (code & 8) ? -v : v;
}

/* Nearest E2M1 code of y; a tie goes to the even magnitude code; |y| >= 6 gives 6. */
uint8_t oracle_e2m1_encode(float y)
{
    uint8_t sign = signbit(y) ? 8 : 0;
    double a = fabs((double)y);
    uint8_t best = 7;
    if (a < 6.0) {
        for (uint8_t c = 0; c < 7; ++c) {
            double lo = E2M1_MAG[c], hi = E2M1_MAG[c + 1];
            if (a <= hi) {
                double mid = 0.5 * (lo + hi);   /* exact in binary64 */
                if (a < mid)
                    best = c;
                else if (a > mid)
                    best = c + 1;
                else
                    best = (c % 2 == 0) ? c : c + 1;
                break;
            }
        }
    }
    return sign | best;
}

/*
 * NVFP4 quantization of a row-major bf16 matrix X [R, C] (C % 16 == 0), blocks of 16 along
 * C.  Xq: [R, C/2] packed codes; sX: [R, C/16] E4M3 block scales; *g: the global scale.
 * Single-threaded (the tensor amax couples every element).
 */
int oracle_quantize_nvfp4(const uint16_t *X, uint8_t *Xq, uint8_t *sX, float *g, int64_t R,
                          int64_t C)
{
    if (R < 0 || C < 0 || C % 16 != 0)
        return -1;
    float amax_t = 0.0f;
    for (int64_t i = 0; i < R * C; ++i) {
        float v = fabsf(bf16_to_f32(X[i]));
        if (v > amax_t)
            amax_t = v;
    }
    float gs = amax_t / 2688.0f;
    *g = gs;
    float six_g = 6.0f * gs;
    int64_t CB = C / 16;
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t b = 0; b < CB; ++b) {
            const uint16_t *xb = X + r * C + b * 16;
            float amax_b = 0.0f;
            for (int j = 0; j < 16; ++j) {
                float v = fabsf(bf16_to_f32(xb[j]));
                if (v > amax_b)
                    amax_b = v;
            }
            uint8_t sb = (six_g == 0.0f) ? 0 : oracle_e4m3_encode(amax_b / six_g);
            sX[r * CB + b] = sb;
            float D = (float)oracle_e4m3_decode(sb) * gs;
            for (int j = 0; j < 16; j += 2) {
                uint8_t c[2];
                for (int h = 0; h < 2; ++h) {
                    float x = bf16_to_f32(xb[j + h]);
                    c[h] = (D == 0.0f) ? (signbit(x) ? 8 : 0) : oracle_e2m1_encode(x / D);
                }
                Xq[(r * C + b * 16 + j) / 2] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
    }
    return 0;
}

/*
 * NVFP4 GEMM reference, rows m0 <= m < m1:  C[m,n] = sum_k a[m,k] b[n,k] with
 * a = gA * dec(sA[m,k/16]) * e2m1(A_q[m,k]) and b = gB * dec(sB[n,k/16]) * e2m1(B_q[n,k])
 * in fp64 (k ascending); S = sum |a b|.  A_q [M, K/2], B_q [N, K/2] packed; K % 16 == 0.
 */
int oracle_gemm_nvfp4_f64(const uint8_t *Aq, const uint8_t *sA, float gA, const uint8_t *Bq,
                          const uint8_t *sB, float gB, int64_t M, int64_t N, int64_t K,
                          double *C, double *S, int64_t m0, int64_t m1)
{
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0 || m0 < 0 || m1 > M || m0 > m1)
        return -1;
    int64_t KB = K / 16;
    double *arow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!arow)
        return -1;
    for (int64_t m = m0; m < m1; ++m) {
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = Aq[(m * K + k) / 2];
            uint8_t code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
            arow[k] = (double)gA * oracle_e4m3_decode(sA[m * KB + k / 16]) * oracle_e2m1_decode(code);
        }
        for (int64_t n = 0; n < N; ++n) {
            double c = 0.0, s = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                uint8_t byte = Bq[(n * K + k) / 2];
                uint8_t code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
                double b = (double)gB * oracle_e4m3_decode(sB[n * KB + k / 16]) *
                           oracle_e2m1_decode(code);
                double p = arow[k] * b;
                c += p;
                s += fabs(p);
            }
            C[m * N + n] = c;
            if (S)
                S[m * N + n] = s;
        }
    }
    free(arow);
    return 0;
}

/* Element-wise encode of n fp32 values (a loop over oracle_e4m3_encode). */
void oracle_e4m3_encode_array(const float *y, uint8_t *q, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        q[i] = oracle_e4m3_encode(y[i]);
}
