/* Runs every entry point of oracle/fgq_oracle.c on small seeded inputs, for a build with
 * -fsanitize=address,undefined (tests/test_sanitize.py): any out-of-bounds access, signed
 * overflow, bad shift or out-of-range float conversion aborts.  Inputs are finite bf16 values
 * spanning the whole exponent range (zeros, subnormals, the largest finite), plus all-zero
 * groups.  Prints "ok" and a checksum, exits 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_e4m3_decode(uint8_t code);
uint8_t oracle_e4m3_encode(float y);
void oracle_e4m3_encode_array(const float *y, uint8_t *q, int64_t n);
int oracle_quantize_act_1x128(const uint16_t *X, uint8_t *Xq, float *sX, int64_t M, int64_t K,
                              int64_t m0, int64_t m1);
int oracle_quantize_weight_128x128(const uint16_t *W, uint8_t *Wq, float *sW, int64_t K,
                                   int64_t N, int64_t kb0, int64_t kb1);
int oracle_gemm_f64(const uint8_t *Aq, const float *sA, const uint8_t *Bq, const float *sB,
                    int64_t M, int64_t N, int64_t K, double *C, double *S, int64_t m0, int64_t m1);
int oracle_gemm_f64_at(const uint8_t *Aq, const float *sA, const uint8_t *Bq, const float *sB,
                       int64_t M, int64_t N, int64_t K, const int64_t *rows, const int64_t *cols,
                       int64_t count, double *C, double *S);
double oracle_ue8m0_decode(uint8_t e);
int oracle_quantize_act_1x128_ue8m0(const uint16_t *X, uint8_t *Xq, uint8_t *sX, int64_t M,
                                    int64_t K, int64_t m0, int64_t m1);
int oracle_quantize_weight_128x128_ue8m0(const uint16_t *W, uint8_t *Wq, uint8_t *sW,
                                         int64_t K, int64_t N, int64_t kb0, int64_t kb1);
double oracle_e2m1_decode(uint8_t code);
uint8_t oracle_e2m1_encode(float y);
int oracle_quantize_nvfp4(const uint16_t *X, uint8_t *Xq, uint8_t *sX, float *g, int64_t R,
                          int64_t C);
int oracle_gemm_nvfp4_f64(const uint8_t *Aq, const uint8_t *sA, float gA, const uint8_t *Bq,
                          const uint8_t *sB, float gB, int64_t M, int64_t N, int64_t K,
                          double *C, double *S, int64_t m0, int64_t m1);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 16);
}

/* a finite bf16 bit pattern: any sign, any exponent below 0xFF, any mantissa */
static uint16_t finite_bf16(void)
{
    uint16_t h = (uint16_t)next32();
    if (((h >> 7) & 0xFF) == 0xFF)
        h &= (uint16_t)~0x0080; /* exponent 0xFE instead */
    return h;
}

static void fill(uint16_t *x, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        x[i] = finite_bf16();
}

static double checksum = 0.0;
static void add(double v)
{
    if (isfinite(v))
        checksum += fabs(v) * 1e-30;
}

static void fail(const char *what)
{
    printf("FAIL %s\n", what);
    exit(1);
}

int main(void)
{
    for (int c = 0; c < 256; ++c)
        add(oracle_e4m3_decode((uint8_t)c)), add(oracle_ue8m0_decode((uint8_t)c));
    for (int c = 0; c < 16; ++c)
        add(oracle_e2m1_decode((uint8_t)c));
    {
        float y[4096];
        uint8_t q[4096];
        for (int i = 0; i < 4096; ++i) {
            uint32_t b = next32();
            if (((b >> 23) & 0xFF) == 0xFF)
                b &= ~(1u << 23);
            memcpy(&y[i], &b, 4);
            add(oracle_e4m3_encode(y[i]) + oracle_e2m1_encode(y[i]));
        }
        oracle_e4m3_encode_array(y, q, 4096);
        for (int i = 0; i < 4096; ++i)
            add(q[i]);
    }

    /* activations [M,K] with one all-zero tile, weights [K,N] with one all-zero block */
    const int64_t M = 5, K = 384, N = 256;
    uint16_t *X = malloc(sizeof(uint16_t) * M * K), *W = malloc(sizeof(uint16_t) * K * N);
    uint8_t *Xq = malloc(M * K), *Wq = malloc(K * N), *eX = malloc(M * (K / 128)),
            *eW = malloc((K / 128) * (N / 128));
    float *sX = malloc(sizeof(float) * M * (K / 128)),
          *sW = malloc(sizeof(float) * (K / 128) * (N / 128));
    double *C = malloc(sizeof(double) * M * N), *S = malloc(sizeof(double) * M * N);
    fill(X, M * K);
    fill(W, K * N);
    memset(X + 2 * K + 128, 0, 128 * sizeof(uint16_t));
    for (int64_t r = 128; r < 256; ++r)
        memset(W + r * N + 128, 0, 128 * sizeof(uint16_t));
    if (oracle_quantize_act_1x128(X, Xq, sX, M, K, 0, M) != 0)
        fail("quantize_act");
    if (oracle_quantize_weight_128x128(W, Wq, sW, K, N, 0, K / 128) != 0)
        fail("quantize_weight");
    if (oracle_gemm_f64(Xq, sX, Wq, sW, M, N, K, C, S, 0, M) != 0)
        fail("gemm_f64");
    for (int64_t i = 0; i < M * N; ++i)
        add(C[i]), add(S[i]);
    {
        int64_t rows[16], cols[16];
        double c1[16], s1[16];
        for (int i = 0; i < 16; ++i)
            rows[i] = next32() % M, cols[i] = next32() % N;
        if (oracle_gemm_f64_at(Xq, sX, Wq, sW, M, N, K, rows, cols, 16, c1, s1) != 0)
            fail("gemm_f64_at");
        for (int i = 0; i < 16; ++i)
            if (c1[i] != C[rows[i] * N + cols[i]] && !(isnan(c1[i]) && isnan(C[rows[i] * N + cols[i]])))
                fail("gemm_f64_at differs from gemm_f64");
    }
    if (oracle_quantize_act_1x128_ue8m0(X, Xq, eX, M, K, 0, M) != 0)
        fail("quantize_act_ue8m0");
    if (oracle_quantize_weight_128x128_ue8m0(W, Wq, eW, K, N, 0, K / 128) != 0)
        fail("quantize_weight_ue8m0");
    for (int64_t i = 0; i < M * (K / 128); ++i)
        add(eX[i]);
    /* bad shapes are refused, not read */
    if (oracle_quantize_act_1x128(X, Xq, sX, M, 100, 0, M) != -1 ||
        oracle_gemm_f64(Xq, sX, Wq, sW, M, 100, K, C, S, 0, M) != -1)
        fail("shape checks");

    /* NVFP4: A [M,K] and the weight's transpose [N,K] (blocks of 16 along K) */
    {
        const int64_t Kn = 64, Nn = 32;
        uint16_t *A = malloc(sizeof(uint16_t) * M * Kn), *B = malloc(sizeof(uint16_t) * Nn * Kn);
        uint8_t *Aq = malloc(M * Kn / 2), *Bq = malloc(Nn * Kn / 2), *sA = malloc(M * Kn / 16),
                *sB = malloc(Nn * Kn / 16);
        double *Cn = malloc(sizeof(double) * M * Nn), *Sn = malloc(sizeof(double) * M * Nn);
        float gA, gB;
        /* moderate magnitudes so the tensor amax and the block scales stay in range */
        for (int64_t i = 0; i < M * Kn; ++i)
            A[i] = (uint16_t)((next32() & 0x807F) | (0x3C00 + (next32() % 0x0800)));
        for (int64_t i = 0; i < Nn * Kn; ++i)
            B[i] = (uint16_t)((next32() & 0x807F) | (0x3800 + (next32() % 0x0800)));
        memset(A + Kn, 0, 16 * sizeof(uint16_t));
        if (oracle_quantize_nvfp4(A, Aq, sA, &gA, M, Kn) != 0 ||
            oracle_quantize_nvfp4(B, Bq, sB, &gB, Nn, Kn) != 0)
            fail("quantize_nvfp4");
        if (oracle_gemm_nvfp4_f64(Aq, sA, gA, Bq, sB, gB, M, Nn, Kn, Cn, Sn, 0, M) != 0)
            fail("gemm_nvfp4_f64");
        for (int64_t i = 0; i < M * Nn; ++i)
            add(Cn[i]), add(Sn[i]);
        free(A), free(B), free(Aq), free(Bq), free(sA), free(sB), free(Cn), free(Sn);
    }
    free(X), free(W), free(Xq), free(Wq), free(eX), free(eW), free(sX), free(sW), free(C), free(S);
    printf("ok %.6g\n", checksum);
    return 0;
}
