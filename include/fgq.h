/*
 * fgq.h -- C ABI of libfgq: fine-grained FP8 (E4M3) quantization and the block-scaled FP8
 * GEMM on AMD MI355X (gfx950).
 *
 * Method: page "Fine-Grained FP8/FP4 Quantization".
 *   - section "Scaling Granularities": activations get one fp32 scale per 1x128 row tile,
 *     weights one per 128x128 block;
 *   - section "DeepGEMM: Tile-wise and Block-wise Scaling": scale_A is [M, K/128] and
 *     scale_B is [K/128, N/128], both fp32 row-major; the GEMM multiplies every 128-wide
 *     K-chunk partial of A_q * B_q by scale_A[m,kb] * scale_B[kb,nb] and accumulates in fp32;
 *   - table "UE8M0 vs E4M3 Scale Formats": E4M3 reaches 448.
 * Readings fixed here where the page is silent: the stored scale is s = amax/448 (fp32
 * IEEE divide) so that x ~= code_value * s; codes are OCP E4M3FN ("fn": bias 7, no
 * infinities, 0x7F/0xFF NaN) of fl32(x/s), rounded to nearest-even, saturating at 448; an
 * all-zero group has s = 0 and signed-zero codes; the GEMM overwrites C.
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers (HIP/ROCm memory on the current device), owned
 *     by the caller; the library allocates and frees nothing.  They must be 16-byte
 *     aligned.  Inputs and outputs must not overlap.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls are
 *     asynchronous on that stream; they return after the launch.
 *   - The return value reports argument validation and the launch status only
 *     (FGQ_OK or a negative fgq_status).  On an error nothing is launched and no output is
 *     touched.  Faults inside a kernel surface on the caller's next synchronisation.
 *   - Empty problems (a zero dimension) are valid and launch nothing, except that the GEMM
 *     with K == 0 writes C = 0.
 *   - No global mutable state: concurrent calls on different streams are safe.
 */
#ifndef FGQ_H
#define FGQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FGQ_OK = 0,
    FGQ_ERR_NULL = -1,   /* a required pointer is NULL */
    FGQ_ERR_SHAPE = -2,  /* negative size, K or N not a multiple of 128, or size too large
                            (including a launch grid beyond the 2^32 work-items one HIP
                            dispatch can count; refused before anything is enqueued) */
    FGQ_ERR_ALIGN = -3,  /* a pointer is not 16-byte aligned */
    FGQ_ERR_DTYPE = -4,  /* unknown out_dtype */
    FGQ_ERR_LAUNCH = -5, /* the HIP launch failed (hipGetLastError) */
    FGQ_ERR_ALIAS = -6,  /* an output overlaps an input or another output */
    FGQ_ERR_VARIANT = -7, /* unknown GEMM kernel variant */
    FGQ_ERR_WORKSPACE = -8 /* a workspace is missing or smaller than the call needs */
} fgq_status;

typedef enum { FGQ_OUT_F32 = 0, FGQ_OUT_BF16 = 1 } fgq_out_dtype;

/*
 * 1x128 activation quantization.
 *   X       in : bf16 [M, K] row-major (2*M*K bytes)
 *   Xq      out: E4M3FN codes [M, K] row-major (M*K bytes)
 *   scale_X out: fp32 [M, K/128] row-major; scale_X[m*(K/128)+kb] = amax/448 of
 *                X[m, 128kb .. 128kb+127]
 * Requires M >= 0, K >= 0, K % 128 == 0, M*K <= 2^36 (the elements one launch covers).
 */
int fgq_quantize_act_1x128(const void* X, void* Xq, float* scale_X, int64_t M, int64_t K,
                           void* stream);

/*
 * 128x128 weight quantization.
 *   W       in : bf16 [K, N] row-major (N contiguous)
 *   Wq      out: E4M3FN codes [K, N] row-major
 *   scale_W out: fp32 [K/128, N/128] row-major; scale_W[kb*(N/128)+nb] = amax/448 of
 *                W[128kb .. 128kb+127][128nb .. 128nb+127]
 * Requires K, N >= 0 and multiples of 128, K/128 < 65536, N/128 < 2^31.
 */
int fgq_quantize_weight_128x128(const void* W, void* Wq, float* scale_W, int64_t K,
                                int64_t N, void* stream);

/*
 * Block-scaled FP8 GEMM:
 *   C[m,n] = sum_{kb < K/128} scale_A[m,kb] * scale_B[kb, n/128]
 *                             * sum_{k in chunk kb} dec(A_q[m,k]) * dec(B_q[k,n])
 * with the chunk partial formed on the matrix cores from the exactly decoded E4M3 codes
 * and every scaled partial added to an fp32 accumulator (summation order differs from a
 * serial sum: results are correct to fp32 rounding, not bit-identical to any particular
 * order; a given shape, variant and input always gives the same bits).
 *   A_q     in : E4M3FN [M, K] row-major       scale_A in: fp32 [M, K/128] row-major
 *   B_q     in : E4M3FN [K, N] row-major (N contiguous)
 *   scale_B in : fp32 [K/128, N/128] row-major
 *   C       out: [M, N] row-major, fp32 (out_dtype FGQ_OUT_F32) or bf16 rounded to
 *                nearest-even (FGQ_OUT_BF16); overwritten.
 * Requires M, N, K >= 0, K % 128 == 0, N % 128 == 0, every dimension below 2^31 and
 * ceil(M/128) * (N/128) below 2^31 (the number of output tiles).
 */
int fgq_gemm_fp8_blockscaled(const void* A_q, const float* scale_A, const void* B_q,
                             const float* scale_B, void* C, int64_t M, int64_t N, int64_t K,
                             int out_dtype, void* stream);

/*
 * Kernel families of the GEMM.  Every variant computes the same function within the same
 * tolerance; they differ in tiling:
 *   WIDE_256x128 / WIDE_128x128: one workgroup per output tile, K walked in order;
 *   NARROW_64x32 / NARROW_64x64: 64x32 or 64x64 tiles whose K chunks are split over the 4
 *                 waves of a workgroup (each wave the whole tile over its own chunks) and
 *                 summed in a fixed order, for shapes with few output tiles;
 *   SKINNY_128x32: 128x32 tiles, 12 waves in three groups of four (32x32 each) that split
 *                 the K chunks, summed in a fixed order, for M <= 128 (decode-like).
 * FGQ_GEMM_AUTO picks from the shape (wide while the wide tiles cover every CU, else one of
 * the narrow and skinny families); it is what fgq_gemm_fp8_blockscaled uses.
 */
typedef enum {
    FGQ_GEMM_AUTO = 0,
    FGQ_GEMM_WIDE_256x128 = 1,
    FGQ_GEMM_WIDE_128x128 = 2,
    FGQ_GEMM_NARROW_64x32 = 3,
    FGQ_GEMM_SKINNY_128x32 = 4,
    FGQ_GEMM_NARROW_64x64 = 5
} fgq_gemm_variant;

/*
 * fgq_gemm_fp8_blockscaled with an explicit kernel family (for tests and tuning).
 * Arguments, requirements and errors as fgq_gemm_fp8_blockscaled; in addition an unknown
 * `variant` gives FGQ_ERR_VARIANT, and NARROW_64x32 / NARROW_64x64 / SKINNY_128x32 require
 * ceil(M/64) * (N/32) / ceil(M/64) * (N/64) / ceil(M/128) * (N/32) below 2^31.
 */
int fgq_gemm_fp8_blockscaled_variant(const void* A_q, const float* scale_A, const void* B_q,
                                     const float* scale_B, void* C, int64_t M, int64_t N,
                                     int64_t K, int out_dtype, int variant, void* stream);

/*
 * The same GEMM with the K chunks also divided between workgroups (a stream-K style split;
 * page "Persistent kernel (grid = SM count, internal tile loop)", section "Variants": one
 * tile's K loop spread over several workgroups), for shapes whose output tiles are too few to
 * occupy the GPU (decode-like M <= 128: 128x7168 has 56 tiles of 128x128 for 256 CUs).
 * Workgroup (s, tile) forms the fp32 partial of its tile over the consecutive K chunks
 * [s*KB/splits, (s+1)*KB/splits), KB = K/128, into slice s of a caller-owned workspace
 * (fp32 [splits][M][N], splits*M*N*4 bytes); a second kernel on the same stream sums the slices
 * in slice order and writes C.  Every workspace element is written once and read once: no
 * atomics, and a given shape and split count always gives the same bits.  The sum differs
 * from the unsplit kernels' by fp32 rounding only (same tolerance).
 *
 * fgq_gemm_workspace_size: bytes fgq_gemm_fp8_blockscaled_ws needs for this shape on the
 *   current device (0: the shape runs unsplit and needs none); a negative fgq_status for an
 *   invalid shape.  The split count it plans: 1 (no workspace) unless K/128 >= 128 and the
 *   128x128 output tiles cover at most half of the GPU's CUs -- the second launch costs
 *   more than the split gains on shorter K -- else the largest power of two up to 16 whose
 *   workgroups fit one round of the CUs with at least 8 K chunks each.
 * fgq_gemm_fp8_blockscaled_ws: fgq_gemm_fp8_blockscaled with a workspace; it splits K as
 *   planned when workspace_bytes >= fgq_gemm_workspace_size(M, N, K), and otherwise (also
 *   with workspace == NULL) computes C exactly as fgq_gemm_fp8_blockscaled does, using no
 *   workspace.  The workspace is device memory owned by the caller, 16-byte aligned, not
 *   overlapping any operand; its contents on entry are irrelevant and on return undefined;
 *   calls that share a workspace must not overlap in time.
 * fgq_gemm_fp8_blockscaled_splitk: the same with an explicit split count (tests, tuning):
 *   1 <= splits <= 16 and splits <= K/128 (FGQ_ERR_SHAPE otherwise); splits == 1 is the
 *   unsplit choice; splits > 1 needs workspace_bytes >= splits*M*N*4 (FGQ_ERR_WORKSPACE).
 * Other arguments, requirements and errors as fgq_gemm_fp8_blockscaled; FGQ_ERR_ALIAS when
 * the workspace overlaps an operand.
 */
int64_t fgq_gemm_workspace_size(int64_t M, int64_t N, int64_t K);
int fgq_gemm_fp8_blockscaled_ws(const void* A_q, const float* scale_A, const void* B_q,
                                const float* scale_B, void* C, int64_t M, int64_t N, int64_t K,
                                int out_dtype, void* workspace, int64_t workspace_bytes,
                                void* stream);
int fgq_gemm_fp8_blockscaled_splitk(const void* A_q, const float* scale_A, const void* B_q,
                                    const float* scale_B, void* C, int64_t M, int64_t N,
                                    int64_t K, int out_dtype, int splits, void* workspace,
                                    int64_t workspace_bytes, void* stream);

/*
 * fgq_gemm_fp8_blockscaled_ws for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): no workspace argument;
 * the planned K split keeps its partials in a device array inside the library, 16 MiB per
 * GPU, set up on the first call on each device and held until the process ends.  The call
 * allocates nothing.  Every call on a GPU shares that GPU's array, so calls that overlap in
 * time on one GPU (different streams, or threads) race and must be serialized by the
 * caller.  Returns FGQ_ERR_WORKSPACE when the planned split would need more than 16 MiB
 * (fgq_gemm_workspace_size(M, N, K) > 16 MiB; never on a GPU of up to 256 CUs, where the
 * plan needs at most 16 MiB), FGQ_ERR_LAUNCH when the array cannot be located on the current
 * device; otherwise arguments, results and errors as fgq_gemm_fp8_blockscaled_ws.
 */
int fgq_gemm_fp8_blockscaled_noalloc(const void* A_q, const float* scale_A, const void* B_q,
                                     const float* scale_B, void* C, int64_t M, int64_t N,
                                     int64_t K, int out_dtype, void* stream);

/*
 * Block-scaled FP8 GEMM with the next layer's activation quantization fused into its
 * epilogue (page "Kernel Fusion": one launch instead of a round trip through memory):
 *   C       out: bf16 [M, N], the GEMM of fgq_gemm_fp8_blockscaled with FGQ_OUT_BF16
 *   C_q     out: E4M3FN [M, N]         } exactly fgq_quantize_act_1x128 applied to the C
 *   scale_C out: fp32 [M, N/128]        } written here (bit for bit)
 * Arguments, requirements and errors as fgq_gemm_fp8_blockscaled; none of the three outputs
 * may overlap each other or an input.  One launch of the wide kernel family (each workgroup
 * owns whole 128-column groups of its rows) when its 128x128 tiles cover the GPU's CUs at
 * least once; for shapes with fewer tiles, where those tiles would leave CUs idle, the call
 * enqueues the GEMM family fgq_gemm_fp8_blockscaled would pick and then the activation
 * quantizer over that C (two launches on the stream, same contract).
 */
int fgq_gemm_fp8_blockscaled_quant(const void* A_q, const float* scale_A, const void* B_q,
                                   const float* scale_B, void* C, void* C_q, float* scale_C,
                                   int64_t M, int64_t N, int64_t K, void* stream);

/*
 * UE8M0 (power-of-two) scale variants.  Page "Fine-Grained FP8/FP4 Quantization", section
 * "Blackwell: Native Block Scaling" and table "UE8M0 vs E4M3 Scale Formats": a scale is one
 * unsigned exponent byte e standing for 2^(e-127).  Same 1x128 / 128x128 groups, shapes and
 * code rule as the fp32-scale calls; the scale of a group is the smallest power of two
 * 2^(e-127), 0 <= e <= 254, with 448 * 2^(e-127) >= amax (e = 0 for groups whose amax is
 * below 448 * 2^-127, including all-zero groups), so codes never saturate and x / scale is
 * exact.  Scale arrays are uint8 with the same shapes as the fp32 ones.  Requirements and
 * errors as the fp32-scale calls.
 */
int fgq_quantize_act_1x128_ue8m0(const void* X, void* Xq, uint8_t* scale_X, int64_t M,
                                 int64_t K, void* stream);
int fgq_quantize_weight_128x128_ue8m0(const void* W, void* Wq, uint8_t* scale_W, int64_t K,
                                      int64_t N, void* stream);
/*
 * GEMM on UE8M0 scales: C as fgq_gemm_fp8_blockscaled with scale_A[m,kb] = 2^(eA-127) and
 * scale_B[kb,nb] = 2^(eB-127); the combined scale of a chunk is the exact power of two
 * 2^(eA+eB-254) (flushed to zero below the fp32 range).  `variant` as in
 * fgq_gemm_fp8_blockscaled_variant (FGQ_GEMM_AUTO to let the shape decide).
 */
int fgq_gemm_fp8_blockscaled_ue8m0(const void* A_q, const uint8_t* scale_A, const void* B_q,
                                   const uint8_t* scale_B, void* C, int64_t M, int64_t N,
                                   int64_t K, int out_dtype, int variant, void* stream);

/*
 * NVFP4 two-level scaling (page "Fine-Grained FP8/FP4 Quantization", section "NVFP4
 * Two-Level Scaling"): E2M1 codes (0, 0.5, 1, 1.5, 2, 3, 4, 6 and signs), one E4M3 scale
 * per 16 consecutive elements along the contiguous dimension, one fp32 global scale per
 * tensor; value = global * block * e2m1.  Scales: global = amax/2688 (2688 = 448*6),
 * block = E4M3(amax_block / (6*global)), code = E2M1(x / (block*global)) nearest-even,
 * saturating at 6 (signed zeros where block*global is 0).
 *   X            in : bf16 [R, C] row-major, C % 16 == 0, R*C <= 2^35
 *   Xq           out: packed codes [R, C/2], element 2i in the low nibble of byte i
 *   scale_X      out: E4M3 [R, C/16]
 *   global_scale out: fp32 [FGQ_NVFP4_GLOBAL_FLOATS]; element 0 receives the global scale, the
 *                     others are scratch of the call (overwritten; the amax pass leaves one
 *                     candidate per workgroup there, so no atomics and no clearing launch)
 * Two launches on `stream` (the tensor amax is needed before any block is coded).
 */
#define FGQ_NVFP4_GLOBAL_FLOATS 512
int fgq_quantize_nvfp4(const void* X, void* Xq, uint8_t* scale_X, float* global_scale,
                       int64_t R, int64_t C, void* stream);
/*
 * NVFP4 GEMM: C[m,n] = sum_k a[m,k] * b[n,k], a and b dequantized as above.  Both operands
 * are quantized along K: A_q [M, K/2] with scale_A [M, K/16], and the weight stored as its
 * transpose B_q [N, K/2] with scale_B [N, K/16]; global_A / global_B are device pointers to
 * the fp32 global scales.  C fp32 or bf16 [M, N], overwritten.  Requires K % 128 == 0 and
 * N % 128 == 0; the products are summed to fp32 accuracy (same tolerance as the FP8 GEMM).
 */
int fgq_gemm_nvfp4(const void* A_q, const uint8_t* scale_A, const float* global_A,
                   const void* B_q, const uint8_t* scale_B, const float* global_B, void* C,
                   int64_t M, int64_t N, int64_t K, int out_dtype, void* stream);

/* Static text for a status code. */
const char* fgq_status_string(int status);

/* ABI version (major*10000 + minor*100 + patch). */
int fgq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FGQ_H */
