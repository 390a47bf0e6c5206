/*
 * fgq_calib.h -- C ABI of libfgq_calib, the measurement library that sits beside libfgq on
 * MI355X (gfx950).  Nothing here is a step of the quantization or of the block-scaled GEMM
 * (those are in fgq.h); these kernels only give the benchmark its measured ceilings and
 * measure the accuracy of an instruction the GEMM does not use.
 *
 * Conventions as in fgq.h: device pointers owned by the caller, 16-byte aligned; `stream` is
 * a hipStream_t passed as void*; calls are asynchronous and return an fgq_status (FGQ_OK or a
 * negative code from fgq.h) for argument validation and the launch only.
 */
#ifndef FGQ_CALIB_H
#define FGQ_CALIB_H

#include <stdint.h>

#include "fgq.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fgq_calib_stream: the activation quantizer's memory traffic with no arithmetic, as a
 * streaming ceiling for its HBM fraction.  For i < n16 it reads the 16 bytes at src + 16*i and
 * writes 8 bytes (an XOR of its words) at dst + 8*i; two 16-byte loads in flight per lane.
 *   src  in: device, n16*16 bytes, 16-byte aligned     dst  out: device, n16*8 bytes
 * Errors: FGQ_ERR_SHAPE (n16 < 0 or too large), FGQ_ERR_NULL, FGQ_ERR_ALIGN, FGQ_ERR_ALIAS.
 */
int fgq_calib_stream(const void* src, void* dst, int64_t n16, void* stream);

/*
 * fgq_calib_mfma_f16: only f16 MFMAs (v_mfma_f32_16x16x32_f16, the instruction that forms the
 * GEMM's chunk partials) in four independent accumulation chains per wave, `blocks` workgroups
 * of 8 waves: the matrix-core rate this GPU sustains at its loaded clock.  Work: blocks * 8 *
 * iters * 16 MFMAs of 16384 flop each.  `out` (device, blocks*512 floats) gets a checksum per
 * thread.  Errors: FGQ_ERR_SHAPE (blocks outside [1, 2^20] or iters outside [0, 2^24]),
 * FGQ_ERR_NULL, FGQ_ERR_ALIGN.
 */
int fgq_calib_mfma_f16(float* out, int64_t blocks, int64_t iters, void* stream);

/*
 * fgq_calib_mfma_fp8: the same with FP8 (E4M3) MFMAs (v_mfma_f32_16x16x128_f8f6f4), which the
 * GEMM does not use.  Work: blocks * 8 * iters * 16 MFMAs of 65536 flop each.  Same arguments
 * and errors as fgq_calib_mfma_f16.
 */
int fgq_calib_mfma_fp8(float* out, int64_t blocks, int64_t iters, void* stream);

/*
 * fgq_probe_fp8_mfma_partials: the 128-K chunk partials P[kb][m][n] = sum over the chunk of
 * A_q[m,k] * B_q[k,n], each formed by one FP8 MFMA (v_mfma_f32_16x16x128_f8f6f4) per 16x16
 * tile, unscaled, so that the accuracy of that instruction's own sum can be measured against
 * the exact sums (it is why the GEMM forms its partials with f16 MFMAs).
 *   A_q  in: device, E4M3 [M, K] row-major, 16-byte aligned
 *   B_q  in: device, E4M3 [K, N] row-major (N contiguous)
 *   P    out: device, fp32 [K/128, M, N], overwritten
 * M and N multiples of 16, K of 128, each at most 65536; any of them 0: no-op.
 * Errors: FGQ_ERR_SHAPE, FGQ_ERR_NULL, FGQ_ERR_ALIGN, FGQ_ERR_ALIAS (P overlaps an input).
 */
int fgq_probe_fp8_mfma_partials(const void* A_q, const void* B_q, float* P, int64_t M,
                                int64_t N, int64_t K, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FGQ_CALIB_H */
