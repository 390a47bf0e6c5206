// calib_launch.hpp -- host-side launchers of the measurement kernels in calib.hip (internal to
// libfgq_calib).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fgq_launch.hpp"

namespace fgq {

// measured ceilings (calib.hip): a streaming kernel with the activation quantizer's traffic
// (n16 lanes' worth: 16 bytes read from src and 8 written to dst each), f16 MFMAs only
// (blocks x 8 waves x iters x 16 MFMAs of 16x16x32; out holds blocks*512 floats), FP8 MFMAs
// only (the same count of 16x16x128 f8f6f4); and the FP8-MFMA chunk partials of A_q [M,K] and
// B_q [K,N] into P [K/128][M][N] (M, N multiples of 16, K of 128)
hipError_t launch_calib_stream(const void* src, void* dst, int64_t n16, hipStream_t stream);
hipError_t launch_calib_mfma_f16(float* out, int64_t blocks, int64_t iters, hipStream_t stream);
hipError_t launch_calib_mfma_fp8(float* out, int64_t blocks, int64_t iters, hipStream_t stream);
hipError_t launch_probe_fp8_mfma_partials(const void* A_q, const void* B_q, float* P, int64_t M,
                                          int64_t N, int64_t K, hipStream_t stream);

}  // namespace fgq
