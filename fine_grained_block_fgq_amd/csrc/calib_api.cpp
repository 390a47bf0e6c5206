// calib_api.cpp -- C entry points of libfgq_calib (declared in include/fgq_calib.h): the
// measurement-only kernels of calib.hip behind the same argument checks and status codes as
// libfgq.  None of them is a step of the quantization or the GEMM.
#include "../../include/fgq_calib.h"
#include "api_util.hpp"
#include "calib_launch.hpp"

#include <stdint.h>

using fgq_api::launch_status;
using fgq_api::misaligned;
using fgq_api::overlap;

extern "C" {

int fgq_calib_stream(const void* src, void* dst, int64_t n16, void* stream)
{
    if (n16 < 0 || n16 > (int64_t(1) << 34))
        return FGQ_ERR_SHAPE;
    if (n16 == 0)
        return FGQ_OK;
    if (!src || !dst)
        return FGQ_ERR_NULL;
    if (misaligned(src) || misaligned(dst))
        return FGQ_ERR_ALIGN;
    if (overlap(src, 16 * n16, dst, 8 * n16))
        return FGQ_ERR_ALIAS;
    return launch_status(fgq::launch_calib_stream(src, dst, n16, static_cast<hipStream_t>(stream)));
}

int fgq_calib_mfma_f16(float* out, int64_t blocks, int64_t iters, void* stream)
{
    if (blocks < 1 || blocks > (int64_t(1) << 20) || iters < 0 || iters > (int64_t(1) << 24))
        return FGQ_ERR_SHAPE;
    if (!out)
        return FGQ_ERR_NULL;
    if (misaligned(out))
        return FGQ_ERR_ALIGN;
    return launch_status(
        fgq::launch_calib_mfma_f16(out, blocks, iters, static_cast<hipStream_t>(stream)));
}

int fgq_calib_mfma_fp8(float* out, int64_t blocks, int64_t iters, void* stream)
{
    if (blocks < 1 || blocks > (int64_t(1) << 20) || iters < 0 || iters > (int64_t(1) << 24))
        return FGQ_ERR_SHAPE;
    if (!out)
        return FGQ_ERR_NULL;
    if (misaligned(out))
        return FGQ_ERR_ALIGN;
    return launch_status(
        fgq::launch_calib_mfma_fp8(out, blocks, iters, static_cast<hipStream_t>(stream)));
}

int fgq_probe_fp8_mfma_partials(const void* A_q, const void* B_q, float* P, int64_t M,
                                int64_t N, int64_t K, void* stream)
{
    if (M < 0 || N < 0 || K < 0 || M % 16 || N % 16 || K % 128 || M > (int64_t(1) << 16) ||
        N > (int64_t(1) << 16) || K > (int64_t(1) << 16))
        return FGQ_ERR_SHAPE;
    if (M == 0 || N == 0 || K == 0)
        return FGQ_OK;
    if (!A_q || !B_q || !P)
        return FGQ_ERR_NULL;
    if (misaligned(A_q) || misaligned(B_q) || misaligned(P))
        return FGQ_ERR_ALIGN;
    const int64_t np = (K / 128) * M * N * 4;
    if (overlap(P, np, A_q, M * K) || overlap(P, np, B_q, K * N))
        return FGQ_ERR_ALIAS;
    return launch_status(fgq::launch_probe_fp8_mfma_partials(A_q, B_q, P, M, N, K,
                                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"
