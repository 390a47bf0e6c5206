// api.cpp -- the C ABI of libfgq (declared in include/fgq.h): argument validation, then
// the gfx950 launch on the caller's stream.  No allocation, no global mutable state.
#include "../../include/fgq.h"
#include "fgq_launch.hpp"
#include "api_util.hpp"

#include <stdint.h>

namespace {

using fgq_api::launch_status;
using fgq_api::misaligned;
using fgq_api::overlap;

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
static_assert(FGQ_NVFP4_GLOBAL_FLOATS == fgq::kNvfp4GlobalFloats, "NVFP4 global-scale array");

// argument checks shared by the fp32-scale and UE8M0-scale entry points (ss: bytes per
// scale); FGQ_OK for a valid call, including an empty one
int check_act(const void* X, const void* Xq, const void* sX, int64_t M, int64_t K, int ss)
{
    if (M < 0 || K < 0 || K % 128 != 0 || M > kMaxDim || K > kMaxDim)
        return FGQ_ERR_SHAPE;
    // one launch: M*K/16 work-items, counted in 32 bits
    if (M > 0 && K > 0 && M > ((int64_t(1) << 36) / K))
        return FGQ_ERR_SHAPE;
    if (M == 0 || K == 0)
        return FGQ_OK;
    if (!X || !Xq || !sX)
        return FGQ_ERR_NULL;
    if (misaligned(X) || misaligned(Xq) || misaligned(sX))
        return FGQ_ERR_ALIGN;
    const int64_t nx = 2 * M * K, nq = M * K, ns = ss * M * (K / 128);
    if (overlap(X, nx, Xq, nq) || overlap(X, nx, sX, ns) || overlap(Xq, nq, sX, ns))
        return FGQ_ERR_ALIAS;
    return FGQ_OK;
}

int check_weight(const void* W, const void* Wq, const void* sW, int64_t K, int64_t N, int ss)
{
    if (K < 0 || N < 0 || K % 128 != 0 || N % 128 != 0 || K / 128 >= 65536 || N > kMaxDim)
        return FGQ_ERR_SHAPE;
    if (K == 0 || N == 0)
        return FGQ_OK;
    if (!W || !Wq || !sW)
        return FGQ_ERR_NULL;
    if (misaligned(W) || misaligned(Wq) || misaligned(sW))
        return FGQ_ERR_ALIGN;
    const int64_t nw = 2 * K * N, nq = K * N, ns = ss * (K / 128) * (N / 128);
    if (overlap(W, nw, Wq, nq) || overlap(W, nw, sW, ns) || overlap(Wq, nq, sW, ns))
        return FGQ_ERR_ALIAS;
    return FGQ_OK;
}

int check_gemm(const void* A_q, const void* scale_A, const void* B_q, const void* scale_B,
               const void* C, int64_t M, int64_t N, int64_t K, int out_dtype, int variant,
               int ss)
{
    if (out_dtype != FGQ_OUT_F32 && out_dtype != FGQ_OUT_BF16)
        return FGQ_ERR_DTYPE;
    if (variant < FGQ_GEMM_AUTO || variant > FGQ_GEMM_NARROW_64x64)
        return FGQ_ERR_VARIANT;
    if (M < 0 || N < 0 || K < 0 || K % 128 != 0 || N % 128 != 0 || M > kMaxDim ||
        N > kMaxDim || K > kMaxDim)
        return FGQ_ERR_SHAPE;
    if (((M + 127) / 128) * (N / 128) > kMaxDim)
        return FGQ_ERR_SHAPE;
    if (((variant == FGQ_GEMM_NARROW_64x32 || variant == FGQ_GEMM_NARROW_64x64) &&
         ((M + 63) / 64) * (N / 32) > kMaxDim) ||
        (variant == FGQ_GEMM_SKINNY_128x32 && ((M + 127) / 128) * (N / 32) > kMaxDim))
        return FGQ_ERR_SHAPE;
    if (M == 0 || N == 0)
        return FGQ_OK;
    if (!C || (K > 0 && (!A_q || !scale_A || !B_q || !scale_B)))
        return FGQ_ERR_NULL;
    if (misaligned(C) || (K > 0 && (misaligned(A_q) || misaligned(scale_A) ||
                                    misaligned(B_q) || misaligned(scale_B))))
        return FGQ_ERR_ALIGN;
    const int64_t nc = M * N * (out_dtype == FGQ_OUT_BF16 ? 2 : 4);
    if (K > 0 && (overlap(C, nc, A_q, M * K) || overlap(C, nc, B_q, K * N) ||
                  overlap(C, nc, scale_A, ss * M * (K / 128)) ||
                  overlap(C, nc, scale_B, ss * (K / 128) * (N / 128))))
        return FGQ_ERR_ALIAS;
    return FGQ_OK;
}

// the workspace of a K-split GEMM: splits * M * N floats that overlap no operand
int check_workspace(const void* A_q, const void* scale_A, const void* B_q, const void* scale_B,
                    const void* C, int64_t M, int64_t N, int64_t K, int out_dtype,
                    const void* ws, int64_t ws_bytes, int64_t need)
{
    if (ws_bytes < 0)
        return FGQ_ERR_SHAPE;
    if (need > 0 && (!ws || ws_bytes < need))
        return FGQ_ERR_WORKSPACE;
    if (need <= 0)
        return FGQ_OK;
    if (misaligned(ws))
        return FGQ_ERR_ALIGN;
    const int64_t nc = M * N * (out_dtype == FGQ_OUT_BF16 ? 2 : 4);
    if (overlap(ws, need, C, nc) || overlap(ws, need, A_q, M * K) ||
        overlap(ws, need, B_q, K * N) || overlap(ws, need, scale_A, 4 * M * (K / 128)) ||
        overlap(ws, need, scale_B, 4 * (K / 128) * (N / 128)))
        return FGQ_ERR_ALIAS;
    return FGQ_OK;
}

// bytes of the K-split workspace for `splits` splits (0 for none)
int64_t split_bytes(int64_t M, int64_t N, int splits)
{
    return splits > 1 ? (int64_t)splits * M * N * 4 : 0;
}

}  // namespace

extern "C" {

int fgq_version(void) { return 100; }

const char* fgq_status_string(int status)
{
    switch (status) {
    case FGQ_OK: return "ok";
    case FGQ_ERR_NULL: return "null pointer";
    case FGQ_ERR_SHAPE: return "invalid shape";
    case FGQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case FGQ_ERR_DTYPE: return "unknown output dtype";
    case FGQ_ERR_LAUNCH: return "kernel launch failed";
    case FGQ_ERR_ALIAS: return "output overlaps another buffer";
    case FGQ_ERR_VARIANT: return "unknown GEMM variant";
    case FGQ_ERR_WORKSPACE: return "workspace too small for the call";
    default: return "unknown status";
    }
}

int fgq_quantize_act_1x128(const void* X, void* Xq, float* scale_X, int64_t M, int64_t K,
                           void* stream)
{
    const int st = check_act(X, Xq, scale_X, M, K, 4);
    if (st != FGQ_OK || M == 0 || K == 0)
        return st;
    return launch_status(fgq::launch_quant_act_1x128(X, Xq, scale_X, M, K,
                                                     static_cast<hipStream_t>(stream)));
}

int fgq_quantize_act_1x128_ue8m0(const void* X, void* Xq, uint8_t* scale_X, int64_t M,
                                 int64_t K, void* stream)
{
    const int st = check_act(X, Xq, scale_X, M, K, 1);
    if (st != FGQ_OK || M == 0 || K == 0)
        return st;
    return launch_status(fgq::launch_quant_act_1x128_ue8m0(X, Xq, scale_X, M, K,
                                                           static_cast<hipStream_t>(stream)));
}

int fgq_quantize_weight_128x128(const void* W, void* Wq, float* scale_W, int64_t K,
                                int64_t N, void* stream)
{
    const int st = check_weight(W, Wq, scale_W, K, N, 4);
    if (st != FGQ_OK || K == 0 || N == 0)
        return st;
    return launch_status(fgq::launch_quant_weight_128x128(W, Wq, scale_W, K, N,
                                                          static_cast<hipStream_t>(stream)));
}

int fgq_quantize_weight_128x128_ue8m0(const void* W, void* Wq, uint8_t* scale_W, int64_t K,
                                      int64_t N, void* stream)
{
    const int st = check_weight(W, Wq, scale_W, K, N, 1);
    if (st != FGQ_OK || K == 0 || N == 0)
        return st;
    return launch_status(fgq::launch_quant_weight_128x128_ue8m0(
        W, Wq, scale_W, K, N, static_cast<hipStream_t>(stream)));
}

int fgq_gemm_fp8_blockscaled_variant(const void* A_q, const float* scale_A, const void* B_q,
                                     const float* scale_B, void* C, int64_t M, int64_t N,
                                     int64_t K, int out_dtype, int variant, void* stream)
{
    const int st = check_gemm(A_q, scale_A, B_q, scale_B, C, M, N, K, out_dtype, variant, 4);
    if (st != FGQ_OK || M == 0 || N == 0)
        return st;
    return launch_status(fgq::launch_gemm_fp8_blockscaled(A_q, scale_A, B_q, scale_B, C, M, N, K,
                                                          out_dtype == FGQ_OUT_BF16, variant,
                                                          static_cast<hipStream_t>(stream)));
}

int64_t fgq_gemm_workspace_size(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0 || K % 128 != 0 || N % 128 != 0 || M > kMaxDim ||
        N > kMaxDim || K > kMaxDim || ((M + 127) / 128) * (N / 128) > kMaxDim)
        return FGQ_ERR_SHAPE;
    if (M == 0 || N == 0 || K == 0)
        return 0;
    return split_bytes(M, N, fgq::gemm_splitk_plan(M, N, K));
}

int fgq_gemm_fp8_blockscaled_splitk(const void* A_q, const float* scale_A, const void* B_q,
                                    const float* scale_B, void* C, int64_t M, int64_t N,
                                    int64_t K, int out_dtype, int splits, void* workspace,
                                    int64_t workspace_bytes, void* stream)
{
    int st = check_gemm(A_q, scale_A, B_q, scale_B, C, M, N, K, out_dtype, FGQ_GEMM_AUTO, 4);
    if (st != FGQ_OK)
        return st;
    if (splits < 1 || splits > fgq::kSplitMax || (K > 0 && splits > K / 128))
        return FGQ_ERR_SHAPE;
    if (M == 0 || N == 0)
        return FGQ_OK;
    if (K == 0)
        splits = 1;
    st = check_workspace(A_q, scale_A, B_q, scale_B, C, M, N, K, out_dtype, workspace,
                         workspace_bytes, split_bytes(M, N, splits));
    if (st != FGQ_OK)
        return st;
    return launch_status(fgq::launch_gemm_fp8_blockscaled_splitk(
        A_q, scale_A, B_q, scale_B, C, M, N, K, out_dtype == FGQ_OUT_BF16, splits,
        static_cast<float*>(workspace), static_cast<hipStream_t>(stream)));
}

int fgq_gemm_fp8_blockscaled_ws(const void* A_q, const float* scale_A, const void* B_q,
                                const float* scale_B, void* C, int64_t M, int64_t N, int64_t K,
                                int out_dtype, void* workspace, int64_t workspace_bytes,
                                void* stream)
{
    int st = check_gemm(A_q, scale_A, B_q, scale_B, C, M, N, K, out_dtype, FGQ_GEMM_AUTO, 4);
    if (st != FGQ_OK || M == 0 || N == 0)
        return st;
    if (workspace_bytes < 0)
        return FGQ_ERR_SHAPE;
    // the K split when the workspace holds its partials, else the no-workspace choice
    int splits = K > 0 ? fgq::gemm_splitk_plan(M, N, K) : 1;
    if (!workspace || workspace_bytes < split_bytes(M, N, splits))
        splits = 1;
    st = check_workspace(A_q, scale_A, B_q, scale_B, C, M, N, K, out_dtype, workspace,
                         workspace_bytes, split_bytes(M, N, splits));
    if (st != FGQ_OK)
        return st;
    return launch_status(fgq::launch_gemm_fp8_blockscaled_splitk(
        A_q, scale_A, B_q, scale_B, C, M, N, K, out_dtype == FGQ_OUT_BF16, splits,
        static_cast<float*>(workspace), static_cast<hipStream_t>(stream)));
}

int fgq_gemm_fp8_blockscaled_noalloc(const void* A_q, const float* scale_A, const void* B_q,
                                     const float* scale_B, void* C, int64_t M, int64_t N,
                                     int64_t K, int out_dtype, void* stream)
{
    const int st = check_gemm(A_q, scale_A, B_q, scale_B, C, M, N, K, out_dtype, FGQ_GEMM_AUTO,
                              4);
    if (st != FGQ_OK || M == 0 || N == 0)
        return st;
    const int splits = K > 0 ? fgq::gemm_splitk_plan(M, N, K) : 1;
    if (split_bytes(M, N, splits) > fgq::kNoallocScratchBytes)
        return FGQ_ERR_WORKSPACE;
    return launch_status(fgq::launch_gemm_fp8_blockscaled_noalloc(
        A_q, scale_A, B_q, scale_B, C, M, N, K, out_dtype == FGQ_OUT_BF16, splits,
        static_cast<hipStream_t>(stream)));
}

int fgq_gemm_fp8_blockscaled_ue8m0(const void* A_q, const uint8_t* scale_A, const void* B_q,
                                   const uint8_t* scale_B, void* C, int64_t M, int64_t N,
                                   int64_t K, int out_dtype, int variant, void* stream)
{
    const int st = check_gemm(A_q, scale_A, B_q, scale_B, C, M, N, K, out_dtype, variant, 1);
    if (st != FGQ_OK || M == 0 || N == 0)
        return st;
    return launch_status(fgq::launch_gemm_fp8_blockscaled_ue8m0(
        A_q, scale_A, B_q, scale_B, C, M, N, K, out_dtype == FGQ_OUT_BF16, variant,
        static_cast<hipStream_t>(stream)));
}

int fgq_gemm_fp8_blockscaled(const void* A_q, const float* scale_A, const void* B_q,
                             const float* scale_B, void* C, int64_t M, int64_t N, int64_t K,
                             int out_dtype, void* stream)
{
    return fgq_gemm_fp8_blockscaled_variant(A_q, scale_A, B_q, scale_B, C, M, N, K, out_dtype,
                                            FGQ_GEMM_AUTO, stream);
}

int fgq_gemm_fp8_blockscaled_quant(const void* A_q, const float* scale_A, const void* B_q,
                                   const float* scale_B, void* C, void* C_q, float* scale_C,
                                   int64_t M, int64_t N, int64_t K, void* stream)
{
    if (M < 0 || N < 0 || K < 0 || K % 128 != 0 || N % 128 != 0 || M > kMaxDim ||
        N > kMaxDim || K > kMaxDim)
        return FGQ_ERR_SHAPE;
    if (((M + 127) / 128) * (N / 128) > kMaxDim)
        return FGQ_ERR_SHAPE;
    if (M == 0 || N == 0)
        return FGQ_OK;
    if (!C || !C_q || !scale_C || (K > 0 && (!A_q || !scale_A || !B_q || !scale_B)))
        return FGQ_ERR_NULL;
    if (misaligned(C) || misaligned(C_q) || misaligned(scale_C) ||
        (K > 0 && (misaligned(A_q) || misaligned(scale_A) || misaligned(B_q) ||
                   misaligned(scale_B))))
        return FGQ_ERR_ALIGN;
    const int64_t nc = 2 * M * N, nq = M * N, ns = 4 * M * (N / 128);
    const void* outs[3] = {C, C_q, scale_C};
    const int64_t nout[3] = {nc, nq, ns};
    for (int o = 0; o < 3; ++o) {
        for (int p = o + 1; p < 3; ++p)
            if (overlap(outs[o], nout[o], outs[p], nout[p]))
                return FGQ_ERR_ALIAS;
        if (K > 0 && (overlap(outs[o], nout[o], A_q, M * K) ||
                      overlap(outs[o], nout[o], B_q, K * N) ||
                      overlap(outs[o], nout[o], scale_A, 4 * M * (K / 128)) ||
                      overlap(outs[o], nout[o], scale_B, 4 * (K / 128) * (N / 128))))
            return FGQ_ERR_ALIAS;
    }
    return launch_status(fgq::launch_gemm_fp8_blockscaled_quant(
        A_q, scale_A, B_q, scale_B, C, C_q, scale_C, M, N, K, static_cast<hipStream_t>(stream)));
}

int fgq_quantize_nvfp4(const void* X, void* Xq, uint8_t* scale_X, float* global_scale,
                       int64_t R, int64_t C, void* stream)
{
    if (R < 0 || C < 0 || C % 16 != 0 || R > kMaxDim || C > kMaxDim)
        return FGQ_ERR_SHAPE;
    // one coding launch: R*C/8 work-items, counted in 32 bits
    if (R > 0 && C > 0 && R > ((int64_t(1) << 35) / C))
        return FGQ_ERR_SHAPE;
    if (R == 0 || C == 0)
        return FGQ_OK;
    if (!X || !Xq || !scale_X || !global_scale)
        return FGQ_ERR_NULL;
    if (misaligned(X) || misaligned(Xq) || misaligned(scale_X) || misaligned(global_scale))
        return FGQ_ERR_ALIGN;
    const void* p[4] = {X, Xq, scale_X, global_scale};
    const int64_t n[4] = {2 * R * C, R * C / 2, R * (C / 16), 4 * FGQ_NVFP4_GLOBAL_FLOATS};
    for (int a = 0; a < 4; ++a)
        for (int b = a + 1; b < 4; ++b)
            if (overlap(p[a], n[a], p[b], n[b]))
                return FGQ_ERR_ALIAS;
    return launch_status(fgq::launch_quant_nvfp4(X, Xq, scale_X, global_scale, R, C,
                                                 static_cast<hipStream_t>(stream)));
}

int fgq_gemm_nvfp4(const void* A_q, const uint8_t* scale_A, const float* global_A,
                   const void* B_q, const uint8_t* scale_B, const float* global_B, void* C,
                   int64_t M, int64_t N, int64_t K, int out_dtype, void* stream)
{
    if (out_dtype != FGQ_OUT_F32 && out_dtype != FGQ_OUT_BF16)
        return FGQ_ERR_DTYPE;
    if (M < 0 || N < 0 || K < 0 || K % 128 != 0 || N % 128 != 0 || M > kMaxDim ||
        N > kMaxDim || K > kMaxDim)
        return FGQ_ERR_SHAPE;
    if (((M + 127) / 128) * (N / 128) > kMaxDim)
        return FGQ_ERR_SHAPE;
    if (M == 0 || N == 0)
        return FGQ_OK;
    if (!C || !global_A || !global_B || (K > 0 && (!A_q || !scale_A || !B_q || !scale_B)))
        return FGQ_ERR_NULL;
    if (misaligned(C) || misaligned(global_A) || misaligned(global_B) ||
        (K > 0 && (misaligned(A_q) || misaligned(scale_A) || misaligned(B_q) ||
                   misaligned(scale_B))))
        return FGQ_ERR_ALIGN;
    const int64_t nc = M * N * (out_dtype == FGQ_OUT_BF16 ? 2 : 4);
    if (overlap(C, nc, global_A, 4) || overlap(C, nc, global_B, 4) ||
        (K > 0 && (overlap(C, nc, A_q, M * K / 2) || overlap(C, nc, B_q, N * K / 2) ||
                   overlap(C, nc, scale_A, M * (K / 16)) ||
                   overlap(C, nc, scale_B, N * (K / 16)))))
        return FGQ_ERR_ALIAS;
    return launch_status(fgq::launch_gemm_nvfp4(A_q, scale_A, global_A, B_q, scale_B, global_B,
                                                C, M, N, K, out_dtype == FGQ_OUT_BF16,
                                                static_cast<hipStream_t>(stream)));
}

}  // extern "C"
