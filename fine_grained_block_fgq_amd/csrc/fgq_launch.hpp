// fgq_launch.hpp -- host-side launchers of the gfx950 kernels (internal to libfgq).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgq {

// A HIP dispatch counts the work-items of each grid dimension in 32 bits; a launch that would
// exceed that is refused with hipErrorInvalidConfiguration before anything is enqueued (the
// C ABI reports it as a shape error).
constexpr int64_t kMaxWorkItems = 0xFFFFFFFFll;
inline bool grid_fits(int64_t blocks, int64_t threads)
{
    return blocks >= 0 && blocks <= kMaxWorkItems / threads;
}

// compute units of the current device (0 if the query fails); cached per device
int device_cus();

hipError_t launch_quant_act_1x128(const void* X, void* Xq, float* sX, int64_t M, int64_t K,
                                  hipStream_t stream);
hipError_t launch_quant_weight_128x128(const void* W, void* Wq, float* sW, int64_t K,
                                       int64_t N, hipStream_t stream);
// the same with UE8M0 (exponent byte) scales
hipError_t launch_quant_act_1x128_ue8m0(const void* X, void* Xq, uint8_t* sX, int64_t M,
                                        int64_t K, hipStream_t stream);
hipError_t launch_quant_weight_128x128_ue8m0(const void* W, void* Wq, uint8_t* sW, int64_t K,
                                             int64_t N, hipStream_t stream);
// GEMM kernel families (values of fgq_gemm_variant)
enum GemmVariant {
    GEMM_AUTO = 0,
    GEMM_WIDE_256x128 = 1,
    GEMM_WIDE_128x128 = 2,
    GEMM_NARROW = 3,
    GEMM_SKINNY = 4,
    GEMM_NARROW_64x64 = 5
};

// out_bf16: 0 -> C is fp32, 1 -> C is bf16 (nearest-even)
hipError_t launch_gemm_fp8_blockscaled(const void* A_q, const float* sA, const void* B_q,
                                       const float* sB, void* C, int64_t M, int64_t N,
                                       int64_t K, int out_bf16, int variant,
                                       hipStream_t stream);

// the same GEMM with UE8M0 exponent-byte scales (2^(e-127))
hipError_t launch_gemm_fp8_blockscaled_ue8m0(const void* A_q, const uint8_t* sA,
                                             const void* B_q, const uint8_t* sB, void* C,
                                             int64_t M, int64_t N, int64_t K, int out_bf16,
                                             int variant, hipStream_t stream);

// K split across workgroups with fp32 partials in a caller's workspace of
// splits * M * N floats (splits <= 1: the automatic no-workspace choice); the number of
// splits the workspace path uses for a shape on the current device (1 = none)
constexpr int kSplitMax = 16;
int gemm_splitk_plan(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_fp8_blockscaled_splitk(const void* A_q, const float* sA, const void* B_q,
                                              const float* sB, void* C, int64_t M, int64_t N,
                                              int64_t K, int out_bf16, int splits, float* ws,
                                              hipStream_t stream);

// the same K-split GEMM with its partials in a static per-device array of
// kNoallocScratchBytes (no workspace argument, no allocation); splits * M * N * 4 beyond that
// size is refused (hipErrorInvalidValue), a failed lookup of the array gives
// hipErrorInvalidSymbol
constexpr int64_t kNoallocScratchBytes = int64_t(16) << 20;
hipError_t launch_gemm_fp8_blockscaled_noalloc(const void* A_q, const float* sA, const void* B_q,
                                               const float* sB, void* C, int64_t M, int64_t N,
                                               int64_t K, int out_bf16, int splits,
                                               hipStream_t stream);

// C = bf16 GEMM result, plus its 1x128 E4M3 quantization (Cq [M,N], sC [M,N/128])
hipError_t launch_gemm_fp8_blockscaled_quant(const void* A_q, const float* sA, const void* B_q,
                                             const float* sB, void* C, void* Cq, float* sC,
                                             int64_t M, int64_t N, int64_t K,
                                             hipStream_t stream);

// NVFP4: quantize X [R,C] (blocks of 16 along C) to packed E2M1 codes [R,C/2], E4M3 block
// scales [R,C/16] and the fp32 global scale g[0] (g: kNvfp4GlobalFloats floats, the rest
// scratch of the call); GEMM of A [M,K] and B stored [N,K]
constexpr int kNvfp4GlobalFloats = 512;
hipError_t launch_quant_nvfp4(const void* X, void* Xq, uint8_t* sX, float* g, int64_t R,
                              int64_t C, hipStream_t stream);
hipError_t launch_gemm_nvfp4(const void* A_q, const uint8_t* sA, const float* gA,
                             const void* B_q, const uint8_t* sB, const float* gB, void* C,
                             int64_t M, int64_t N, int64_t K, int out_bf16, hipStream_t stream);

}  // namespace fgq
