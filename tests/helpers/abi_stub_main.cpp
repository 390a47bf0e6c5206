// Host-only check of the C ABI layers of libfgq (api.cpp) and libfgq_calib (calib_api.cpp) with the kernel launchers replaced by
// stubs: every entry point with valid arguments reaches its launcher exactly once and
// passes the launcher's status through (hipSuccess -> FGQ_OK, a launch failure ->
// FGQ_ERR_LAUNCH, a grid the dispatch cannot count -> FGQ_ERR_SHAPE); invalid arguments
// never reach a launcher.  Built with g++ and -fsanitize=address,undefined by
// tests/test_sanitize.py; no GPU, no HIP runtime library.  Prints "ok" and exits 0.
#include <cstdio>
#include <cstdlib>

#include "../../include/fgq.h"
#include "../../include/fgq_calib.h"
#include "../../fine_grained_block_fgq_amd/csrc/calib_launch.hpp"
#include "../../fine_grained_block_fgq_amd/csrc/fgq_launch.hpp"

namespace {
hipError_t g_status = hipSuccess;
int g_calls = 0;
hipError_t stub()
{
    ++g_calls;
    return g_status;
}
}  // namespace

namespace fgq {
hipError_t launch_quant_act_1x128(const void*, void*, float*, int64_t, int64_t, hipStream_t)
{
    return stub();
}
hipError_t launch_quant_weight_128x128(const void*, void*, float*, int64_t, int64_t, hipStream_t)
{
    return stub();
}
hipError_t launch_quant_act_1x128_ue8m0(const void*, void*, uint8_t*, int64_t, int64_t,
                                        hipStream_t)
{
    return stub();
}
hipError_t launch_quant_weight_128x128_ue8m0(const void*, void*, uint8_t*, int64_t, int64_t,
                                             hipStream_t)
{
    return stub();
}
hipError_t launch_gemm_fp8_blockscaled(const void*, const float*, const void*, const float*,
                                       void*, int64_t, int64_t, int64_t, int, int, hipStream_t)
{
    return stub();
}
hipError_t launch_gemm_fp8_blockscaled_ue8m0(const void*, const uint8_t*, const void*,
                                             const uint8_t*, void*, int64_t, int64_t, int64_t,
                                             int, int, hipStream_t)
{
    return stub();
}
hipError_t launch_gemm_fp8_blockscaled_quant(const void*, const float*, const void*, const float*,
                                             void*, void*, float*, int64_t, int64_t, int64_t,
                                             hipStream_t)
{
    return stub();
}
hipError_t launch_quant_nvfp4(const void*, void*, uint8_t*, float*, int64_t, int64_t, hipStream_t)
{
    return stub();
}
hipError_t launch_gemm_nvfp4(const void*, const uint8_t*, const float*, const void*,
                             const uint8_t*, const float*, void*, int64_t, int64_t, int64_t, int,
                             hipStream_t)
{
    return stub();
}
hipError_t launch_gemm_fp8_blockscaled_splitk(const void*, const float*, const void*,
                                              const float*, void*, int64_t, int64_t, int64_t, int,
                                              int, float*, hipStream_t)
{
    return stub();
}
hipError_t launch_gemm_fp8_blockscaled_noalloc(const void*, const float*, const void*,
                                               const float*, void*, int64_t, int64_t, int64_t,
                                               int, int, hipStream_t)
{
    return stub();
}
// the plan of the stubbed device: 4 splits for M <= 128, else none
int gemm_splitk_plan(int64_t M, int64_t, int64_t K) { return M <= 128 && K >= 2048 ? 4 : 1; }
hipError_t launch_calib_stream(const void*, void*, int64_t, hipStream_t) { return stub(); }
hipError_t launch_calib_mfma_f16(float*, int64_t, int64_t, hipStream_t) { return stub(); }
hipError_t launch_calib_mfma_fp8(float*, int64_t, int64_t, hipStream_t) { return stub(); }
hipError_t launch_probe_fp8_mfma_partials(const void*, const void*, float*, int64_t, int64_t,
                                          int64_t, hipStream_t)
{
    return stub();
}
}  // namespace fgq

namespace {
int failures = 0;

void expect(const char* what, int got, int want, int calls_want)
{
    if (got != want || g_calls != calls_want) {
        std::printf("FAIL %s: status %d (want %d), launcher calls %d (want %d)\n", what, got,
                    want, g_calls, calls_want);
        ++failures;
    }
    g_calls = 0;
}

// fake, 16-byte aligned, far-apart device addresses: never dereferenced by the host code
void* at(unsigned long long a) { return reinterpret_cast<void*>(a << 24); }
float* fat(unsigned long long a) { return static_cast<float*>(at(a)); }
uint8_t* uat(unsigned long long a) { return static_cast<uint8_t*>(at(a)); }

// every entry point once with valid arguments; the stub's status must come back mapped
void all_entry_points(int want)
{
    expect("quantize_act", fgq_quantize_act_1x128(at(1), at(2), fat(3), 4, 256, nullptr), want, 1);
    expect("quantize_act_ue8m0",
           fgq_quantize_act_1x128_ue8m0(at(1), at(2), uat(3), 4, 256, nullptr), want, 1);
    expect("quantize_weight", fgq_quantize_weight_128x128(at(1), at(2), fat(3), 256, 128, nullptr),
           want, 1);
    expect("quantize_weight_ue8m0",
           fgq_quantize_weight_128x128_ue8m0(at(1), at(2), uat(3), 256, 128, nullptr), want, 1);
    expect("gemm", fgq_gemm_fp8_blockscaled(at(1), fat(2), at(3), fat(4), at(5), 4, 128, 256,
                                            FGQ_OUT_BF16, nullptr),
           want, 1);
    for (int v = FGQ_GEMM_AUTO; v <= FGQ_GEMM_NARROW_64x64; ++v)
        expect("gemm_variant", fgq_gemm_fp8_blockscaled_variant(at(1), fat(2), at(3), fat(4),
                                                                at(5), 4, 128, 256, FGQ_OUT_F32,
                                                                v, nullptr),
               want, 1);
    expect("gemm_ue8m0", fgq_gemm_fp8_blockscaled_ue8m0(uat(1), uat(2), uat(3), uat(4), at(5), 4,
                                                        128, 256, FGQ_OUT_F32, 0, nullptr),
           want, 1);
    expect("gemm_quant", fgq_gemm_fp8_blockscaled_quant(at(1), fat(2), at(3), fat(4), at(5),
                                                        at(6), fat(7), 4, 128, 256, nullptr),
           want, 1);
    expect("quantize_nvfp4", fgq_quantize_nvfp4(at(1), at(2), uat(3), fat(4), 4, 64, nullptr),
           want, 1);
    expect("gemm_nvfp4", fgq_gemm_nvfp4(at(1), uat(2), fat(3), at(4), uat(5), fat(6), at(7), 4,
                                        128, 256, FGQ_OUT_F32, nullptr),
           want, 1);
    expect("gemm_ws", fgq_gemm_fp8_blockscaled_ws(at(1), fat(2), at(3), fat(4), at(5), 4, 128,
                                                  2048, FGQ_OUT_F32, at(6), 4 * 4 * 128 * 4,
                                                  nullptr),
           want, 1);
    expect("gemm_splitk", fgq_gemm_fp8_blockscaled_splitk(at(1), fat(2), at(3), fat(4), at(5),
                                                          4, 128, 256, FGQ_OUT_BF16, 2, at(6),
                                                          2 * 4 * 128 * 4, nullptr),
           want, 1);
    expect("gemm_noalloc", fgq_gemm_fp8_blockscaled_noalloc(at(1), fat(2), at(3), fat(4), at(5),
                                                            4, 128, 2048, FGQ_OUT_F32, nullptr),
           want, 1);
    expect("calib_stream", fgq_calib_stream(at(1), at(2), 100, nullptr), want, 1);
    expect("calib_mfma_f16", fgq_calib_mfma_f16(fat(1), 4, 10, nullptr), want, 1);
    expect("calib_mfma_fp8", fgq_calib_mfma_fp8(fat(1), 4, 10, nullptr), want, 1);
    expect("probe_fp8_mfma", fgq_probe_fp8_mfma_partials(at(1), at(2), fat(3), 16, 16, 128,
                                                         nullptr),
           want, 1);
}
}  // namespace

int main()
{
    g_status = hipSuccess;
    all_entry_points(FGQ_OK);
    g_status = hipErrorLaunchFailure;
    all_entry_points(FGQ_ERR_LAUNCH);
    g_status = hipErrorInvalidConfiguration;
    all_entry_points(FGQ_ERR_SHAPE);

    // invalid or empty calls never reach a launcher
    g_status = hipSuccess;
    expect("act K%128", fgq_quantize_act_1x128(at(1), at(2), fat(3), 4, 100, nullptr),
           FGQ_ERR_SHAPE, 0);
    expect("act null", fgq_quantize_act_1x128(nullptr, at(2), fat(3), 4, 128, nullptr),
           FGQ_ERR_NULL, 0);
    expect("act empty", fgq_quantize_act_1x128(nullptr, nullptr, nullptr, 0, 128, nullptr),
           FGQ_OK, 0);
    expect("weight alias", fgq_quantize_weight_128x128(at(1), at(1), fat(3), 128, 128, nullptr),
           FGQ_ERR_ALIAS, 0);
    expect("gemm dtype", fgq_gemm_fp8_blockscaled(at(1), fat(2), at(3), fat(4), at(5), 4, 128,
                                                  128, 7, nullptr),
           FGQ_ERR_DTYPE, 0);
    expect("gemm variant", fgq_gemm_fp8_blockscaled_variant(at(1), fat(2), at(3), fat(4), at(5),
                                                            4, 128, 128, 0, 99, nullptr),
           FGQ_ERR_VARIANT, 0);
    expect("gemm misaligned", fgq_gemm_fp8_blockscaled(static_cast<char*>(at(1)) + 4, fat(2),
                                                       at(3), fat(4), at(5), 4, 128, 128, 0,
                                                       nullptr),
           FGQ_ERR_ALIGN, 0);
    expect("gemm empty K", fgq_gemm_fp8_blockscaled(nullptr, nullptr, nullptr, nullptr, at(5), 4,
                                                    128, 0, 0, nullptr),
           FGQ_OK, 1);   // K == 0 still writes C = 0: the launcher runs
    expect("nvfp4 C%16", fgq_quantize_nvfp4(at(1), at(2), uat(3), fat(4), 4, 24, nullptr),
           FGQ_ERR_SHAPE, 0);
    expect("splitk small workspace",
           fgq_gemm_fp8_blockscaled_splitk(at(1), fat(2), at(3), fat(4), at(5), 4, 128, 256,
                                           FGQ_OUT_F32, 2, at(6), 2 * 4 * 128 * 4 - 1, nullptr),
           FGQ_ERR_WORKSPACE, 0);
    expect("splitk no workspace",
           fgq_gemm_fp8_blockscaled_splitk(at(1), fat(2), at(3), fat(4), at(5), 4, 128, 256,
                                           FGQ_OUT_F32, 2, nullptr, 0, nullptr),
           FGQ_ERR_WORKSPACE, 0);
    expect("splitk splits > K/128",
           fgq_gemm_fp8_blockscaled_splitk(at(1), fat(2), at(3), fat(4), at(5), 4, 128, 256,
                                           FGQ_OUT_F32, 3, at(6), 1 << 20, nullptr),
           FGQ_ERR_SHAPE, 0);
    expect("splitk workspace alias",
           fgq_gemm_fp8_blockscaled_splitk(at(1), fat(2), at(3), fat(4), at(5), 4, 128, 256,
                                           FGQ_OUT_F32, 2, at(5), 1 << 20, nullptr),
           FGQ_ERR_ALIAS, 0);
    // the workspace path: too small a workspace falls back to the unsplit launch
    expect("ws fallback", fgq_gemm_fp8_blockscaled_ws(at(1), fat(2), at(3), fat(4), at(5), 4,
                                                      128, 2048, FGQ_OUT_F32, at(6), 16,
                                                      nullptr),
           FGQ_OK, 1);
    if (fgq_gemm_workspace_size(4, 128, 2048) != 4 * 4 * 128 * 4 ||
        fgq_gemm_workspace_size(256, 128, 2048) != 0 ||
        fgq_gemm_workspace_size(4, 100, 2048) != FGQ_ERR_SHAPE) {
        std::printf("FAIL workspace size\n");
        ++failures;
    }
    // the no-allocation GEMM refuses a planned split beyond its 16 MiB array
    expect("noalloc too large", fgq_gemm_fp8_blockscaled_noalloc(at(1), fat(2), at(3), fat(4),
                                                                 at(5), 128, 16384, 2048,
                                                                 FGQ_OUT_F32, nullptr),
           FGQ_ERR_WORKSPACE, 0);
    for (int s = 0; s >= -8; --s)
        if (!fgq_status_string(s) || !fgq_status_string(s)[0]) {
            std::printf("FAIL status string %d\n", s);
            ++failures;
        }
    if (failures) {
        std::printf("%d failures\n", failures);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
