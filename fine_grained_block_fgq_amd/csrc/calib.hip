// calib.hip -- kernels of libfgq_calib, the measurement library (not a step of the method).
// Datasheet peaks are not reachable on a real box; these kernels give what plain code of the
// same shape gets, next to which the quantizer and the GEMM are judged, and measure the FP8
// matrix cores' own accuracy:
//
//   calib_stream: the activation quantizer's traffic with no arithmetic -- every lane reads
//     16 bytes and writes 8, non-temporal, two loads in flight per lane.
//   calib_mfma_f16: only v_mfma_f32_16x16x32_f16, the instruction the GEMM's partials use, in
//     four independent accumulation chains per wave on register operands, two waves per SIMD,
//     so that the matrix cores run at their issue rate.
//   calib_mfma_fp8: the same with v_mfma_f32_16x16x128_f8f6f4 on E4M3 operands: what the FP8
//     matrix cores reach on this GPU.
//   probe_fp8_mfma_partials: the 128-K chunk partials sum_k A_q[m,k] * B_q[k,n] formed by one
//     v_mfma_f32_16x16x128_f8f6f4 per 16x16 tile and chunk, written out unscaled, so that their
//     error against the exact sums can be measured.  The method promotes every 128-K partial
//     to fp32 because FP8 tensor-core sums are kept at reduced precision (page "Fine-Grained
//     FP8/FP4 Quantization", section "Hopper: CUDA Core Promotion (Nc=128)"); on gfx950 the
//     reduced precision is inside each FP8 instruction, so the GEMM forms its partials with
//     f16 MFMAs instead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "calib_launch.hpp"

namespace fgq {

typedef unsigned u32x4c __attribute__((ext_vector_type(4)));
typedef unsigned u32x2c __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8c __attribute__((ext_vector_type(8)));
typedef float f32x4c __attribute__((ext_vector_type(4)));
typedef int i32x8c __attribute__((ext_vector_type(8)));

constexpr int STREAM_THREADS = 256;
constexpr int STREAM_UNROLL = 2;

__global__ __launch_bounds__(STREAM_THREADS) void calib_stream_kernel(
    const u32x4c* __restrict__ src, u32x2c* __restrict__ dst, int64_t n16)
{
    const int64_t base = (int64_t)blockIdx.x * STREAM_THREADS * STREAM_UNROLL + threadIdx.x;
    u32x4c v[STREAM_UNROLL];
#pragma unroll
    for (int u = 0; u < STREAM_UNROLL; ++u) {
        const int64_t i = base + u * STREAM_THREADS;
        v[u] = i < n16 ? __builtin_nontemporal_load(&src[i]) : u32x4c{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < STREAM_UNROLL; ++u) {
        const int64_t i = base + u * STREAM_THREADS;
        if (i < n16)
            __builtin_nontemporal_store(u32x2c{v[u].x ^ v[u].y, v[u].z ^ v[u].w}, &dst[i]);
    }
}

constexpr int MFMA_THREADS = 512;   // 8 waves: two per SIMD

__global__ __launch_bounds__(MFMA_THREADS) void calib_mfma_f16_kernel(float* __restrict__ out,
                                                                      int64_t iters)
{
    const int lane = threadIdx.x & 63;
    f16x8c a[4], b[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[t][e] = (_Float16)(0.001f * (float)(lane + e + t));
            b[t][e] = (_Float16)(0.002f * (float)(e - t));
        }
    f32x4c acc[4] = {};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], b[(t + c) & 3], acc[c], 0,
                                                                0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
        s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[(int64_t)blockIdx.x * MFMA_THREADS + threadIdx.x] = s;
}

__global__ __launch_bounds__(MFMA_THREADS) void calib_mfma_fp8_kernel(float* __restrict__ out,
                                                                      int64_t iters)
{
    const int lane = threadIdx.x & 63;
    // E4M3 bytes of small finite values (exponent field 1..6, any sign)
    i32x8c a[4], b[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[t][e] = (int)(0x0c0b0a09u + 0x01010101u * (unsigned)((lane + e + t) & 7));
            b[t][e] = (int)(0x8a0b8c0du + 0x01000100u * (unsigned)((e + 3 * t) & 15));
        }
    f32x4c acc[4] = {};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                // zero scale operands select the unscaled v_mfma_f32_16x16x128_f8f6f4;
                // format 0 on both sides = FP8 E4M3
                acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    a[t], b[(t + c) & 3], acc[c], 0, 0, 0, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
        s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[(int64_t)blockIdx.x * MFMA_THREADS + threadIdx.x] = s;
}

// One wave per (16x16 tile, 128-K chunk).  Lane (g = lane/16, q = lane%16) holds A_q row q,
// k = 32g..32g+31 (byte e = k - 32g) and B_q column q over the same k; the instruction leaves
// rows 4g..4g+3 of column q.  P is [K/128][M][N].
constexpr int PROBE_THREADS = 256;

__global__ __launch_bounds__(PROBE_THREADS) void probe_fp8_mfma_partials_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, float* __restrict__ P,
    int64_t M, int64_t N, int64_t K)
{
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * (PROBE_THREADS / 64) + (threadIdx.x >> 6);
    const int64_t tm = M / 16, tn = N / 16;
    if (w >= tm * tn * (K / 128))
        return;
    const int64_t kb = w / (tm * tn), m0 = (w % (tm * tn)) / tn * 16, n0 = w % tn * 16;
    const int g = lane >> 4, q = lane & 15;
    const int64_t k0 = kb * 128 + 32 * g;
    const u32x4c* arow = reinterpret_cast<const u32x4c*>(A + (m0 + q) * K + k0);
    const u32x4c a0 = arow[0], a1 = arow[1];
    i32x8c av, bv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        av[e] = (int)a0[e];
        av[4 + e] = (int)a1[e];
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        unsigned word = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            word |= (unsigned)B[(k0 + 4 * d + e) * N + n0 + q] << (8 * e);
        bv[d] = (int)word;
    }
    const f32x4c p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        av, bv, f32x4c{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r)
        P[(kb * M + m0 + 4 * g + r) * N + n0 + q] = p[r];
}

hipError_t launch_calib_stream(const void* src, void* dst, int64_t n16, hipStream_t stream)
{
    const int64_t per = (int64_t)STREAM_THREADS * STREAM_UNROLL;
    if (!grid_fits((n16 + per - 1) / per, STREAM_THREADS))
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(calib_stream_kernel, dim3((unsigned)((n16 + per - 1) / per)),
                       dim3(STREAM_THREADS), 0, stream, static_cast<const u32x4c*>(src),
                       static_cast<u32x2c*>(dst), n16);
    return hipGetLastError();
}

hipError_t launch_calib_mfma_f16(float* out, int64_t blocks, int64_t iters, hipStream_t stream)
{
    hipLaunchKernelGGL(calib_mfma_f16_kernel, dim3((unsigned)blocks), dim3(MFMA_THREADS), 0,
                       stream, out, iters);
    return hipGetLastError();
}

hipError_t launch_calib_mfma_fp8(float* out, int64_t blocks, int64_t iters, hipStream_t stream)
{
    hipLaunchKernelGGL(calib_mfma_fp8_kernel, dim3((unsigned)blocks), dim3(MFMA_THREADS), 0,
                       stream, out, iters);
    return hipGetLastError();
}

hipError_t launch_probe_fp8_mfma_partials(const void* A_q, const void* B_q, float* P, int64_t M,
                                          int64_t N, int64_t K, hipStream_t stream)
{
    const int64_t waves = (M / 16) * (N / 16) * (K / 128);
    const int64_t per = PROBE_THREADS / 64;
    if (!grid_fits((waves + per - 1) / per, PROBE_THREADS))
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(probe_fp8_mfma_partials_kernel, dim3((unsigned)((waves + per - 1) / per)),
                       dim3(PROBE_THREADS), 0, stream, static_cast<const uint8_t*>(A_q),
                       static_cast<const uint8_t*>(B_q), P, M, N, K);
    return hipGetLastError();
}

}  // namespace fgq
