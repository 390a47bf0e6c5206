// calib.hip -- measured ceilings for the roofline fractions (measurement only, not a step of
// the method).  Datasheet peaks are not reachable on a real box; these two kernels give what
// plain code of the same shape gets, next to which the quantizer and the GEMM are judged:
//
//   calib_stream: the activation quantizer's traffic with no arithmetic -- every lane reads
//     16 bytes and writes 8, non-temporal, two loads in flight per lane.  Page "Asynchronous
//     Data Copies (LDGSTS)", section on maximizing memory bandwidth: bandwidth is reached by
//     keeping enough bytes in flight, and a vanilla elementwise kernel is the reference.
//   calib_mfma_f16: only v_mfma_f32_16x16x32_f16, the instruction the GEMM's partials use, in
//     four independent accumulation chains per wave on register operands, two waves per SIMD.
//     Page "Instruction-Level Parallelism (ILP)": independent chains are what let a pipelined
//     unit reach its issue rate.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fgq_launch.hpp"

namespace fgq {

typedef unsigned u32x4c __attribute__((ext_vector_type(4)));
typedef unsigned u32x2c __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8c __attribute__((ext_vector_type(8)));
typedef float f32x4c __attribute__((ext_vector_type(4)));

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

hipError_t launch_calib_stream(const void* src, void* dst, int64_t n16, hipStream_t stream)
{
    const int64_t per = (int64_t)STREAM_THREADS * STREAM_UNROLL;
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

}  // namespace fgq
