// quant.hip -- E4M3 quantization kernels for gfx950.
//
//   quant_act_1x128:    page "Fine-Grained FP8/FP4 Quantization", section "Scaling
//                       Granularities" (per-tile 1x128 activation scaling) and section
//                       "DeepGEMM: Tile-wise and Block-wise Scaling" (scale_A [M, K/128]).
//   quant_weight_128x128: same page and sections (per-block 128x128 weight scaling,
//                       scale_B [K/128, N/128]).
//
// Both are HBM-bound streams (2 bytes in, 1 byte out per element).  Loads are 16-byte
// global loads straight into registers (no LDS staging: nothing is reused), each lane keeps
// several loads in flight, and the group amax is an integer max reduced with DPP.
#include "fgq_device.hpp"
#include "fgq_launch.hpp"

namespace fgq {

// ---------------------------------------------------------------------------------------
// 1x128 activation tiles.  With K % 128 == 0 the tiles of a row-major [M,K] matrix are
// consecutive 256-byte runs, tile t = flat elements [128t, 128t+128), and its scale is
// scale_X[t] (= scale_X[m*(K/128)+kb]).  A 16-lane DPP row owns one tile: lane j holds
// bytes [16j, 16j+16) of it (8 bf16 -> 8 codes).  A wave covers 4 consecutive tiles per
// load (1 KB, fully coalesced) and issues ACT_UNROLL such loads before using any of them.
// ---------------------------------------------------------------------------------------
#ifndef FGQ_ACT_UNROLL
#define FGQ_ACT_UNROLL 2
#endif
#ifndef FGQ_ACT_WAVES
#define FGQ_ACT_WAVES 4
#endif
constexpr int ACT_UNROLL = FGQ_ACT_UNROLL;
constexpr int ACT_WAVES = FGQ_ACT_WAVES;
constexpr int ACT_TILES_PER_WAVE = 4 * ACT_UNROLL;
constexpr int ACT_TILES_PER_BLOCK = ACT_WAVES * ACT_TILES_PER_WAVE;

#ifndef FGQ_ACT_GRID
#define FGQ_ACT_GRID 0
#endif
// workgroups launched (0: one per ACT_TILES_PER_BLOCK tiles; else at most this many, each
// looping over the tile groups with a grid stride)
constexpr int64_t ACT_GRID = FGQ_ACT_GRID;

template <class Scale>
__global__ __launch_bounds__(64 * ACT_WAVES) void quant_act_1x128_kernel(
    const u32x4* __restrict__ X, u32x2* __restrict__ Xq, typename Scale::stored_t* __restrict__ sX,
    int64_t T)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane >> 4;
    const int j = lane & 15;
    const int64_t nblocks = (T + ACT_TILES_PER_BLOCK - 1) / ACT_TILES_PER_BLOCK;
    for (int64_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
    const int64_t t0 = (blk * ACT_WAVES + wave) * ACT_TILES_PER_WAVE + sub;

    u32x4 v[ACT_UNROLL];
#pragma unroll
    for (int u = 0; u < ACT_UNROLL; ++u) {
        const int64_t t = t0 + 4 * u;
        v[u] = (t < T) ? __builtin_nontemporal_load(&X[t * 16 + j]) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < ACT_UNROLL; ++u) {
        const int64_t t = t0 + 4 * u;
        const Scale g(row16_max(absmax_bits8(v[u])));
        const u32x2 q = g.quant(v[u]);
        if (t < T) {
            __builtin_nontemporal_store(q, &Xq[t * 16 + j]);
            if (j == 0)
                sX[t] = g.stored();
        }
    }
    }
}

// ---------------------------------------------------------------------------------------
// 128x128 weight blocks.  One 512-thread workgroup per block: the block is 128 rows of 256
// bytes = 2048 16-byte chunks, 4 per thread, all loaded before the reduction (32 KB in
// flight per workgroup).  Chunk c = i*512 + tid covers row c/16, columns 8*(c%16)..+7, so
// each load instruction of a wave reads 4 whole 256-byte row segments.  amax: per-thread
// max, DPP + readlane across the wave, LDS across the 8 waves.  Loads are non-temporal, the
// code stores ordinary.  (Timed on [16384,7168]: 128/256/512/1024 threads 65.3/61.9/60.8/62.5
// us per launch with non-temporal stores, 57.3 us with ordinary stores; ordinary loads 66.4,
// workgroups ordered down the K blocks first 69.2.)
// ---------------------------------------------------------------------------------------
constexpr int WQ_THREADS = 512;
constexpr int WQ_CHUNKS = 2048 / WQ_THREADS;
constexpr int WQ_WAVES = WQ_THREADS / 64;

template <class Scale>
__global__ __launch_bounds__(WQ_THREADS) void quant_weight_128x128_kernel(
    const uint8_t* __restrict__ W, uint8_t* __restrict__ Wq,
    typename Scale::stored_t* __restrict__ sW, int64_t N)
{
    __shared__ uint32_t wave_amax[WQ_WAVES];
    const int tid = threadIdx.x;
    const int64_t nb = blockIdx.x, kb = blockIdx.y;
    const int64_t NB = N / 128;
    const uint8_t* wblk = W + (kb * 128 * N + nb * 128) * 2;
    uint8_t* qblk = Wq + kb * 128 * N + nb * 128;

    u32x4 v[WQ_CHUNKS];
#pragma unroll
    for (int i = 0; i < WQ_CHUNKS; ++i) {
        const int c = i * WQ_THREADS + tid;
        const int row = c >> 4, col8 = (c & 15) * 8;
        v[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(wblk + ((int64_t)row * N + col8) * 2));
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < WQ_CHUNKS; ++i)
        m = max(m, absmax_bits8(v[i]));
    m = wave_max(m);
    if ((tid & 63) == 0)
        wave_amax[tid >> 6] = m;
    __syncthreads();
    m = wave_amax[0];
#pragma unroll
    for (int w = 1; w < WQ_WAVES; ++w)
        m = max(m, wave_amax[w]);
    const Scale g(m);
#pragma unroll
    for (int i = 0; i < WQ_CHUNKS; ++i) {
        const int c = i * WQ_THREADS + tid;
        const int row = c >> 4, col8 = (c & 15) * 8;
        // ordinary stores, measured faster than non-temporal ones here (likely because a row's
        // 128-byte code segment is combined in L2 with the adjacent column blocks' segments
        // before it is written to HBM)
        *reinterpret_cast<u32x2*>(qblk + (int64_t)row * N + col8) = g.quant(v[i]);
    }
    if (tid == 0)
        sW[kb * NB + nb] = g.stored();
}

template <class Scale>
static hipError_t launch_act(const void* X, void* Xq, typename Scale::stored_t* sX, int64_t M,
                             int64_t K, hipStream_t stream)
{
    const int64_t T = M * (K / 128);
    int64_t blocks = (T + ACT_TILES_PER_BLOCK - 1) / ACT_TILES_PER_BLOCK;
    if (ACT_GRID > 0 && blocks > ACT_GRID)
        blocks = ACT_GRID;
    if (!grid_fits(blocks, 64 * ACT_WAVES))
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(quant_act_1x128_kernel<Scale>, dim3((unsigned)blocks),
                       dim3(64 * ACT_WAVES), 0, stream, static_cast<const u32x4*>(X),
                       static_cast<u32x2*>(Xq), sX, T);
    return hipGetLastError();
}

template <class Scale>
static hipError_t launch_weight(const void* W, void* Wq, typename Scale::stored_t* sW,
                                int64_t K, int64_t N, hipStream_t stream)
{
    if (!grid_fits(N / 128, WQ_THREADS))
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(quant_weight_128x128_kernel<Scale>,
                       dim3((unsigned)(N / 128), (unsigned)(K / 128)), dim3(WQ_THREADS), 0,
                       stream, static_cast<const uint8_t*>(W), static_cast<uint8_t*>(Wq), sW,
                       N);
    return hipGetLastError();
}

hipError_t launch_quant_act_1x128(const void* X, void* Xq, float* sX, int64_t M, int64_t K,
                                  hipStream_t stream)
{
    return launch_act<ScaleF32>(X, Xq, sX, M, K, stream);
}

hipError_t launch_quant_weight_128x128(const void* W, void* Wq, float* sW, int64_t K,
                                       int64_t N, hipStream_t stream)
{
    return launch_weight<ScaleF32>(W, Wq, sW, K, N, stream);
}

hipError_t launch_quant_act_1x128_ue8m0(const void* X, void* Xq, uint8_t* sX, int64_t M,
                                        int64_t K, hipStream_t stream)
{
    return launch_act<ScaleUE8M0>(X, Xq, sX, M, K, stream);
}

hipError_t launch_quant_weight_128x128_ue8m0(const void* W, void* Wq, uint8_t* sW, int64_t K,
                                             int64_t N, hipStream_t stream)
{
    return launch_weight<ScaleUE8M0>(W, Wq, sW, K, N, stream);
}

}  // namespace fgq
