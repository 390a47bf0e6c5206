// nvfp4.hip -- NVFP4 (two-level scaled E2M1) quantization and GEMM for gfx950.
//
// Page "Fine-Grained FP8/FP4 Quantization", section "NVFP4 Two-Level Scaling": E2M1 codes
// (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), one E4M3 block scale per 16 consecutive elements
// along K, one FP32 global scale per tensor; value = global * block * e2m1.  Scales are
// chosen as g = amax/2688 (the largest block scale 448 times the largest code 6), block =
// E4M3(amax_block / (6g)), code = E2M1(x / (block * g)) nearest-even, saturating at 6.
// Both GEMM operands are row-major [rows, K] with K contiguous (the weight is stored as its
// [N, K] transpose, so its blocks of 16 are contiguous too); two codes per byte, element 2i
// in the low nibble.
#include "fgq_device.hpp"
#include "fgq_launch.hpp"
#include "gemm_common.hpp"

namespace fgq {

// ---------------------------------------------------------------------------------------
// Quantizer.  The global scale needs the tensor amax before any block can be coded, so a
// call is two launches on one stream.  The caller's global-scale argument is an array of
// kNvfp4GlobalFloats floats: the amax pass writes one candidate per workgroup into
// g[2 .. 2+blocks) (fl32(amax_w/2688) of its share; a correctly rounded divide is monotonic,
// so the largest candidate is the global scale of the tensor amax), with no atomics; every
// wave of the coding pass reduces the candidates itself (non-negative fp32 values order like
// their bit patterns), and the first workgroup writes g[0].  Nothing reads g[0] during the
// call and nothing writes the candidates in the coding pass, so the two passes share the
// array without a race.
// ---------------------------------------------------------------------------------------
// up to 256 candidates, at g[4 .. 259] (16-byte aligned): every coding wave reads them with
// one 16-byte load per lane and reduces them itself
constexpr int NVFP4_AMAX_BLOCKS = 256;
constexpr int NVFP4_CAND_OFF = 4;
static_assert(NVFP4_CAND_OFF + NVFP4_AMAX_BLOCKS <= kNvfp4GlobalFloats, "candidate slots");
constexpr int NVFP4_AMAX_VPT = 16;
constexpr int NVFP4_AMAX_THREADS = 512;   // 8 waves (1024: 82 -> 85 us at 16384x7168)
constexpr int NVFP4_AMAX_WAVES = NVFP4_AMAX_THREADS / 64;

// grid-stride max with four loads in flight per lane, reduced over the workgroup in LDS,
// written as this workgroup's candidate.  Ordinary (temporal) loads, so that X stays in the
// Infinity Cache for the coding pass where it fits (4096x4096: 15.3 -> 14.6 us per call;
// the coding pass's own loads, the last use of X, are non-temporal)
#define AMAX_LOAD(p) (*(p))
__global__ __launch_bounds__(NVFP4_AMAX_THREADS) void nvfp4_amax_kernel(
    const u32x4* __restrict__ X, int64_t nvec, uint32_t* __restrict__ cand)
{
    __shared__ uint32_t wave_amax[NVFP4_AMAX_WAVES];
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * NVFP4_AMAX_THREADS;
    int64_t i = (int64_t)blockIdx.x * NVFP4_AMAX_THREADS + threadIdx.x;
    for (; i + 3 * stride < nvec; i += 4 * stride) {
        const u32x4 a = AMAX_LOAD(&X[i]);
        const u32x4 b = AMAX_LOAD(&X[i + stride]);
        const u32x4 c = AMAX_LOAD(&X[i + 2 * stride]);
        const u32x4 d = AMAX_LOAD(&X[i + 3 * stride]);
        m = max(max(m, max(absmax_bits8(a), absmax_bits8(b))),
                max(absmax_bits8(c), absmax_bits8(d)));
    }
    for (; i < nvec; i += stride)
        m = max(m, absmax_bits8(AMAX_LOAD(&X[i])));
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0)
        wave_amax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t b = 0;
#pragma unroll
        for (int w = 0; w < NVFP4_AMAX_WAVES; ++w)
            b = max(b, wave_amax[w]);
        cand[blockIdx.x] = __float_as_uint(__uint_as_float(b << 16) / 2688.0f);
    }
}

// E2M1 code of y: count the rounding boundaries passed (ties at 0.25, 1.25, 2.5, 5 go down
// to the even code, ties at 0.75, 1.75, 3.5 go up to it), saturating at 6; sign in bit 3
__device__ __forceinline__ uint32_t e2m1_code(float y)
{
    const float a = __builtin_fabsf(y);
    const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
    return c | ((__float_as_uint(y) >> 28) & 8u);
}

// one lane = 8 consecutive elements (16 bytes) -> 8 codes (4 bytes); a block of 16 is the
// lane pair (2b, 2b+1), whose amax is exchanged by a DPP quad permute [1,0,3,2]
constexpr int NVFP4_QV = 2;   // two vectors per lane: 7-9% faster than one, and than four

// the 8 codes of one vector (packed nibbles) and its lane pair's E4M3 block scale
__device__ __forceinline__ uint32_t nvfp4_code8(u32x4 v, float g, float six_g, uint32_t& sb_out)
{
    uint32_t am = absmax_bits8(v);
    am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0xB1, 0xF, 0xF, false));
    uint32_t sb = 0;
    if (six_g != 0.0f)
        sb = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(am << 16) / six_g, 0.0f,
                                                      0, false) &
             0xFFu;
    const float D = __builtin_amdgcn_cvt_f32_fp8((int)sb, 0) * g;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t packed = 0;
    if (D >= 0x1p-100f && D <= 0x1p100f) {
        // y = fl32(x / D) without a divide per element: r = 1/D correctly rounded (one IEEE
        // divide per lane), q = x*r, then Markstein's correction with the exact remainder
        // x - q*D gives the correctly rounded quotient (Markstein's theorem: r within half an
        // ulp of 1/D and q within one ulp of x/D; with the range guard, r and q stay normal
        // and the remainder is exact wherever x/D is near an E2M1 rounding boundary, since
        // the block scale keeps |x| < 9*D).  The E2M1 code is
        // then the hardware convert at unit scale, which applies exactly the nearest-even,
        // saturating rule (checked against it on every finite fp32 input).
        const float r = 1.0f / D;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t xb = (e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16);
            const float x = __uint_as_float(xb);
            const float q = x * r;
            // negated remainder q*D - x, so that x = -0 keeps its sign: y = -0
            y[e] = __builtin_fmaf(-__builtin_fmaf(q, D, -x), r, q);
        }
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[0], y[1], 1.0f, 0);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[2], y[3], 1.0f, 1);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[4], y[5], 1.0f, 2);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[6], y[7], 1.0f, 3);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t b = (e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16);
            const uint32_t c = D == 0.0f ? ((b >> 28) & 8u) : e2m1_code(__uint_as_float(b) / D);
            packed |= c << (4 * e);
        }
    }
    sb_out = sb;
    return packed;
}

// the global scale: the largest of the amax pass's candidates (at most 256, four per lane),
// for every wave by itself; the first workgroup's first lane writes it to gs[0]
__device__ __forceinline__ float nvfp4_global(uint32_t* __restrict__ gs, int ncand)
{
    const int l = (int)(threadIdx.x & 63);
    const uint32_t* cand = gs + NVFP4_CAND_OFF;
    u32x4 c = u32x4{0u, 0u, 0u, 0u};
    if (4 * l + 3 < ncand) {
        c = *(const u32x4*)(cand + 4 * l);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * l + e < ncand)
                c[e] = cand[4 * l + e];
    }
    const uint32_t gb = wave_max(max(max(c.x, c.y), max(c.z, c.w)));
    if (blockIdx.x == 0 && threadIdx.x == 0)
        gs[0] = gb;
    return __uint_as_float(gb);
}

// coding pass: one workgroup per 256*NVFP4_QV vectors, the vectors requested before the global
// scale is reduced; codes stored non-temporally (3-5% faster than ordinary stores; the block
// scale bytes gain nothing from it)
__global__ __launch_bounds__(256) void nvfp4_quant_kernel(const u32x4* __restrict__ X,
                                                          uint32_t* __restrict__ Xq,
                                                          uint8_t* __restrict__ sX,
                                                          uint32_t* __restrict__ gs,
                                                          int ncand, int64_t nvec)
{
    const int64_t wg = blockIdx.x;
    u32x4 v[NVFP4_QV];
#pragma unroll
    for (int u = 0; u < NVFP4_QV; ++u) {
        const int64_t i = wg * (256 * NVFP4_QV) + u * 256 + threadIdx.x;
        v[u] = i < nvec ? __builtin_nontemporal_load(&X[i]) : u32x4{0u, 0u, 0u, 0u};
    }
    const float g = nvfp4_global(gs, ncand);
    const float six_g = 6.0f * g;
#pragma unroll
    for (int u = 0; u < NVFP4_QV; ++u) {
        const int64_t i = wg * (256 * NVFP4_QV) + u * 256 + threadIdx.x;
        uint32_t sb;
        const uint32_t packed = nvfp4_code8(v[u], g, six_g, sb);
        if (i < nvec) {
            __builtin_nontemporal_store(packed, &Xq[i]);
            if ((threadIdx.x & 1) == 0)
                sX[i >> 1] = (uint8_t)sb;
        }
    }
}

hipError_t launch_quant_nvfp4(const void* X, void* Xq, uint8_t* sX, float* g, int64_t R,
                              int64_t C, hipStream_t stream)
{
    uint32_t* const gs = reinterpret_cast<uint32_t*>(g);
    const int64_t nvec = R * C / 8;
    if (!grid_fits((nvec + 255) / 256, 256))
        return hipErrorInvalidConfiguration;
    int64_t ablocks = (nvec + NVFP4_AMAX_THREADS * NVFP4_AMAX_VPT - 1) /
                      (NVFP4_AMAX_THREADS * NVFP4_AMAX_VPT);
    ablocks = ablocks < 1 ? 1 : (ablocks > NVFP4_AMAX_BLOCKS ? NVFP4_AMAX_BLOCKS : ablocks);
    hipLaunchKernelGGL(nvfp4_amax_kernel, dim3((unsigned)ablocks), dim3(NVFP4_AMAX_THREADS), 0,
                       stream, static_cast<const u32x4*>(X), nvec, gs + NVFP4_CAND_OFF);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t qblocks = (nvec + 256 * NVFP4_QV - 1) / (256 * NVFP4_QV);
    hipLaunchKernelGGL(nvfp4_quant_kernel, dim3((unsigned)qblocks), dim3(256), 0, stream,
                       static_cast<const u32x4*>(X), static_cast<uint32_t*>(Xq), sX, gs,
                       (int)ablocks, nvec);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// GEMM.  C[m,n] = gA*gB * sum_k (e2m1(a[m,k]) * sA[m,k/16]) * (e2m1(b[n,k]) * sB[n,k/16]).
// Every product e2m1 * E4M3 has at most 6 significant bits and lies in [2^-10, 2688], so the
// scaled operand is an exact f16; f16 MFMAs sum the products to fp32 accuracy and accumulate
// straight into the fp32 accumulators over all of K (the block scales are inside the
// operands, so no per-chunk promotion step is needed); the two global scales multiply the
// result once.  Operands: v_cvt_scalef32_pk_f16_fp4 with a unit scale (its scale operand is
// applied as a power of two only, measured) then v_pk_mul_f16 by the block scale.  Both
// operands are K-contiguous, so every fragment is a plain 16-byte LDS read: lane (q, g)
// takes 32 consecutive k (bytes 16g..16g+15 of the row's 64-byte chunk), blocks 2g and
// 2g+1.  The 16-byte chunk of a row is XORed with (row/4)%4 so the 16 rows of a fragment
// read hit distinct banks.
// ---------------------------------------------------------------------------------------
template <int BM_, int BN_, int WM_, int WN_>
struct Nvfp4Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int NW = WM * WN, NT = 64 * NW;
    static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
    static constexpr int A_BYTES = BM * 64, B_BYTES = BN * 64;
    static constexpr int SA_BYTES = BM * 8, SB_BYTES = BN * 8;
    static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
    static constexpr int A_LOADS = A_BYTES / 1024, B_LOADS = B_BYTES / 1024;
    static constexpr int SA_LOADS = SA_BYTES / 256, SB_LOADS = SB_BYTES / 256;
    static_assert(A_LOADS % NW == 0 && B_LOADS % NW == 0, "data loads split evenly");
    static_assert(2 * STAGE <= 160 * 1024, "LDS capacity");
    static __device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }
};

// block scales of rows r0.. (8 bytes = 8 blocks of 16 per 128-K chunk), two dwords per row,
// rows past the end repeat the last row
template <int LOADS, int NW>
__device__ __forceinline__ void dma_scales(const uint8_t* __restrict__ s, int64_t rows_left,
                                           int64_t K, int64_t r0, int64_t kb, uint32_t lds,
                                           int wave, int lane)
{
#pragma unroll
    for (int u = 0; u < (LOADS + NW - 1) / NW; ++u) {
        const int is = u * NW + wave;
        if (is < LOADS) {
            const int idx = is * 64 + lane;
            int64_t row = idx >> 1;
            row = row < rows_left ? row : rows_left - 1;
            dma_b32(s + (r0 + row) * (K / 16) + kb * 8 + (idx & 1) * 4, lds + is * 256);
        }
    }
}

template <class Cfg>
__device__ __forceinline__ void nvfp4_load(uint8_t LDS* stage, const uint8_t* __restrict__ A,
                                           const uint8_t* __restrict__ sA,
                                           const uint8_t* __restrict__ B,
                                           const uint8_t* __restrict__ sB, int64_t M, int64_t N,
                                           int64_t K, int64_t m0, int64_t n0, int64_t kb,
                                           int wave, int lane)
{
    // instruction ia covers tile rows 16ia..16ia+15: lane -> row 16ia + lane/4, physical
    // 16-byte chunk lane%4 holding logical chunk (lane%4) ^ swz(row)
#pragma unroll
    for (int u = 0; u < Cfg::A_LOADS / Cfg::NW; ++u) {
        const int ia = u * Cfg::NW + wave;
        const int row = ia * 16 + (lane >> 2);
        const int c = (lane & 3) ^ Cfg::swz(row);
        int64_t gm = m0 + row;
        gm = gm < M ? gm : M - 1;
        dma_b128(A + gm * (K / 2) + kb * 64 + c * 16, lds_addr(stage + ia * 1024));
    }
#pragma unroll
    for (int u = 0; u < Cfg::B_LOADS / Cfg::NW; ++u) {
        const int ib = u * Cfg::NW + wave;
        const int row = ib * 16 + (lane >> 2);
        const int c = (lane & 3) ^ Cfg::swz(row);
        int64_t gn = n0 + row;
        gn = gn < N ? gn : N - 1;
        dma_b128(B + gn * (K / 2) + kb * 64 + c * 16,
                 lds_addr(stage + Cfg::A_BYTES + ib * 1024));
    }
    dma_scales<Cfg::SA_LOADS, Cfg::NW>(sA, M - m0, K, m0, kb,
                                       lds_addr(stage + Cfg::A_BYTES + Cfg::B_BYTES), wave,
                                       lane);
    dma_scales<Cfg::SB_LOADS, Cfg::NW>(
        sB, N - n0, K, n0, kb, lds_addr(stage + Cfg::A_BYTES + Cfg::B_BYTES + Cfg::SA_BYTES),
        wave, lane);
}

// 32 E2M1 codes (16 bytes: k 32g..32g+31) with the E4M3 scales of their two blocks -> the
// four f16x8 MFMA operands of sub-steps t = 0..3 (sub-step t is bytes 4t..4t+3, block t/2)
__device__ __forceinline__ void fp4_operands(i32x4 raw, uint32_t scale2, f16x8 (&op)[4])
{
    const f16x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)scale2, 1.0f, false);
    const f16x2 s0 = f16x2{sc[0], sc[0]}, s1 = f16x2{sc[1], sc[1]};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const f16x2 s = t < 2 ? s0 : s1;
        const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw[t], 1.0f, 0) * s;
        const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw[t], 1.0f, 1) * s;
        const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw[t], 1.0f, 2) * s;
        const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw[t], 1.0f, 3) * s;
        op[t] = f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    }
}

// KG > 1 (shapes with few output tiles): the workgroup holds KG groups of NW waves; group c
// takes chunks c, c+KG, ... with its own 2-stage ring, and the KG partial tiles are summed in
// LDS in group order (a fixed order: results are repeatable bit for bit).
template <class Cfg, bool OUT_BF16, int KG = 1>
__global__ __launch_bounds__(Cfg::NT * KG) void gemm_nvfp4_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ sA, const float* __restrict__ gA,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ sB, const float* __restrict__ gB,
    void* __restrict__ Cout, int64_t M, int64_t N, int64_t K)
{
    constexpr int RING = KG * 2 * Cfg::STAGE;
    constexpr int RED = (KG - 1) * Cfg::NT * Cfg::FM * Cfg::FN * 16;
    __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[RING > RED ? RING : RED];
    const int lane = threadIdx.x & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kg = wave_all / Cfg::NW, wave = wave_all % Cfg::NW;
    uint8_t LDS* const smem = (uint8_t LDS*)smem_raw + kg * 2 * Cfg::STAGE;
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
    const int g = lane >> 4, q = lane & 15;

    // tiles: XCD-contiguous ranges, walked in groups of 4 tile rows (as the FP8 GEMM)
    const int64_t tiles_m = (M + Cfg::BM - 1) / Cfg::BM, tiles_n = N / Cfg::BN;
    const int64_t G = (int64_t)gridDim.x;
    int64_t pid = blockIdx.x;
    if (G % 8 == 0)
        pid = (pid % 8) * (G / 8) + pid / 8;
    constexpr int GROUP_M = 4;
    const int64_t first_m = (pid / (GROUP_M * tiles_n)) * GROUP_M;
    const int64_t gsize = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
    const int64_t m0 = (first_m + pid % gsize) * Cfg::BM;
    const int64_t n0 = ((pid % (GROUP_M * tiles_n)) / gsize) * Cfg::BN;
    const int64_t KB = K / 128;

    int a_off[Cfg::FM], sa_off[Cfg::FM], b_off[Cfg::FN], sb_off[Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
        const int row = wm * Cfg::TM + 16 * i + q;
        a_off[i] = row * 64 + ((g ^ Cfg::swz(row)) * 16);
        sa_off[i] = Cfg::A_BYTES + Cfg::B_BYTES + row * 8 + 2 * g;
    }
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
        const int row = wn * Cfg::TN + 16 * j + q;
        b_off[j] = Cfg::A_BYTES + row * 64 + ((g ^ Cfg::swz(row)) * 16);
        sb_off[j] = Cfg::A_BYTES + Cfg::B_BYTES + Cfg::SA_BYTES + row * 8 + 2 * g;
    }

    f32x4 acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // step st: this group's chunk kb = st*KG + kg (when below KB)
    const int64_t steps = (KB + KG - 1) / KG;
    if (steps > 0 && kg < KB)
        nvfp4_load<Cfg>(smem, A, sA, B, sB, M, N, K, m0, n0, kg, wave, lane);
    for (int64_t st = 0; st < steps; ++st) {
        const int64_t kb = st * KG + kg;
        const uint8_t LDS* cur = smem + (st & 1) * Cfg::STAGE;
        wait_vm<0>();
        lds_barrier();   // step st visible to all; step st-1 fully read
        if (kb + KG < KB)
            nvfp4_load<Cfg>(smem + ((st + 1) & 1) * Cfg::STAGE, A, sA, B, sB, M, N, K, m0, n0,
                            kb + KG, wave, lane);
        if (kb >= KB)
            continue;
        f16x8 af[Cfg::FM][4];
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i) {
            const i32x4 raw = *(const i32x4 LDS*)(cur + a_off[i]);
            const uint32_t s2 = *(const uint16_t LDS*)(cur + sa_off[i]);
            fp4_operands(raw, s2, af[i]);
        }
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) {
            f16x8 bf[4];
            const i32x4 raw = *(const i32x4 LDS*)(cur + b_off[j]);
            const uint32_t s2 = *(const uint16_t LDS*)(cur + sb_off[j]);
            fp4_operands(raw, s2, bf);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < Cfg::FM; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i][t], bf[t],
                                                                       acc[i][j], 0, 0, 0);
        }
    }

    if (KG > 1) {
        // the KG partial tiles, summed in group order
        lds_barrier();
        float LDS* const red = (float LDS*)smem_raw;
        constexpr int PER_LANE = Cfg::FM * Cfg::FN * 4;
        if (kg > 0) {
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j)
                    *(f32x4 LDS*)(red + (((kg - 1) * Cfg::NT + wave * 64 + lane) * PER_LANE +
                                         (i * Cfg::FN + j) * 4)) = acc[i][j];
        }
        lds_barrier();
        if (kg != 0)
            return;
#pragma unroll
        for (int c = 1; c < KG; ++c)
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FN; ++j)
                    acc[i][j] += *(const f32x4 LDS*)(red + (((c - 1) * Cfg::NT + wave * 64 + lane) *
                                                                PER_LANE +
                                                            (i * Cfg::FN + j) * 4));
    }
    // lane holds C[16i + 4g + r][16j + q] of the wave tile.  The two global scales multiply
    // as mantissas (each in [0.5, 1)) and one exponent applied last by ldexp, so the product
    // gA*gB cannot overflow where C itself is finite.
    int ea = 0, eb = 0;
    const float ma = frexpf(*gA, &ea), mb = frexpf(*gB, &eb);
    const float gm = ma * mb;
    const int ge = ea + eb;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + wm * Cfg::TM + 16 * i + 4 * g + r;
            if (row >= M)
                continue;
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j) {
                const int64_t col = n0 + wn * Cfg::TN + 16 * j + q;
                const float v = ldexpf(acc[i][j][r] * gm, ge);
                if (OUT_BF16)
                    static_cast<__bf16*>(Cout)[row * N + col] = (__bf16)v;
                else
                    static_cast<float*>(Cout)[row * N + col] = v;
            }
        }
}

template <class Cfg, int KG = 1>
static hipError_t launch_nvfp4_cfg(const void* A_q, const uint8_t* sA, const float* gA,
                                   const void* B_q, const uint8_t* sB, const float* gB, void* C,
                                   int64_t M, int64_t N, int64_t K, int out_bf16,
                                   hipStream_t stream)
{
    const int64_t tiles = ((M + Cfg::BM - 1) / Cfg::BM) * (N / Cfg::BN);
    if (!grid_fits(tiles, Cfg::NT * KG))
        return hipErrorInvalidConfiguration;
    if (out_bf16)
        hipLaunchKernelGGL((gemm_nvfp4_kernel<Cfg, true, KG>), dim3((unsigned)tiles),
                           dim3(Cfg::NT * KG), 0, stream, static_cast<const uint8_t*>(A_q), sA,
                           gA, static_cast<const uint8_t*>(B_q), sB, gB, C, M, N, K);
    else
        hipLaunchKernelGGL((gemm_nvfp4_kernel<Cfg, false, KG>), dim3((unsigned)tiles),
                           dim3(Cfg::NT * KG), 0, stream, static_cast<const uint8_t*>(A_q), sA,
                           gA, static_cast<const uint8_t*>(B_q), sB, gB, C, M, N, K);
    return hipGetLastError();
}

// few output tiles: 64x32 tiles (2 waves of 32x32) with the K chunks over 4 wave groups while
// they fit one round of the CUs, else 64x64 tiles (4 waves of 32x32) over 2 wave groups
#ifndef FGQ_NVFP4_NARROW_CFG
#define FGQ_NVFP4_NARROW_CFG 64, 32, 2, 1
#endif
#ifndef FGQ_NVFP4_NARROW_KG
#define FGQ_NVFP4_NARROW_KG 4
#endif
#ifndef FGQ_NVFP4_SMALL_CFG
#define FGQ_NVFP4_SMALL_CFG 64, 64, 2, 2
#endif
#ifndef FGQ_NVFP4_SMALL_KG
#define FGQ_NVFP4_SMALL_KG 2
#endif

hipError_t launch_gemm_nvfp4(const void* A_q, const uint8_t* sA, const float* gA,
                             const void* B_q, const uint8_t* sB, const float* gB, void* C,
                             int64_t M, int64_t N, int64_t K, int out_bf16, hipStream_t stream)
{
    // 128x128 tiles while they cover the 256 CUs at least once (256x128 from M = 256); fewer
    // tiles than that: the K-split families above (measured back to back: 128x7168x2048 21.7 ->
    // 10.6 us, 1x7168x2048 20.3 -> 7.0 us, 128x256x512 7.9 -> 4.5 us)
    const int64_t tiles128 = ((M + 127) / 128) * (N / 128);
    if (tiles128 < 256) {
        using Narrow = Nvfp4Cfg<FGQ_NVFP4_NARROW_CFG>;
        const int cus = device_cus() > 0 ? device_cus() : 256;
        if (((M + Narrow::BM - 1) / Narrow::BM) * (N / Narrow::BN) <= cus)
            return launch_nvfp4_cfg<Narrow, FGQ_NVFP4_NARROW_KG>(A_q, sA, gA, B_q, sB, gB, C, M,
                                                                 N, K, out_bf16, stream);
        return launch_nvfp4_cfg<Nvfp4Cfg<FGQ_NVFP4_SMALL_CFG>, FGQ_NVFP4_SMALL_KG>(
            A_q, sA, gA, B_q, sB, gB, C, M, N, K, out_bf16, stream);
    }
    if (M >= 256)
        return launch_nvfp4_cfg<Nvfp4Cfg<256, 128, 4, 2>>(A_q, sA, gA, B_q, sB, gB, C, M, N, K,
                                                          out_bf16, stream);
    return launch_nvfp4_cfg<Nvfp4Cfg<128, 128, 2, 2>>(A_q, sA, gA, B_q, sB, gB, C, M, N, K,
                                                      out_bf16, stream);
}

}  // namespace fgq
