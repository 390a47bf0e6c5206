// gemm.hip -- block-scaled FP8 (E4M3) GEMM for gfx950.
//
// Page "Fine-Grained FP8/FP4 Quantization", section "DeepGEMM: Tile-wise and Block-wise
// Scaling": A_q [M,K] with scale_A [M, K/128], B_q [K,N] (N contiguous) with scale_B
// [K/128, N/128]; for every 128-wide K chunk kb the FP8 partial P = A_q[:,kb] * B_q[kb,:]
// is multiplied by scale_A[m,kb] * scale_B[kb, n/128] and accumulated in fp32 (the idea of
// the page's Hopper section: promote each 128-K partial into an fp32 accumulator, here in
// VGPRs).  C is overwritten, fp32 or bf16.
//
// gfx950 mapping:
//   * the chunk partial is formed by f16 MFMAs (v_mfma_f32_16x16x32_f16, four chained per
//     128-K chunk) on operands converted exactly from E4M3 (every E4M3 value is an f16
//     value).  The FP8 MFMAs of gfx950 are not used for the partial: their internal sum
//     keeps only about 14 bits below the largest product of a reduction, measured at up to
//     1.9e-4 * sum|a*b| of error per 128-K chunk, while the f16 MFMA sums to fp32 accuracy
//     (about 3e-7 * sum|a*b|), the accuracy the fp32 accumulation of the method needs;
//   * the scale is applied by one v_fma_f32 per output element per chunk,
//     acc = fma(P, sA*sB, acc);
//   * A/B chunks are staged in LDS as E4M3 bytes, double-buffered, filled by
//     global_load_lds_dwordx4 (direct to LDS, no VGPR staging), the refill of one stage
//     issued a few loads at a time between the column blocks of the other's compute;
//     16-byte columns are XOR-swizzled by row so that fragment reads spread over the banks;
//     operands are converted to f16 in registers after the LDS read
//     (v_cvt_scalef32_pk_f16_fp8);
//   * B stays N-contiguous in LDS; its operand (one column, consecutive k per lane) is
//     gathered by ds_read_b64_tr_b8, which transposes an 8(k) x 16(n) byte block across
//     each 16-lane group;
//   * scale_A rows of the tile ride along in the LDS stage; scale_B is one scalar per wave
//     per chunk (a wave's columns never straddle a 128-column block).
#include "fgq_device.hpp"
#include "fgq_launch.hpp"
#include "gemm_common.hpp"

#include <atomic>
#include <type_traits>

// compile-time tuning knobs (defaults are the shipped configuration)
#ifndef FGQ_SCHED
#define FGQ_SCHED 0
#endif
#ifndef FGQ_SWZ
#define FGQ_SWZ 1
#endif
#ifndef FGQ_STAGED_STORE
#define FGQ_STAGED_STORE 1
#endif
#ifndef FGQ_SPREAD_DMA
#define FGQ_SPREAD_DMA 1
#endif

namespace fgq {

template <int BM_, int BN_, int WM_, int WN_, int STAGES_>
struct GemmCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, STAGES = STAGES_;
    static constexpr int NW = WM * WN, NT = 64 * NW;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 16, FN = TN / 16;
    static constexpr int A_BYTES = BM * 128, B_BYTES = 128 * BN, S_BYTES = BM * 4;
    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    // the bf16 tile staged for the epilogue: rows of BN values plus 16 bytes
    static constexpr int STAGED_LD = BN * 2 + 16;
    static constexpr int SMEM = STAGES * STAGE > BM * STAGED_LD ? STAGES * STAGE : BM * STAGED_LD;
    static constexpr int A_LOADS = A_BYTES / 1024;   // 1 KB per wave instruction
    static constexpr int B_LOADS = B_BYTES / 1024;
    static constexpr int S_LOADS = BM / 64;           // 256 B per wave instruction
    static constexpr int B_ROWS_PER_LOAD = 1024 / BN;
    static constexpr int B_CHUNKS = BN / 16;
    static_assert(TN <= 128 && 128 % TN == 0, "a wave's columns must sit in one 128-block");
    static_assert(TM % 16 == 0 && TN % 16 == 0 && BN >= 32 && BM % 64 == 0, "tile shape");
    static_assert(A_LOADS % NW == 0 && B_LOADS % NW == 0, "loads split evenly over waves");
    static_assert(S_LOADS <= NW, "one scale load per wave at most");
    static_assert(STAGES >= 2 && STAGES <= 4, "LDS ring depth");
    static_assert(SMEM <= 160 * 1024, "LDS capacity (160 KB per CU)");
    // 16-byte column swizzles.  gfx950 LDS has 64 banks of 4 bytes (256 B per cycle): a
    // ds_read_b128 serves 16 lanes per cycle, a ds_read_b64(_tr) 32 lanes.  A rows are 128 B
    // (two per bank line): the 16 rows of a fragment read in one cycle take 16 distinct
    // 16-byte slots when the column is XORed with (row/2)%8.  B rows read together by one
    // b64 transposed read are k = 32g + 8t + 0..7 for g in {0,1}: the swizzle mixes k%8 and
    // bit 5 of k so those 16 rows hit distinct slots too.
    static __device__ __forceinline__ int a_swz(int row)
    {
#if FGQ_SWZ
        return (row >> 1) & 7;
#else
        return row & 7;
#endif
    }
    static __device__ __forceinline__ int b_swz(int k)
    {
#if FGQ_SWZ
        // BN = 32: rows are two 16-byte chunks; the 8 rows of one transposed read already
        // cover 32 banks, and bit 5 of k separates the two groups read in the same cycle
        if (B_CHUNKS == 2)
            return (k >> 5) & 1;
        // BN = 64: four rows per 256-byte bank line; bit 2 and bit 5 of k separate the 16
        // rows read in one cycle
        if (B_CHUNKS == 4)
            return ((k >> 2) & 1) | (((k >> 5) & 1) << 1);
        return B_CHUNKS == 8 ? (((k >> 1) & 3) | (((k >> 5) & 1) << 2))
                             : ((k & 7) | (((k >> 5) & 1) << 3));
#else
        return k & 7;
#endif
    }
    static_assert(B_CHUNKS == 2 || B_CHUNKS == 4 || B_CHUNKS == 8 || B_CHUNKS == 16,
                  "BN is 32, 64, 128 or 256");
    // waits: every wave issues this many direct-to-LDS loads per stage (S loads go to the
    // first S_LOADS waves); the pipeline waits with the smallest count, which is safe.
    static constexpr int MIN_LOADS = (A_LOADS + B_LOADS) / NW;
};

// Scale formats the GEMM reads: fp32 scales, or UE8M0 exponent bytes e standing for
// 2^(e-127) (page "Fine-Grained FP8/FP4 Quantization", section "Blackwell: Native Block
// Scaling").  Either way one 4-byte LDS slot per tile row carries scale_A of the chunk.
// The scaled partial P*sA*sB is formed without an overflow that C itself would not have:
//   sB <= 1: acc = fma(P, sA*sB, acc) -- the combined scale is at most sA, so it cannot
//            overflow (an underflow of it costs less than 2^-149 * |P|, far below the
//            tolerance's absolute term);
//   sB >  1: acc = fma(P*sA, sB, acc) -- P*sA can only overflow where P*sA*sB, a term of C,
//            lies beyond the fp32 range anyway.
// sB is uniform over a wave, so the choice is a scalar branch per chunk (row()/combine()
// give the per-row factor of each form).
template <bool E8>
struct ScaleIn;
template <>
struct ScaleIn<false> {
    typedef float T;
    static __device__ __forceinline__ void dma(const T* p, uint32_t lds) { dma_b32(p, lds); }
    static __device__ __forceinline__ float value(T v) { return v; }
    static __device__ __forceinline__ f32x4 combine(const uint8_t LDS* p, float sb)
    {
        return *(const f32x4 LDS*)p * sb;
    }
    static __device__ __forceinline__ f32x4 row(const uint8_t LDS* p)
    {
        return *(const f32x4 LDS*)p;
    }
};
template <>
struct ScaleIn<true> {
    typedef uint8_t T;
    static __device__ __forceinline__ void dma(const T* p, uint32_t lds) { dma_u8(p, lds); }
    static __device__ __forceinline__ float value(T e)
    {
        return __builtin_ldexpf(1.0f, (int)e - 127);
    }
    // 2^(eA-127) * sB by an exponent add: exact unless it falls below the fp32 range
    static __device__ __forceinline__ f32x4 combine(const uint8_t LDS* p, float sb)
    {
        const i32x4 e = *(const i32x4 LDS*)p;
        return f32x4{__builtin_ldexpf(sb, e[0] - 127), __builtin_ldexpf(sb, e[1] - 127),
                     __builtin_ldexpf(sb, e[2] - 127), __builtin_ldexpf(sb, e[3] - 127)};
    }
    // 2^(eA-127) itself (exact in fp32 for every byte 0..254)
    static __device__ __forceinline__ f32x4 row(const uint8_t LDS* p)
    {
        return combine(p, 1.0f);
    }
};

// The scale_B values one wave uses, one per chunk it computes, taken in order i = 0, 1, ...
// from p[i * stride] (i < n).  fp32 scales come by scalar loads, each issued one chunk ahead so
// that it completes under the LDS barrier's wait.  UE8M0 bytes can only come by vector loads,
// and a chunk waiting for its own byte would also wait for every operand prefetch in flight;
// so the bytes of 64 chunks are loaded at once, one per lane, and chunk i reads lane i % 64.
template <class SI>
struct ScaleBWalk;
template <>
struct ScaleBWalk<ScaleIn<false>> {
    const float* p;
    int64_t stride, n;
    float next;
    __device__ __forceinline__ ScaleBWalk(const float* p_, int64_t stride_, int64_t n_, int)
        : p(p_), stride(stride_), n(n_), next(n_ > 0 ? p_[0] : 0.0f)
    {
    }
    __device__ __forceinline__ float get(int64_t i)
    {
        const float v = next;
        if (i + 1 < n)
            next = p[(i + 1) * stride];
        return v;
    }
};
template <>
struct ScaleBWalk<ScaleIn<true>> {
    const uint8_t* p;
    int64_t stride, n;
    int lane, raw;
    __device__ __forceinline__ ScaleBWalk(const uint8_t* p_, int64_t stride_, int64_t n_,
                                          int lane_)
        : p(p_), stride(stride_), n(n_), lane(lane_)
    {
        fill(0);
    }
    __device__ __forceinline__ void fill(int64_t i0)
    {
        const int64_t i = i0 + lane;
        raw = i < n ? (int)p[i * stride] : 127;
    }
    __device__ __forceinline__ float get(int64_t i)
    {
        if ((i & 63) == 0 && i > 0)
            fill(i);
        return ScaleIn<true>::value((uint8_t)__builtin_amdgcn_readlane(raw, (int)(i & 63)));
    }
};


template <class Cfg, class SI>
__device__ __forceinline__ void load_stage(uint8_t LDS* stage, const uint8_t* __restrict__ A,
                                           const typename SI::T* __restrict__ sA,
                                           const uint8_t* __restrict__ B, int64_t M,
                                           int64_t N, int64_t K, int64_t m0, int64_t n0,
                                           int64_t kb, int wave, int lane)
{
    const int64_t KB = K / 128;
    // A: instruction ia covers tile rows 8ia..8ia+7; lane -> row 8ia + lane/8, physical
    // 16-byte column lane%8, which holds logical column (lane%8) ^ (row%8).
#pragma unroll
    for (int u = 0; u < Cfg::A_LOADS / Cfg::NW; ++u) {
        const int ia = u * Cfg::NW + wave;
        const int row = ia * 8 + (lane >> 3);
        const int c = (lane & 7) ^ Cfg::a_swz(row);
        int64_t gm = m0 + row;
        gm = gm < M ? gm : M - 1;
        dma_b128(A + gm * K + kb * 128 + c * 16, lds_addr(stage + ia * 1024));
    }
    // B: instruction ib covers k rows ib*R..ib*R+R-1 (R = 1024/BN); lane -> row
    // ib*R + lane/(BN/16), physical column lane%(BN/16) holding logical column p ^ (k%8).
#pragma unroll
    for (int u = 0; u < Cfg::B_LOADS / Cfg::NW; ++u) {
        const int ib = u * Cfg::NW + wave;
        const int k = ib * Cfg::B_ROWS_PER_LOAD + lane / Cfg::B_CHUNKS;
        const int p = lane % Cfg::B_CHUNKS;
        const int c = p ^ Cfg::b_swz(k);
        int64_t gn = n0 + c * 16;
        gn = gn < N ? gn : N - 16;
        dma_b128(B + (kb * 128 + k) * N + gn, lds_addr(stage + Cfg::A_BYTES + ib * 1024));
    }
    // scale_A rows of the tile: one fp32 per row, gathered with stride K/128.
    if (wave < Cfg::S_LOADS) {
        int64_t gm = m0 + wave * 64 + lane;
        gm = gm < M ? gm : M - 1;
        SI::dma(sA + gm * KB + kb, lds_addr(stage + Cfg::A_BYTES + Cfg::B_BYTES + wave * 256));
    }
}

// LDS byte offsets of a wave's operand fragments inside a stage.  A: fragment i (rows
// row0 + 16i + q) is a0/a1 + 2048*i -- the row swizzle (row/2)%8 does not change with i -- so
// the 16 offsets are two registers plus immediates.  B: the wave's column block j is 16-byte
// chunk ch0 + j; with ch0 a multiple of the power-of-two FN, (ch0 + j) ^ swz = (ch0 ^ swz) ^ j
// and the address fields (k*BN, chunk*16, half*8) occupy disjoint bits, so block j's offset
// for sub-step t is b[t] ^ 16*j.
template <class Cfg>
struct FragOffsets {
    static_assert((Cfg::FN & (Cfg::FN - 1)) == 0, "power-of-two column blocks per wave");
    int a0, a1;
    int b[4];
    __device__ __forceinline__ FragOffsets(int row0, int ch0, int g, int q)
    {
        const int row = row0 + q;
        a0 = row * 128 + (((2 * g) ^ Cfg::a_swz(row)) * 16);
        a1 = row * 128 + (((2 * g + 1) ^ Cfg::a_swz(row)) * 16);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int k = 32 * g + 8 * t + (q >> 1);
            b[t] = Cfg::A_BYTES + k * Cfg::BN + ((ch0 ^ Cfg::b_swz(k)) * 16) + 8 * (q & 1);
        }
    }
    __device__ __forceinline__ int a(int i, int h) const { return (h ? a1 : a0) + 2048 * i; }
    __device__ __forceinline__ int bo(int j, int t) const { return b[t] ^ (16 * j); }
};

// The wave's direct-to-LDS loads of one stage as separately issued pieces (A loads, then B
// loads, then the scale load), so that a chunk's refill can be spread over the column
// blocks of the previous chunk's compute: issued all at once right after a barrier, the 56
// loads of the eight waves queue at the CU's address unit (about 1 KB per 16 cycles) and
// hold every wave for hundreds of cycles while its SIMD's matrix core idles.
template <class Cfg, class SI>
struct StageLoader {
    static constexpr int NA = Cfg::A_LOADS / Cfg::NW, NBL = Cfg::B_LOADS / Cfg::NW;
    static constexpr int PIECES = NA + NBL + 1;
    // pieces per column block, over the first FN-1 blocks (the last block issues none, so
    // the last piece still has most of a chunk to land)
    static constexpr int PER = Cfg::FN > 1 ? (PIECES + Cfg::FN - 2) / (Cfg::FN - 1) : PIECES;
    uint8_t LDS* stage;
    const uint8_t* __restrict__ A;
    const typename SI::T* __restrict__ sA;
    const uint8_t* __restrict__ B;
    int64_t M, N, K, m0, n0, kb;
    int wave, lane;
    bool active;

    __device__ __forceinline__ void piece(int pc) const
    {
        if (pc < NA) {
            const int ia = pc * Cfg::NW + wave;
            const int row = ia * 8 + (lane >> 3);
            const int c = (lane & 7) ^ Cfg::a_swz(row);
            int64_t gm = m0 + row;
            gm = gm < M ? gm : M - 1;
            dma_b128(A + gm * K + kb * 128 + c * 16, lds_addr(stage + ia * 1024));
        } else if (pc < NA + NBL) {
            const int ib = (pc - NA) * Cfg::NW + wave;
            const int k = ib * Cfg::B_ROWS_PER_LOAD + lane / Cfg::B_CHUNKS;
            const int q = lane % Cfg::B_CHUNKS;
            const int c = q ^ Cfg::b_swz(k);
            int64_t gn = n0 + c * 16;
            gn = gn < N ? gn : N - 16;
            dma_b128(B + (kb * 128 + k) * N + gn, lds_addr(stage + Cfg::A_BYTES + ib * 1024));
        } else if (wave < Cfg::S_LOADS) {
            int64_t gm = m0 + wave * 64 + lane;
            gm = gm < M ? gm : M - 1;
            SI::dma(sA + gm * (K / 128) + kb,
                    lds_addr(stage + Cfg::A_BYTES + Cfg::B_BYTES + wave * 256));
        }
    }
    // the pieces that go out just before column block j
    __device__ __forceinline__ void before_block(int j) const
    {
        if (!active)
            return;
#pragma unroll
        for (int pc = j * PER; pc < (j + 1) * PER && pc < PIECES; ++pc)
            piece(pc);
    }
};

// loader that issues nothing (the chunk's refill went out elsewhere)
struct NoLoader {
    __device__ __forceinline__ void before_block(int) const {}
};

// One 128-K chunk of the wave's 16x16 tiles (and, with a StageLoader, the refill of another
// stage between its column blocks).  The chunk's combined scales and the wave's A operands
// are read and converted once; then per column block j the B operands, four chained f16
// MFMAs per tile, and acc += P * (sA*sB).
template <class Cfg, class SI, bool BIG_SB, class Loader>
__device__ __forceinline__ void compute_chunk_impl(const uint8_t LDS* cur,
                                                   const FragOffsets<Cfg>& fo, int s_off, float sb,
                                                   f32x4 (&acc)[Cfg::FM][Cfg::FN],
                                                   const Loader& loader)
{
    // per-row factors for this lane's rows: sA[row, kb] * sB[kb, nb], or sA alone when
    // sB > 1 (then sB multiplies after sA, see ScaleIn)
    f32x4 cs[Cfg::FM];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
        cs[i] = BIG_SB ? SI::row(cur + s_off + i * 64) : SI::combine(cur + s_off + i * 64, sb);
    // A operands: lane bytes 8t..8t+7 of its 32 (k = 32g + 8t + b) -> sub-step t
    i32x4 araw[Cfg::FM][2];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
        araw[i][0] = *(const i32x4 LDS*)(cur + fo.a(i, 0));
        araw[i][1] = *(const i32x4 LDS*)(cur + fo.a(i, 1));
    }
    // B operands: transposed read t gives k = 32g + 8t + b for column q -> sub-step t
    i32x2 braw[2][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        braw[0][t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 LDS*)(cur + fo.bo(0, t)));
    f16x8 af[Cfg::FM][4];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
        af[i][0] = e4m3x8_to_f16(araw[i][0][0], araw[i][0][1]);
        af[i][1] = e4m3x8_to_f16(araw[i][0][2], araw[i][0][3]);
        af[i][2] = e4m3x8_to_f16(araw[i][1][0], araw[i][1][1]);
        af[i][3] = e4m3x8_to_f16(araw[i][1][2], araw[i][1][3]);
    }
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
        loader.before_block(j);
        if (j + 1 < Cfg::FN) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                braw[(j + 1) & 1][t] =
                    __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 LDS*)(cur + fo.bo(j + 1, t)));
        }
        f16x8 bf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            bf[t] = e4m3x8_to_f16(braw[j & 1][t][0], braw[j & 1][t][1]);
        f32x4 p[Cfg::FM];
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
            p[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i][0], bf[0], f32x4{0.f, 0.f, 0.f, 0.f},
                                                          0, 0, 0);
#pragma unroll
        for (int t = 1; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < Cfg::FM; ++i)
                p[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i][t], bf[t], p[i], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[i][j][r] = BIG_SB ? __builtin_fmaf(p[i][r] * cs[i][r], sb, acc[i][j][r])
                                      : __builtin_fmaf(p[i][r], cs[i][r], acc[i][j][r]);
    }
#if FGQ_SCHED == 1
    __builtin_amdgcn_iglp_opt(0);
#elif FGQ_SCHED == 2
    __builtin_amdgcn_iglp_opt(1);
#endif
}

// one chunk in the scale form of the loop it belongs to (BIG_SB: some sB of the wave > 1)
template <class Cfg, class SI, bool BIG_SB, class Loader = NoLoader>
__device__ __forceinline__ void compute_chunk(const uint8_t LDS* cur, const FragOffsets<Cfg>& fo,
                                              int s_off, float sb,
                                              f32x4 (&acc)[Cfg::FM][Cfg::FN],
                                              const Loader& loader = Loader())
{
    compute_chunk_impl<Cfg, SI, BIG_SB>(cur, fo, s_off, sb, acc, loader);
}

// Whether any of the n scale_B values p[i * stride] (i < n) a wave uses exceeds 1, as a
// wave-uniform flag: the wave then runs its K loop in the overflow-safe form (see ScaleIn).
// The first 64 values are loaded by the constructor, one per lane, before the kernel's
// prologue loads, so that their latency hides under those; any() reads the rest (K beyond
// 64 chunks per wave) and votes.
template <class SI>
struct ScaleBFlag {
    const typename SI::T* __restrict__ p;
    int64_t stride, n;
    int lane;
    float first;
    __device__ __forceinline__ ScaleBFlag(const typename SI::T* __restrict__ p_, int64_t stride_,
                                          int64_t n_, int lane_)
        : p(p_), stride(stride_), n(n_), lane(lane_),
          first(lane_ < n_ ? SI::value(p_[lane_ * stride_]) : 0.0f)
    {
    }
    __device__ __forceinline__ bool any_above_one() const
    {
        bool big = first > 1.0f;
        for (int64_t i0 = 64; i0 < n; i0 += 64) {
            const int64_t i = i0 + lane;
            if (i < n && SI::value(p[i * stride]) > 1.0f)
                big = true;
        }
        return __builtin_amdgcn_ballot_w64(big) != 0;
    }
};

// Fused epilogue: the tile's bf16 results are staged in LDS, then every 1x128 row group is
// written to C and quantized exactly as the activation quantizer does it (same amax, scale
// and E4M3 conversion routines), giving the next layer's codes and scales without a second
// pass over C.  Page "Kernel Fusion" (overview: one launch instead of a global-memory round
// trip) applied to the 1x128 activation rule of page "Fine-Grained FP8/FP4 Quantization",
// section "Scaling Granularities".
template <class Cfg, bool QUANT>
__device__ __forceinline__ void store_quant_tile(uint8_t LDS* smem,
                                                 const f32x4 (&acc)[Cfg::FM][Cfg::FN],
                                                 __bf16* __restrict__ C, uint8_t* __restrict__ Cq,
                                                 float* __restrict__ sC, int64_t M, int64_t N,
                                                 int64_t m0, int64_t n0, int wm, int wn, int g,
                                                 int q)
{
    // staged row: BN bf16 plus 16 bytes, so the four row groups 4g+r written together by a
    // wave land on different banks
    constexpr int LD = Cfg::STAGED_LD;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wm * Cfg::TM + 16 * i + 4 * g + r;
                const int col = wn * Cfg::TN + 16 * j + q;
                *(__bf16 LDS*)(smem + row * LD + col * 2) = (__bf16)acc[i][j][r];
            }
    lds_barrier();
    // one 16-lane DPP row per 1x128 group: 16 bytes (8 values) per lane
    constexpr int GPR = Cfg::BN / 128;
    const int l16 = threadIdx.x & 15;
    const int64_t NB = N / 128;
#pragma unroll
    for (int g0 = 0; g0 < Cfg::BM * GPR; g0 += Cfg::NT / 16) {
        const int grp = g0 + (int)(threadIdx.x >> 4);
        const int row = grp / GPR, cg = grp % GPR;
        const u32x4 v = *(const u32x4 LDS*)(smem + row * LD + cg * 256 + l16 * 16);
        const int64_t grow = m0 + row, gcol = n0 + cg * 128 + l16 * 8;
        if (QUANT) {
            const GroupScale gs = group_scale(row16_max(absmax_bits8(v)));
            const u32x2 codes = quantize8(v, gs);
            if (grow < M && gcol < N) {
                *(u32x2*)(Cq + grow * N + gcol) = codes;
                if (l16 == 0)
                    sC[grow * NB + (n0 / 128 + cg)] = gs.s;
            }
        }
        if (grow < M && gcol < N)
            *(u32x4*)(C + grow * N + gcol) = v;
    }
}

// two waves per SIMD (the 128x128 tiles' 4 waves leave room for two workgroups per CU only if
// a wave keeps within 256 registers)
template <class Cfg, class SI, bool OUT_BF16, bool FUSE = false>
__global__ __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_fp8_blockscaled_kernel(
    const uint8_t* __restrict__ A, const typename SI::T* __restrict__ sA,
    const uint8_t* __restrict__ B, const typename SI::T* __restrict__ sB,
    void* __restrict__ Cout, int64_t M, int64_t N, int64_t K, int64_t n_begin, int64_t n_end,
    uint8_t* __restrict__ Cq = nullptr, float* __restrict__ sC = nullptr)
{
    // the ring, or the staged bf16 tile of the epilogue where that is larger
    constexpr bool STAGED = FUSE || (OUT_BF16 && FGQ_STAGED_STORE && Cfg::BN >= 128);
    __shared__ __attribute__((aligned(1024)))
    uint8_t smem_raw[STAGED ? Cfg::SMEM : Cfg::STAGES * Cfg::STAGE];
    uint8_t LDS* const smem = (uint8_t LDS*)smem_raw;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;

    // tile index: spread consecutive workgroups (which the dispatcher deals round-robin to
    // the 8 XCDs) so that each XCD works on one contiguous range of tiles, then walk that
    // range in groups of GROUP_M tile rows so neighbours share A and B panels in L2.  The
    // launch covers the output columns [n_begin, n_end) (all of them unless the launcher
    // splits the columns between two tile shapes).
    const int64_t tiles_m = (M + Cfg::BM - 1) / Cfg::BM;
    const int64_t tiles_n = (n_end - n_begin + Cfg::BN - 1) / Cfg::BN;
    const int64_t G = (int64_t)gridDim.x;
    int64_t pid = blockIdx.x;
    if (G % 8 == 0)
        pid = (pid % 8) * (G / 8) + pid / 8;
    constexpr int GROUP_M = 4;
    const int64_t group = pid / (GROUP_M * tiles_n);
    const int64_t first_m = group * GROUP_M;
    const int64_t gsize = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
    const int64_t tm = first_m + (pid % gsize);
    const int64_t tn = (pid % (GROUP_M * tiles_n)) / gsize;
    const int64_t m0 = tm * Cfg::BM, n0 = n_begin + tn * Cfg::BN;

    const int64_t KB = K / 128, NB = N / 128;
    const int g = lane >> 4;      // k-group of the MFMA operands (32 k each)
    const int q = lane & 15;      // row (A) / column (B) within a 16x16 fragment

    // per-lane LDS offsets inside a stage
    const FragOffsets<Cfg> fo(wm * Cfg::TM, wn * Cfg::FN, g, q);
    const int s_off = Cfg::A_BYTES + Cfg::B_BYTES + (wm * Cfg::TM + 4 * g) * 4;
    const int64_t nb_wave = (n0 + wn * Cfg::TN) / 128;

    f32x4 acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // scale_B of the wave's column block, chunk by chunk (and whether any of it exceeds 1)
    ScaleBWalk<SI> sbw(sB + (nb_wave < NB ? nb_wave : NB - 1), NB, KB, lane);
    const ScaleBFlag<SI> sbf(sB + (nb_wave < NB ? nb_wave : NB - 1), NB, KB, lane);

    // prologue: the first STAGES-1 chunks in flight
#pragma unroll
    for (int st = 0; st < Cfg::STAGES - 1; ++st)
        if (st < KB)
            load_stage<Cfg, SI>(smem + st * Cfg::STAGE, A, sA, B, M, N, K, m0, n0, st, wave, lane);

    // the K loop, in the scale form the wave's scale_B values call for
    auto k_loop = [&](auto big_tag) {
        constexpr bool BIG = decltype(big_tag)::value;
        for (int64_t kb = 0; kb < KB; ++kb) {
            const uint8_t LDS* cur = smem + (kb % Cfg::STAGES) * Cfg::STAGE;
            // chunk kb has landed once only the later chunks' loads may still be outstanding
            // (chunks kb+1 .. kb+STAGES-2, those already issued)
            const int64_t later = (KB - 1 - kb) < (Cfg::STAGES - 2) ? (KB - 1 - kb) : (Cfg::STAGES - 2);
            if (Cfg::STAGES >= 4 && later >= 2)
                wait_vm<2 * Cfg::MIN_LOADS>();
            else if (Cfg::STAGES >= 3 && later >= 1)
                wait_vm<Cfg::MIN_LOADS>();
            else
                wait_vm<0>();
            // all waves: chunk kb visible, and chunk kb-1 fully read (its buffer may refill)
            lds_barrier();
            const int64_t nxt = kb + Cfg::STAGES - 1;
#if FGQ_SPREAD_DMA
            // chunk nxt's loads go out a few at a time between this chunk's column blocks
            const StageLoader<Cfg, SI> loader{smem + (nxt % Cfg::STAGES) * Cfg::STAGE, A, sA, B, M, N,
                                              K, m0, n0, nxt, wave, lane, nxt < KB};
#else
            if (nxt < KB)
                load_stage<Cfg, SI>(smem + (nxt % Cfg::STAGES) * Cfg::STAGE, A, sA, B, M, N, K, m0, n0,
                                nxt, wave, lane);
            const NoLoader loader;
#endif
            const float sb = sbw.get(kb);
            compute_chunk<Cfg, SI, BIG>(cur, fo, s_off, sb, acc, loader);
            if (Cfg::STAGES == 2)
                lds_barrier();   // keeps the waves in step (measured faster than letting them drift)
        }
    };
    if (sbf.any_above_one())
        k_loop(std::true_type{});
    else
        k_loop(std::false_type{});

    static_assert(!FUSE || Cfg::BN >= 128, "the fused epilogue needs whole 128-column groups");
    if constexpr (STAGED) {
        // bf16 C leaves through an LDS-staged tile: 16-byte row-contiguous stores (and, fused,
        // the quantization of every row group)
        lds_barrier();   // every wave is done with the ring: it becomes the staging tile
        store_quant_tile<Cfg, FUSE>(smem, acc, static_cast<__bf16*>(Cout), Cq, sC, M, N, m0,
                                    n0, wm, wn, g, q);
        return;
    }
    static_assert(!FUSE || OUT_BF16, "the fused epilogue writes bf16 C");
    // epilogue: lane holds C[16i + 4g + r][16j + q] of the wave tile
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + wm * Cfg::TM + 16 * i + 4 * g + r;
            if (row >= M)
                continue;
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j) {
                const int64_t col = n0 + wn * Cfg::TN + 16 * j + q;
                if (col >= N)
                    continue;
                if (OUT_BF16)
                    static_cast<__bf16*>(Cout)[row * N + col] = (__bf16)acc[i][j][r];
                else
                    static_cast<float*>(Cout)[row * N + col] = acc[i][j][r];
            }
        }
    }
}

// one launch of a wide tile shape over the output columns [n_begin, n_end)
template <class Cfg, class SI>
static hipError_t launch_cfg(const void* A_q, const void* sA_, const void* B_q, const void* sB_,
                             void* C, int64_t M, int64_t N, int64_t K, int out_bf16,
                             hipStream_t stream, int64_t n_begin = 0, int64_t n_end = -1)
{
    if (n_end < 0)
        n_end = N;
    const typename SI::T* sA = static_cast<const typename SI::T*>(sA_);
    const typename SI::T* sB = static_cast<const typename SI::T*>(sB_);
    const int64_t tiles =
        ((M + Cfg::BM - 1) / Cfg::BM) * ((n_end - n_begin + Cfg::BN - 1) / Cfg::BN);
    if (!grid_fits(tiles, Cfg::NT))
        return hipErrorInvalidConfiguration;
    if (out_bf16)
        hipLaunchKernelGGL((gemm_fp8_blockscaled_kernel<Cfg, SI, true>), dim3((unsigned)tiles),
                           dim3(Cfg::NT), 0, stream, static_cast<const uint8_t*>(A_q), sA,
                           static_cast<const uint8_t*>(B_q), sB, C, M, N, K, n_begin, n_end);
    else
        hipLaunchKernelGGL((gemm_fp8_blockscaled_kernel<Cfg, SI, false>), dim3((unsigned)tiles),
                           dim3(Cfg::NT), 0, stream, static_cast<const uint8_t*>(A_q), sA,
                           static_cast<const uint8_t*>(B_q), sB, C, M, N, K, n_begin, n_end);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Skinny shapes (M <= 128, decode-like): one workgroup per BM x 32 output tile with its K
// chunks split over KG groups of NW waves.  Group c takes chunks c, c+KG, ...: a ring stage
// holds KG chunks side by side, each loaded and computed by its own group with the wide
// kernel's per-chunk code, so KG waves share each SIMD (latency hiding) while the A/B
// stages stay within LDS.  The KG partial tiles are summed in LDS in group order (fixed:
// results are repeatable bit for bit) and stored by group 0.
//
// With splits > 1 (PARTIAL) the K chunks are also divided between workgroups: the grid is
// splits x tiles, workgroup (sp, tile) takes the consecutive chunks [sp*KB/splits,
// (sp+1)*KB/splits) and writes its fp32 partial tile to the workspace slice sp (an [M, N]
// array); splitk_reduce_kernel then sums the slices in slice order.
template <class Cfg, class SI, bool OUT_BF16, int KG, bool PARTIAL = false>
__global__ __launch_bounds__(Cfg::NT * KG) void gemm_fp8_blockscaled_ksplit_kernel(
    const uint8_t* __restrict__ A, const typename SI::T* __restrict__ sA,
    const uint8_t* __restrict__ B, const typename SI::T* __restrict__ sB,
    void* __restrict__ Cout, int64_t M, int64_t N, int64_t K, int64_t splits = 1)
{
    static_assert(Cfg::WN * Cfg::TN == Cfg::BN && Cfg::BN <= 128, "skinny tile");
    static_assert(!(PARTIAL && OUT_BF16), "partials are fp32");
    constexpr int RING = Cfg::STAGES * KG * Cfg::STAGE;
    constexpr int RED = (KG - 1) * Cfg::NT * Cfg::FM * Cfg::FN * 16;
    __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[RING > RED ? RING : RED];
    uint8_t LDS* const smem = (uint8_t LDS*)smem_raw;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kg = wave / Cfg::NW, wl = wave % Cfg::NW;   // K group, wave within the group
    const int wm = wl / Cfg::WN, wn = wl % Cfg::WN;
    const int g = lane >> 4, q = lane & 15;

    // tiles: row tiles fastest, then column tiles, then K splits; XCD-contiguous ranges (ids
    // are dealt round-robin to XCDs), so the workgroups of one XCD share A's K range
    const int64_t tiles_m = (M + Cfg::BM - 1) / Cfg::BM;
    const int64_t tiles = tiles_m * (N / Cfg::BN);
    const int64_t G = (int64_t)gridDim.x;
    int64_t pid = blockIdx.x;
    if (G % 8 == 0)
        pid = (pid % 8) * (G / 8) + pid / 8;
    const int64_t sp = pid / tiles, tile = pid % tiles;
    const int64_t m0 = (tile % tiles_m) * Cfg::BM, n0 = (tile / tiles_m) * Cfg::BN;
    const int64_t KB_ALL = K / 128, NB = N / 128;
    // this workgroup's chunks kb0 .. kb0+KB-1 (all of them without a split)
    const int64_t kb0 = sp * KB_ALL / splits;
    const int64_t KB = (sp + 1) * KB_ALL / splits - kb0;
    const int64_t steps = (KB + KG - 1) / KG;

    const FragOffsets<Cfg> fo(wm * Cfg::TM, wn * Cfg::FN, g, q);
    const int s_off = Cfg::A_BYTES + Cfg::B_BYTES + (wm * Cfg::TM + 4 * g) * 4;
    const int64_t nb = (n0 + wn * Cfg::TN) / 128;

    f32x4 acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // this group's chunk of step s is kb = s*KG + kg (if < KB)
    ScaleBWalk<SI> sbw(sB + (kb0 + kg) * NB + nb, KG * NB, kg < KB ? (KB - kg + KG - 1) / KG : 0,
                       lane);
    const ScaleBFlag<SI> sbf(sB + (kb0 + kg) * NB + nb, KG * NB,
                             kg < KB ? (KB - kg + KG - 1) / KG : 0, lane);
    auto stage_of = [&](int64_t st) { return smem + ((st % Cfg::STAGES) * KG + kg) * Cfg::STAGE; };
    // this group has a chunk in step c (its loads are issued only then)
    auto has_chunk = [&](int64_t c) { return c < steps && c * KG + kg < KB; };
    // every slot of the ring filled at once: with steps <= STAGES (the K range of a split
    // workgroup) all of the workgroup's operands are requested before the first wait
#pragma unroll
    for (int st = 0; st < Cfg::STAGES; ++st)
        if (has_chunk(st))
            load_stage<Cfg, SI>(stage_of(st), A, sA, B, M, N, K, m0, n0, kb0 + st * KG + kg, wl,
                                lane);

    auto k_loop = [&](auto big_tag) {
        constexpr bool BIG = decltype(big_tag)::value;
        for (int64_t st = 0; st < steps; ++st) {
            const int64_t kb = st * KG + kg;
            // this wave's loads of later steps already issued (the prologue's, then one step
            // per iteration): step st has landed once only those may be outstanding
            int later = 0;
#pragma unroll
            for (int d = 1; d < Cfg::STAGES; ++d) {
                const int64_t c = st + d;
                const bool issued = c < Cfg::STAGES || c <= st + Cfg::STAGES - 2;
                later += (issued && has_chunk(c)) ? 1 : 0;
            }
            if (later >= 3)
                wait_vm<3 * Cfg::MIN_LOADS>();
            else if (later == 2)
                wait_vm<2 * Cfg::MIN_LOADS>();
            else if (later == 1)
                wait_vm<Cfg::MIN_LOADS>();
            else
                wait_vm<0>();
            lds_barrier();   // step st visible to all; step st-1 fully read (its slot refills)
            const int64_t nxt = st - 1 + Cfg::STAGES;
            if (st >= 1 && has_chunk(nxt))
                load_stage<Cfg, SI>(stage_of(nxt), A, sA, B, M, N, K, m0, n0,
                                    kb0 + nxt * KG + kg, wl, lane);
            if (kb < KB) {
                const float sb = sbw.get(st);
                compute_chunk<Cfg, SI, BIG>(stage_of(st), fo, s_off, sb, acc);
            }
            if (Cfg::STAGES == 2)
                lds_barrier();
        }
    };
    if (sbf.any_above_one())
        k_loop(std::true_type{});
    else
        k_loop(std::false_type{});

    // sum the KG partial tiles in group order
    lds_barrier();
    float LDS* const red = (float LDS*)smem_raw;
    constexpr int PER_LANE = Cfg::FM * Cfg::FN * 4;
    if (kg > 0) {
#pragma unroll
        for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
            for (int j = 0; j < Cfg::FN; ++j)
                *(f32x4 LDS*)(red + (((kg - 1) * Cfg::NT + wl * 64 + lane) * PER_LANE +
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
                acc[i][j] += *(const f32x4 LDS*)(red + (((c - 1) * Cfg::NT + wl * 64 + lane) *
                                                            PER_LANE +
                                                        (i * Cfg::FN + j) * 4));
    // lane holds C[16i + 4g + r][16j + q] of the wave tile (or, split, the partial of it)
    float* const P = PARTIAL ? static_cast<float*>(Cout) + sp * M * N : nullptr;
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
                if (PARTIAL)
                    P[row * N + col] = acc[i][j][r];
                else if (OUT_BF16)
                    static_cast<__bf16*>(Cout)[row * N + col] = (__bf16)acc[i][j][r];
                else
                    static_cast<float*>(Cout)[row * N + col] = acc[i][j][r];
            }
        }
}

template <class Cfg, class SI, int KG>
static hipError_t launch_ksplit(const void* A_q, const void* sA_, const void* B_q,
                                const void* sB_, void* C, int64_t M, int64_t N, int64_t K,
                                int out_bf16, hipStream_t stream)
{
    const typename SI::T* sA = static_cast<const typename SI::T*>(sA_);
    const typename SI::T* sB = static_cast<const typename SI::T*>(sB_);
    const int64_t tiles = ((M + Cfg::BM - 1) / Cfg::BM) * (N / Cfg::BN);
    if (!grid_fits(tiles, Cfg::NT * KG))
        return hipErrorInvalidConfiguration;
    if (out_bf16)
        hipLaunchKernelGGL((gemm_fp8_blockscaled_ksplit_kernel<Cfg, SI, true, KG>),
                           dim3((unsigned)tiles), dim3(Cfg::NT * KG), 0, stream,
                           static_cast<const uint8_t*>(A_q), sA,
                           static_cast<const uint8_t*>(B_q), sB, C, M, N, K);
    else
        hipLaunchKernelGGL((gemm_fp8_blockscaled_ksplit_kernel<Cfg, SI, false, KG>),
                           dim3((unsigned)tiles), dim3(Cfg::NT * KG), 0, stream,
                           static_cast<const uint8_t*>(A_q), sA,
                           static_cast<const uint8_t*>(B_q), sB, C, M, N, K);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Narrow tiles for few output tiles (decode-like M, e.g. M = 128 with N = 7168: 56 tiles of
// 128x128 would leave most of the 256 CUs idle).  A workgroup owns a BM x 32 tile and its
// KW waves split the K chunks round-robin (wave w takes chunks w, w+KW, ...); each wave
// stages its own chunks in a private LDS ring, so the main loop has no workgroup barrier.
// The KW partial tiles are summed in LDS in wave order ((w0 + w1) + w2) + ..., a fixed
// order, so results are deterministic.  The per-chunk arithmetic is that of the wide
// kernel: f16 MFMA partials over the 128-K chunk, then acc = fma(P, sA*sB, acc).
template <int BM_, int KW_, int STAGES_, int BN_ = 32>
struct NarrowCfg {
    static constexpr int BM = BM_, BN = BN_, KW = KW_, STAGES = STAGES_;
    static constexpr int NT = 64 * KW;
    static constexpr int FM = BM / 16, FN = BN / 16;
    static constexpr int B_CHUNKS = BN / 16, B_ROWS_PER_LOAD = 1024 / BN;
    static constexpr int A_BYTES = BM * 128, B_BYTES = 128 * BN, S_BYTES = 256;
    static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    // the bf16 tile staged for the epilogue: rows of BN values plus 16 bytes
    static constexpr int STAGED_LD = BN * 2 + 16;
    static constexpr int SMEM = STAGES * STAGE > BM * STAGED_LD ? STAGES * STAGE : BM * STAGED_LD;
    static constexpr int A_LOADS = A_BYTES / 1024, B_LOADS = B_BYTES / 1024;
    static constexpr int LOADS = A_LOADS + B_LOADS + 1;   // per chunk and wave
    static constexpr int RED_LD = BN + 4;                  // padded row of the reduction
    static constexpr int LDS_BYTES = KW * STAGES * STAGE > KW * BM * RED_LD * 4
                                         ? KW * STAGES * STAGE
                                         : KW * BM * RED_LD * 4;
    static_assert(BM == 32 || BM == 64, "tile rows");
    static_assert(BN == 32 || BN == 64, "tile columns");
    static_assert(STAGES == 2 || STAGES == 3, "LDS ring depth");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity (160 KB per CU)");
    static_assert(LOADS < 64, "wait count range");
    // A: same row swizzle as the wide kernel.  B rows of 32 bytes (two 16-byte chunks): the
    // chunk is XORed with bit 5 of k, so the two 16-lane groups of one transposed read (k and
    // k+32) fall on disjoint banks.  B rows of 64 bytes (four chunks, four rows per 256-byte
    // bank line): the chunk is XORed with bit 2 of k and bit 5 of k, so the 16 rows one
    // transposed read serves per cycle (8t..8t+7 and 32+8t..32+8t+7) take 16 distinct
    // 16-byte bank slots.
    static __device__ __forceinline__ int a_swz(int row) { return (row >> 1) & 7; }
    static __device__ __forceinline__ int b_swz(int k)
    {
        return BN == 32 ? (k >> 5) & 1 : ((k >> 2) & 1) | (((k >> 5) & 1) << 1);
    }
};

// one wave fills its stage with chunk kb: A rows m0..m0+BM-1, B rows of the chunk for
// columns n0..n0+BN-1, and scale_A of the rows
template <class Cfg, class SI>
__device__ __forceinline__ void narrow_load(uint8_t LDS* stage, const uint8_t* __restrict__ A,
                                            const typename SI::T* __restrict__ sA,
                                            const uint8_t* __restrict__ B, int64_t M, int64_t N,
                                            int64_t K, int64_t m0, int64_t n0, int64_t kb,
                                            int lane)
{
#pragma unroll
    for (int u = 0; u < Cfg::A_LOADS; ++u) {
        const int row = u * 8 + (lane >> 3);
        const int c = (lane & 7) ^ Cfg::a_swz(row);
        int64_t gm = m0 + row;
        gm = gm < M ? gm : M - 1;
        dma_b128(A + gm * K + kb * 128 + c * 16, lds_addr(stage + u * 1024));
    }
    // B: instruction u covers k rows u*R..u*R+R-1 (R = 1024/BN); lane -> row u*R +
    // lane/(BN/16), physical 16-byte column lane%(BN/16) holding logical column p ^ swz(k)
#pragma unroll
    for (int u = 0; u < Cfg::B_LOADS; ++u) {
        const int k = u * Cfg::B_ROWS_PER_LOAD + lane / Cfg::B_CHUNKS;
        const int c = (lane % Cfg::B_CHUNKS) ^ Cfg::b_swz(k);
        dma_b128(B + (kb * 128 + k) * N + n0 + c * 16,
                 lds_addr(stage + Cfg::A_BYTES + u * 1024));
    }
    int64_t gm = m0 + lane;
    gm = gm < M ? gm : M - 1;
    SI::dma(sA + gm * (K / 128) + kb, lds_addr(stage + Cfg::A_BYTES + Cfg::B_BYTES));
}

template <class Cfg, class SI, bool OUT_BF16>
__global__ __launch_bounds__(Cfg::NT) void gemm_fp8_blockscaled_narrow_kernel(
    const uint8_t* __restrict__ A, const typename SI::T* __restrict__ sA,
    const uint8_t* __restrict__ B, const typename SI::T* __restrict__ sB,
    void* __restrict__ Cout, int64_t M, int64_t N, int64_t K)
{
    __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[Cfg::LDS_BYTES];
    uint8_t LDS* const smem = (uint8_t LDS*)smem_raw;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, q = lane & 15;

    // tiles: row tiles fastest, so the workgroups sharing a B column panel are neighbours;
    // consecutive ids of one XCD form one contiguous range (ids are dealt round-robin to
    // the 8 XCDs)
    const int64_t tiles_m = (M + Cfg::BM - 1) / Cfg::BM;
    const int64_t G = (int64_t)gridDim.x;
    int64_t pid = blockIdx.x;
    if (G % 8 == 0)
        pid = (pid % 8) * (G / 8) + pid / 8;
    const int64_t m0 = (pid % tiles_m) * Cfg::BM, n0 = (pid / tiles_m) * Cfg::BN;
    const int64_t KB = K / 128, NB = N / 128, nb = n0 / 128;

    uint8_t LDS* const ring = smem + wave * (Cfg::STAGES * Cfg::STAGE);
    const FragOffsets<Cfg> fo(0, 0, g, q);
    const int s_off = Cfg::A_BYTES + Cfg::B_BYTES + 4 * g * 4;

    f32x4 acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // this wave's chunks: kb = wave + c*KW, c < nc
    const int64_t nc = wave < KB ? (KB - wave + Cfg::KW - 1) / Cfg::KW : 0;
    ScaleBWalk<SI> sbw(sB + wave * NB + nb, Cfg::KW * NB, nc, lane);
    const ScaleBFlag<SI> sbf(sB + wave * NB + nb, Cfg::KW * NB, nc, lane);
#pragma unroll
    for (int st = 0; st < Cfg::STAGES - 1; ++st)
        if (st < nc)
            narrow_load<Cfg, SI>(ring + st * Cfg::STAGE, A, sA, B, M, N, K, m0, n0,
                             wave + st * Cfg::KW, lane);
    auto k_loop = [&](auto big_tag) {
        constexpr bool BIG = decltype(big_tag)::value;
        for (int64_t c = 0; c < nc; ++c) {
            // chunk c has landed once only the next chunk's loads may be outstanding; every
            // LDS read of the previous chunk has returned (its stage is refilled next)
            if (Cfg::STAGES == 3 && c + 1 < nc)
                wait_vm<Cfg::LOADS>();
            else
                wait_vm<0>();
            __builtin_amdgcn_s_waitcnt(0xC07F);
            asm volatile("" ::: "memory");
            const int64_t nxt = c + Cfg::STAGES - 1;
            if (nxt < nc)
                narrow_load<Cfg, SI>(ring + (nxt % Cfg::STAGES) * Cfg::STAGE, A, sA, B, M, N, K, m0,
                                 n0, wave + nxt * Cfg::KW, lane);
            const float sb = sbw.get(c);
            compute_chunk<Cfg, SI, BIG>(ring + (c % Cfg::STAGES) * Cfg::STAGE, fo, s_off, sb,
                                         acc);
        }
    };
    if (sbf.any_above_one())
        k_loop(std::true_type{});
    else
        k_loop(std::false_type{});

    // sum the KW partial tiles in wave order, then store coalesced
    __syncthreads();
    float LDS* const red = (float LDS*)smem_raw;
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[(wave * Cfg::BM + 16 * i + 4 * g + r) * Cfg::RED_LD + 16 * j + q] =
                    acc[i][j][r];
    __syncthreads();
#pragma unroll
    for (int e0 = 0; e0 < Cfg::BM * Cfg::BN; e0 += Cfg::NT) {
        const int e = e0 + (int)threadIdx.x;
        const int row = e / Cfg::BN, col = e % Cfg::BN;
        float v = red[row * Cfg::RED_LD + col];
#pragma unroll
        for (int w = 1; w < Cfg::KW; ++w)
            v += red[(w * Cfg::BM + row) * Cfg::RED_LD + col];
        const int64_t grow = m0 + row;
        if (grow < M) {
            if (OUT_BF16)
                static_cast<__bf16*>(Cout)[grow * N + n0 + col] = (__bf16)v;
            else
                static_cast<float*>(Cout)[grow * N + n0 + col] = v;
        }
    }
}

template <class Cfg, class SI>
static hipError_t launch_narrow(const void* A_q, const void* sA_, const void* B_q,
                                const void* sB_, void* C, int64_t M, int64_t N, int64_t K,
                                int out_bf16, hipStream_t stream)
{
    const typename SI::T* sA = static_cast<const typename SI::T*>(sA_);
    const typename SI::T* sB = static_cast<const typename SI::T*>(sB_);
    const int64_t tiles = ((M + Cfg::BM - 1) / Cfg::BM) * (N / Cfg::BN);
    if (!grid_fits(tiles, Cfg::NT))
        return hipErrorInvalidConfiguration;
    if (out_bf16)
        hipLaunchKernelGGL((gemm_fp8_blockscaled_narrow_kernel<Cfg, SI, true>),
                           dim3((unsigned)tiles), dim3(Cfg::NT), 0, stream,
                           static_cast<const uint8_t*>(A_q), sA,
                           static_cast<const uint8_t*>(B_q), sB, C, M, N, K);
    else
        hipLaunchKernelGGL((gemm_fp8_blockscaled_narrow_kernel<Cfg, SI, false>),
                           dim3((unsigned)tiles), dim3(Cfg::NT), 0, stream,
                           static_cast<const uint8_t*>(A_q), sA,
                           static_cast<const uint8_t*>(B_q), sB, C, M, N, K);
    return hipGetLastError();
}

template <class Cfg>
static hipError_t launch_fused(const void* A_q, const float* sA, const void* B_q, const float* sB,
                               void* C, void* Cq, float* sC, int64_t M, int64_t N, int64_t K,
                               hipStream_t stream)
{
    const int64_t tiles = ((M + Cfg::BM - 1) / Cfg::BM) * ((N + Cfg::BN - 1) / Cfg::BN);
    if (!grid_fits(tiles, Cfg::NT))
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemm_fp8_blockscaled_kernel<Cfg, ScaleIn<false>, true, true>), dim3((unsigned)tiles),
                       dim3(Cfg::NT), 0, stream, static_cast<const uint8_t*>(A_q), sA,
                       static_cast<const uint8_t*>(B_q), sB, C, M, N, K, (int64_t)0, N,
                       static_cast<uint8_t*>(Cq), sC);
    return hipGetLastError();
}

#ifndef FGQ_LARGE_CFG
#define FGQ_LARGE_CFG 256, 128, 4, 2, 2
#endif
#ifndef FGQ_SMALL_CFG
#define FGQ_SMALL_CFG 128, 128, 2, 2, 2
#endif
using CfgLarge = GemmCfg<FGQ_LARGE_CFG>;
using CfgSmall = GemmCfg<FGQ_SMALL_CFG>;
#ifndef FGQ_NARROW_CFG
#define FGQ_NARROW_CFG 64, 4, 2
#endif
using CfgNarrow = NarrowCfg<FGQ_NARROW_CFG>;
#ifndef FGQ_NARROW64_CFG
#define FGQ_NARROW64_CFG 64, 4, 2, 64
#endif
using CfgNarrow64 = NarrowCfg<FGQ_NARROW64_CFG>;
#ifndef FGQ_SKINNY_CFG
#define FGQ_SKINNY_CFG 128, 32, 4, 1, 2
#endif
#ifndef FGQ_SKINNY_KG
#define FGQ_SKINNY_KG 3
#endif
using CfgSkinny = GemmCfg<FGQ_SKINNY_CFG>;

// compute units of the current device (queried once per device)
int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return 0;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0)
            return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (dev < 64)
        cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// Wave quantization of the 256x128 tiles (one resident workgroup per CU): when the tiles
// fill R whole rounds of the CUs plus a last round at most half full, and that remainder is
// whole tile columns, the remainder's columns run as 128x128 tiles instead -- twice as many
// tiles of half the work, one round of half the duration -- so the last round has no idle
// half.  Returns the first column of that tail, or N when the split does not apply.
static int64_t tail_split_column(int64_t M, int64_t N)
{
    const int cus = device_cus();
    const int64_t tm = (M + CfgLarge::BM - 1) / CfgLarge::BM, tn = N / CfgLarge::BN;
    if (cus <= 0 || tm * tn <= cus)
        return N;
    const int64_t r = (tm * tn) % cus;
    if (r == 0 || 2 * r > cus || r % tm != 0)
        return N;
    return N - (r / tm) * CfgLarge::BN;
}

template <class SI>
static hipError_t launch_gemm(const void* A_q, const void* sA, const void* B_q, const void* sB,
                              void* C, int64_t M, int64_t N, int64_t K, int out_bf16,
                              int variant, hipStream_t stream)
{
    if (variant == GEMM_AUTO && M >= 256) {
        const int64_t split = tail_split_column(M, N);
        if (split < N) {
            const int64_t tiles_l = ((M + CfgLarge::BM - 1) / CfgLarge::BM) * (split / CfgLarge::BN);
            const int64_t tiles_s =
                ((M + CfgSmall::BM - 1) / CfgSmall::BM) * ((N - split) / CfgSmall::BN);
            if (!grid_fits(tiles_l, CfgLarge::NT) || !grid_fits(tiles_s, CfgSmall::NT))
                return hipErrorInvalidConfiguration;
            const hipError_t e = launch_cfg<CfgLarge, SI>(A_q, sA, B_q, sB, C, M, N, K, out_bf16,
                                                          stream, 0, split);
            if (e != hipSuccess)
                return e;
            return launch_cfg<CfgSmall, SI>(A_q, sA, B_q, sB, C, M, N, K, out_bf16, stream,
                                            split, N);
        }
    }
    if (variant == GEMM_AUTO) {
        // Wide tiles while they fill the 256 CUs at least once.  Below that (measured back to
        // back over M = 1..640, N = 256..7168, K = 256..4096): the narrow 64x32 tiles (one
        // workgroup per CU, each wave a whole tile over its own chunks, so no operand is
        // converted twice) while they fit one round of the CUs; else the narrow 64x64 tiles
        // (half the workgroups, each operand still converted once) while they fit two rounds,
        // except for M <= 128 with at most two K chunks, where the skinny tiles are quicker;
        // else 128x128 wide tiles (one round).
        const int64_t tiles_large = ((M + CfgLarge::BM - 1) / CfgLarge::BM) * (N / CfgLarge::BN);
        const int64_t tiles_small = ((M + CfgSmall::BM - 1) / CfgSmall::BM) * (N / CfgSmall::BN);
        const int64_t tiles_n32 = ((M + CfgNarrow::BM - 1) / CfgNarrow::BM) * (N / CfgNarrow::BN);
        const int64_t tiles_n64 =
            ((M + CfgNarrow64::BM - 1) / CfgNarrow64::BM) * (N / CfgNarrow64::BN);
        const int cus = device_cus() > 0 ? device_cus() : 256;
        variant = (M >= 256 && tiles_large >= 256) ? GEMM_WIDE_256x128
                  : tiles_small >= 256             ? GEMM_WIDE_128x128
                  : tiles_n32 <= cus               ? GEMM_NARROW
                  : M <= 128 && K <= 256           ? GEMM_SKINNY
                  : tiles_n64 <= 2 * cus           ? GEMM_NARROW_64x64
                                                   : GEMM_WIDE_128x128;
    }
    switch (variant) {
    case GEMM_WIDE_256x128:
        return launch_cfg<CfgLarge, SI>(A_q, sA, B_q, sB, C, M, N, K, out_bf16, stream);
    case GEMM_WIDE_128x128:
        return launch_cfg<CfgSmall, SI>(A_q, sA, B_q, sB, C, M, N, K, out_bf16, stream);
    case GEMM_NARROW:
        return launch_narrow<CfgNarrow, SI>(A_q, sA, B_q, sB, C, M, N, K, out_bf16, stream);
    case GEMM_NARROW_64x64:
        return launch_narrow<CfgNarrow64, SI>(A_q, sA, B_q, sB, C, M, N, K, out_bf16, stream);
    case GEMM_SKINNY:
        return launch_ksplit<CfgSkinny, SI, FGQ_SKINNY_KG>(A_q, sA, B_q, sB, C, M, N, K, out_bf16,
                                                           stream);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_fp8_blockscaled(const void* A_q, const float* sA, const void* B_q,
                                       const float* sB, void* C, int64_t M, int64_t N,
                                       int64_t K, int out_bf16, int variant,
                                       hipStream_t stream)
{
    return launch_gemm<ScaleIn<false>>(A_q, sA, B_q, sB, C, M, N, K, out_bf16, variant, stream);
}

hipError_t launch_gemm_fp8_blockscaled_ue8m0(const void* A_q, const uint8_t* sA,
                                             const void* B_q, const uint8_t* sB, void* C,
                                             int64_t M, int64_t N, int64_t K, int out_bf16,
                                             int variant, hipStream_t stream)
{
    return launch_gemm<ScaleIn<true>>(A_q, sA, B_q, sB, C, M, N, K, out_bf16, variant, stream);
}

hipError_t launch_gemm_fp8_blockscaled_quant(const void* A_q, const float* sA, const void* B_q,
                                             const float* sB, void* C, void* Cq, float* sC,
                                             int64_t M, int64_t N, int64_t K, hipStream_t stream)
{
    // Few output tiles (the 128x128 tiles do not cover the CUs once): the fused kernel's tiles
    // would leave CUs idle, so the GEMM family the shape calls for runs first and the
    // activation quantizer then codes the bf16 C it wrote -- two launches with the same
    // results (the codes are the quantization of that C), measured 24.4 -> 13.5 us at
    // 128x7168x2048 and 23.7 -> 9.2 us at 1x7168x2048.
    const int64_t tiles_small = ((M + CfgSmall::BM - 1) / CfgSmall::BM) * (N / CfgSmall::BN);
    if (tiles_small < 256) {
        const hipError_t e = launch_gemm<ScaleIn<false>>(A_q, sA, B_q, sB, C, M, N, K, 1,
                                                         GEMM_AUTO, stream);
        if (e != hipSuccess)
            return e;
        return launch_quant_act_1x128(C, Cq, sC, M, N, stream);
    }
    // whole 128-column groups per workgroup: the wide tiles only
    const int64_t tiles_large = ((M + CfgLarge::BM - 1) / CfgLarge::BM) * (N / CfgLarge::BN);
    if (M >= 256 && tiles_large >= 256)
        return launch_fused<CfgLarge>(A_q, sA, B_q, sB, C, Cq, sC, M, N, K, stream);
    return launch_fused<CfgSmall>(A_q, sA, B_q, sB, C, Cq, sC, M, N, K, stream);
}

// ---------------------------------------------------------------------------------------
// K split across workgroups (stream-K style, for shapes with few output tiles such as the
// decode-like M <= 128).  Pass 1 runs splits x tiles workgroups of the K-group kernel with
// 128x128 tiles (8 waves: a 2x2 grid of 64x64 wave tiles in each of two K groups), each over a
// contiguous range of K chunks, writing fp32 partial tiles to the workspace slices [splits][M][N];
// pass 2 sums the slices in slice order ((p0 + p1) + p2) + ..., so results are repeatable bit
// for bit, and writes C.  No atomics: every workspace element is written by exactly one
// workgroup of pass 1 and read by pass 2, which the stream orders after it.
using CfgSplit = GemmCfg<128, 128, 2, 2, 2>;
constexpr int SPLIT_KG = 2;
constexpr int SPLIT_MAX = kSplitMax;

// sum of the partial slices, 8 consecutive elements per thread (M*N is a multiple of 128):
// all slices' loads are issued before the first add, then added in slice order
template <bool OUT_BF16, int S>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P,
                                                            void* __restrict__ C, int64_t MN)
{
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (i >= MN)
        return;
    f32x4 part[S][2];
#pragma unroll
    for (int sp = 0; sp < S; ++sp) {
        part[sp][0] = __builtin_nontemporal_load((const f32x4*)(P + sp * MN + i));
        part[sp][1] = __builtin_nontemporal_load((const f32x4*)(P + sp * MN + i + 4));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        f32x4 v = part[0][h];
#pragma unroll
        for (int sp = 1; sp < S; ++sp)
            v += part[sp][h];
        if (OUT_BF16) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            *(bf16x4*)(static_cast<__bf16*>(C) + i + 4 * h) =
                bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
        } else {
            *(f32x4*)(static_cast<float*>(C) + i + 4 * h) = v;
        }
    }
}

template <bool OUT_BF16, int S = 2>
static void launch_reduce(const float* ws, void* C, int64_t MN, int splits, int64_t blocks,
                          hipStream_t stream)
{
    if constexpr (S < SPLIT_MAX) {
        if (splits != S)
            return launch_reduce<OUT_BF16, S + 1>(ws, C, MN, splits, blocks, stream);
    }
    hipLaunchKernelGGL((splitk_reduce_kernel<OUT_BF16, S>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, ws, C, MN);
}

// K splits the workspace path uses for a shape (1 = none).  Two launches cost ~8 us of fixed
// time more than one on this GPU (measured: the reduction pass alone adds 8 us at
// 128x7168x2048), so the split pays only where the unsplit kernels would walk long K chains
// on few workgroups: 128 or more K chunks with 128x128 tiles covering at most half of the
// CUs (back to back: 128x512x32768 72 -> 29 us, 128x1024x16384 31 -> 23 us,
// 512x1024x16384 39 -> 33 us; with 32-64 chunks the unsplit kernels were as fast or faster).
// Then the largest power of two (<= SPLIT_MAX) whose workgroups fit one round of the CUs with
// at least 8 chunks each.
int gemm_splitk_plan(int64_t M, int64_t N, int64_t K)
{
    const int cus = device_cus() > 0 ? device_cus() : 256;
    const int64_t tiles = ((M + 127) / 128) * (N / 128), KB = K / 128;
    if (tiles <= 0 || 2 * tiles > cus || KB < 128)
        return 1;
    int sp = 1;
    while (2 * sp <= SPLIT_MAX && tiles * 2 * sp <= cus && KB / (2 * sp) >= 8)
        sp *= 2;
    return sp;
}

template <class SI>
static hipError_t launch_splitk(const void* A_q, const void* sA_, const void* B_q,
                                const void* sB_, void* C, int64_t M, int64_t N, int64_t K,
                                int out_bf16, int splits, float* ws, hipStream_t stream)
{
    const typename SI::T* sA = static_cast<const typename SI::T*>(sA_);
    const typename SI::T* sB = static_cast<const typename SI::T*>(sB_);
    const int64_t tiles = ((M + CfgSplit::BM - 1) / CfgSplit::BM) * (N / CfgSplit::BN);
    const int64_t MN = M * N;
    const int64_t rblocks = (MN / 8 + 255) / 256;
    if (!grid_fits(tiles * splits, CfgSplit::NT * SPLIT_KG) || !grid_fits(rblocks, 256))
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemm_fp8_blockscaled_ksplit_kernel<CfgSplit, SI, false, SPLIT_KG, true>),
                       dim3((unsigned)(tiles * splits)), dim3(CfgSplit::NT * SPLIT_KG), 0,
                       stream, static_cast<const uint8_t*>(A_q), sA,
                       static_cast<const uint8_t*>(B_q), sB, ws, M, N, K, (int64_t)splits);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (out_bf16)
        launch_reduce<true>(ws, C, MN, splits, rblocks, stream);
    else
        launch_reduce<false>(ws, C, MN, splits, rblocks, stream);
    return hipGetLastError();
}

hipError_t launch_gemm_fp8_blockscaled_splitk(const void* A_q, const float* sA, const void* B_q,
                                              const float* sB, void* C, int64_t M, int64_t N,
                                              int64_t K, int out_bf16, int splits, float* ws,
                                              hipStream_t stream)
{
    if (splits <= 1)
        return launch_gemm<ScaleIn<false>>(A_q, sA, B_q, sB, C, M, N, K, out_bf16, GEMM_AUTO,
                                           stream);
    return launch_splitk<ScaleIn<false>>(A_q, sA, B_q, sB, C, M, N, K, out_bf16, splits, ws,
                                         stream);
}

// ---------------------------------------------------------------------------------------
// For callers that cannot allocate (fgq_gemm_fp8_blockscaled_noalloc): the K-split partials
// in a file-scope device array instead of a caller's workspace.  Every GPU the library runs
// on holds its own copy (kNoallocScratchBytes) until the process ends; every call on a GPU
// shares it, so calls that overlap in time on one GPU race.  Nothing in it has to start at
// zero: pass 1 writes every partial element that pass 2 reads.
static __device__ __align__(256) float scratch[kNoallocScratchBytes / 4];

// the array's device address on the current GPU, looked up on the first call on each device
// with that device current (the host-side name of a __device__ array is only a stand-in)
static float* scratch_ptr()
{
    static std::atomic<float*> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return nullptr;
    float* p = cache[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q)
        return nullptr;
    cache[dev].store(static_cast<float*>(q), std::memory_order_release);
    return static_cast<float*>(q);
}

hipError_t launch_gemm_fp8_blockscaled_noalloc(const void* A_q, const float* sA, const void* B_q,
                                               const float* sB, void* C, int64_t M, int64_t N,
                                               int64_t K, int out_bf16, int splits,
                                               hipStream_t stream)
{
    if (splits > 1 && (int64_t)splits * M * N * 4 > kNoallocScratchBytes)
        return hipErrorInvalidValue;
    float* const ws = scratch_ptr();
    if (!ws)
        return hipErrorInvalidSymbol;
    return launch_gemm_fp8_blockscaled_splitk(A_q, sA, B_q, sB, C, M, N, K, out_bf16, splits,
                                              ws, stream);
}

}  // namespace fgq
