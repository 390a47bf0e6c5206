// fgq_device.hpp -- gfx950 device helpers shared by the quantization kernels.
//
// Quantization rule (page "Fine-Grained FP8/FP4 Quantization", sections "Scaling
// Granularities" and "DeepGEMM: Tile-wise and Block-wise Scaling"; E4M3 range from its
// table "UE8M0 vs E4M3 Scale Formats"): a group (1x128 activation tile or 128x128 weight
// block) shares the fp32 dequantization scale s = amax/448; each element is stored as the
// E4M3 (OCP E4M3FN) code of the fp32 quotient x/s, rounded to nearest-even.
//
// How the device computes it:
//   * amax is an exact integer max over the bf16 magnitude bits (sign cleared): for
//     non-NaN values the unsigned order of those bits is the order of |x|;
//   * s = amax/448 is reached by Markstein's correction with the rounded constant 1/448
//     (IEEE divide for amax < 2^-100), r = 1/s by v_rcp_f32 plus one Newton step, once per
//     group and lane;
//   * per element, y = fl32(x/s) is reached from q = x*r with one exact-remainder
//     correction (Markstein's quotient correction: e = q*s - x is exact by FMA, then
//     y = q - e*r).  The negated remainder keeps the sign of zero: -0 stays -0.  Groups
//     whose s is below 2^-96 (a reciprocal near the fp32 overflow) take a plain divide;
//   * y is converted by v_cvt_pk_fp8_f32 (gfx950: OCP E4M3FN, nearest-even).  |y| never
//     exceeds 448*(1+2^-8) < 464, so the convert's overflow-to-NaN never triggers and no
//     clamp is needed.
// Every possible (x, amax) pair is run through this path by the device domain-sweep test
// and compared with the CPU reference bit for bit.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef FGQ_FAST_SCALE
#define FGQ_FAST_SCALE 1
#endif

namespace fgq {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// max over the 8 bf16 magnitudes held in one 16-byte vector, as 16-bit magnitude bits
__device__ __forceinline__ uint32_t absmax_bits8(u32x4 v)
{
    u16x2 a = __builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu);
    u16x2 b = __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu);
    u16x2 c = __builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu);
    u16x2 d = __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu);
    u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                        __builtin_elementwise_max(c, d));
    return m.x > m.y ? (uint32_t)m.x : (uint32_t)m.y;
}

// max across the 16 lanes of a DPP row (row_ror 8, 4, 2, 1): every lane gets the result
__device__ __forceinline__ uint32_t row16_max(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));
    return v;
}

// max across all 64 lanes (result valid in every lane)
__device__ __forceinline__ uint32_t wave_max(uint32_t v)
{
    v = row16_max(v);
    uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

struct GroupScale {
    float s;    // stored dequantization scale amax/448
    float r;    // 1/s (0 when s == 0)
    bool slow;  // s tiny: per-element IEEE divide instead of the reciprocal path
};

__device__ __forceinline__ GroupScale group_scale(uint32_t amax_bits16)
{
    float amax = __uint_as_float(amax_bits16 << 16);
    GroupScale g;
#if FGQ_FAST_SCALE
    // s = fl32(amax/448) by Markstein's correction with the rounded constant 1/448 (exact
    // for normal s; tiny amax takes the IEEE divide), r = 1/s by v_rcp_f32 and one Newton
    // step.  Both are checked over every bf16 amax by the device domain sweep.
    if (amax >= 0x1p-100f) {
        const float c = 1.0f / 448.0f;
        const float q0 = amax * c;
        const float e = __builtin_fmaf(-q0, 448.0f, amax);
        g.s = __builtin_fmaf(e, c, q0);
    } else {
        g.s = amax / 448.0f;
    }
    {
        const float r0 = __builtin_amdgcn_rcpf(g.s);
        const float er = __builtin_fmaf(-g.s, r0, 1.0f);
        g.r = (g.s == 0.0f) ? 0.0f : __builtin_fmaf(er, r0, r0);
    }
#else
    g.s = amax / 448.0f;
    g.r = (g.s == 0.0f) ? 0.0f : 1.0f / g.s;
#endif
    g.slow = (g.s != 0.0f) && (g.s < 0x1p-96f);
    return g;
}

// fl32(x / s) for one element, reciprocal path (groups with s == 0 or s >= 2^-96)
__device__ __forceinline__ float quotient_fast(float x, const GroupScale& g)
{
    float q = x * g.r;
    float e = __builtin_fmaf(q, g.s, -x);   // exact: q*s - x
    return __builtin_fmaf(-e, g.r, q);      // q - e*r, rounded once
}

// quantize 8 bf16 values (one 16-byte vector) to 8 E4M3 codes (one 8-byte vector)
template <bool SLOW>
__device__ __forceinline__ u32x2 quantize8_impl(u32x4 v, const GroupScale& g)
{
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float x[4] = {__uint_as_float(w[2 * h] << 16), __uint_as_float(w[2 * h] & 0xFFFF0000u),
                      __uint_as_float(w[2 * h + 1] << 16),
                      __uint_as_float(w[2 * h + 1] & 0xFFFF0000u)};
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            y[i] = SLOW ? x[i] / g.s : quotient_fast(x[i], g);
        int packed = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        packed = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], packed, true);
        out[h] = (uint32_t)packed;
    }
    return u32x2{out[0], out[1]};
}

__device__ __forceinline__ u32x2 quantize8(u32x4 v, const GroupScale& g)
{
    u32x2 q = quantize8_impl<false>(v, g);
    if (__builtin_expect(g.slow, 0))        // divergent only in groups with a tiny scale
        q = quantize8_impl<true>(v, g);
    return q;
}

// ---------------------------------------------------------------------------------------
// UE8M0 (power-of-two) group scales: the stored byte e stands for s = 2^(e-127) (page
// "Fine-Grained FP8/FP4 Quantization", section "Blackwell: Native Block Scaling"); e is the
// smallest exponent with 448*s >= amax, so no code saturates.  With amax = 1.f * 2^E in
// bf16 (E from the exponent field, f from the 7 mantissa bits): 448 = 1.75 * 2^8, so
// 448 * 2^(E-8) covers amax exactly when f <= 1.75 (mantissa bits <= 0x60), otherwise one
// more power of two is needed; e = E - 8 (+1) + 127, clamped at 0 for amax below 448*2^-127
// (tiny and all-zero groups).  The quotient x/s is x * 2^(127-e): a product with an exact
// power of two, so it is the correctly rounded quotient itself.
// ---------------------------------------------------------------------------------------
struct Pow2Scale {
    uint32_t e;   // stored exponent byte
    float r;      // 1/s = 2^(127-e), a normal float for every e this rule gives (0..247)
};

__device__ __forceinline__ Pow2Scale pow2_scale(uint32_t amax_bits16)
{
    const int ef = (int)((amax_bits16 >> 7) & 0xFF);
    int e = ef - 8 + ((amax_bits16 & 0x7F) > 0x60 ? 1 : 0);
    e = e < 0 ? 0 : e;
    Pow2Scale p;
    p.e = (uint32_t)e;
    p.r = __uint_as_float((uint32_t)(254 - e) << 23);
    return p;
}

// quantize 8 bf16 values with a power-of-two scale
__device__ __forceinline__ u32x2 quantize8_pow2(u32x4 v, const Pow2Scale& p)
{
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float y0 = __uint_as_float(w[2 * h] << 16) * p.r;
        const float y1 = __uint_as_float(w[2 * h] & 0xFFFF0000u) * p.r;
        const float y2 = __uint_as_float(w[2 * h + 1] << 16) * p.r;
        const float y3 = __uint_as_float(w[2 * h + 1] & 0xFFFF0000u) * p.r;
        int packed = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
        packed = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, packed, true);
        out[h] = (uint32_t)packed;
    }
    return u32x2{out[0], out[1]};
}

// Scale policies for the quantization kernels: fp32 scale amax/448, or UE8M0 exponent
struct ScaleF32 {
    typedef float stored_t;
    GroupScale g;
    __device__ __forceinline__ explicit ScaleF32(uint32_t amax_bits16)
        : g(group_scale(amax_bits16)) {}
    __device__ __forceinline__ u32x2 quant(u32x4 v) const { return quantize8(v, g); }
    __device__ __forceinline__ float stored() const { return g.s; }
};
struct ScaleUE8M0 {
    typedef uint8_t stored_t;
    Pow2Scale p;
    __device__ __forceinline__ explicit ScaleUE8M0(uint32_t amax_bits16)
        : p(pow2_scale(amax_bits16)) {}
    __device__ __forceinline__ u32x2 quant(u32x4 v) const { return quantize8_pow2(v, p); }
    __device__ __forceinline__ uint8_t stored() const { return (uint8_t)p.e; }
};

}  // namespace fgq
