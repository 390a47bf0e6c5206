// gemm_common.hpp -- gfx950 building blocks shared by the GEMM kernels: vector types, the
// E4M3 -> f16 operand conversion, explicit wait counts, the LDS-only barrier and the
// direct-to-LDS loads.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgq {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// 8 E4M3 codes (two dwords) -> 8 f16, exact
__device__ __forceinline__ f16x8 e4m3x8_to_f16(int w0, int w1)
{
    const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
    const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
    const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
    const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
#define LDS __attribute__((address_space(3)))

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt [6:4] and
// lgkmcnt [11:8] left at their maxima, i.e. not waited on)
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// workgroup barrier that orders LDS accesses only (no wait on outstanding global loads)
__device__ __forceinline__ void lds_barrier()
{
    // lgkmcnt(0): this wave's LDS reads have returned (vmcnt/expcnt not waited on)
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One direct-to-LDS load: 16 bytes per lane from gptr to LDS [lds + 16*lane] (or 4 bytes
// per lane to [lds + 4*lane]).  Written as inline asm so the compiler's wait-count pass
// does not see an outstanding LDS write and does not put a vmcnt(0) in front of every LDS
// read of the other stage; the pipeline waits for these loads explicitly (wait_vm).
// M0 holds the LDS base; one wait state separates the M0 write from its use.
__device__ __forceinline__ void dma_b128(const void* gptr, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(const void* gptr, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(gptr), "s"(lds)
                 : "memory", "m0");
}

// one byte per lane, zero-extended into the lane's dword slot [lds + 4*lane]
__device__ __forceinline__ void dma_u8(const void* gptr, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ubyte %0, off"
                 :
                 : "v"(gptr), "s"(lds)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t LDS* p)
{
    return (uint32_t)(uintptr_t)p;
}

}  // namespace fgq
