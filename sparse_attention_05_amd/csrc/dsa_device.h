// dsa_device.h -- device-side helpers shared by the DSA kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v8f __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// 16x16x128 fp8 (OCP e4m3fn) x fp8 -> fp32 MFMA.  Zero scale operands select the unscaled
// v_mfma_f32_16x16x128_f8f6f4.  Lane l supplies row (A) / column (B) l%16 and 32 bytes of
// K; A and B use the same K assignment, so a kernel only has to load both operands with
// one lane->K mapping.  Output: lane l holds C[4*(l/16) + i][l%16], i = 0..3.
__device__ __forceinline__ v4f mfma_f8(const v8i& a, const v8i& b, const v4f& c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16x16x32 bf16 MFMA, fp32 accumulate.  Lane l supplies row/column l%16 and 8 elements
// of K (K group l/16); same output layout as above.
__device__ __forceinline__ v4f mfma_bf16(const v8bf& a, const v8bf& b, const v4f& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_bf16x8(const u32x4& v) { return __builtin_bit_cast(v8bf, v); }

__device__ __forceinline__ v8i as_i8(const u32x4& lo, const u32x4& hi)
{
    v8i r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return bf16_bits(lo) | (bf16_bits(hi) << 16);
}

// Order-preserving image of an fp32 score: larger float -> larger uint32, -0 == +0.
__device__ __forceinline__ uint32_t score_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// max over lanes {l, l ^ 32} / {l, l ^ 16} on the lane-swap instructions (VALU, no LDS)
__device__ __forceinline__ float max_xor32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Reduce-scatter helpers on gfx950's lane-swap instructions.
// fold32(x, y): lanes 0-31 get x summed over lanes l and l+32, lanes 32-63 get y so summed.
__device__ __forceinline__ float fold32(float x, float y)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// fold16(x, y): even 16-lane rows get x summed over the row pair (0,1) or (2,3), odd rows y.
__device__ __forceinline__ float fold16(float x, float y)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ unsigned long long lanemask_lt(int lane)
{
    return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4s lds_v4s_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

// Direct global->LDS load of 16 bytes per lane: lane l's bytes land at LDS byte address
// lds_dst + 16 l (lds_dst wave-uniform, passed in M0).  Written as one asm statement because
// the compiler cannot tell that the LDS reads which follow it (of the other tile buffer) do not
// touch the bytes in flight, and would otherwise wait for the load before each of them.  The
// statement has no register results; completion is awaited explicitly (s_waitcnt 0 and a
// barrier) before the destination buffer is read.  M0 is listed as clobbered (the compiler
// notes that it is a reserved register): each statement loads it itself right before the
// load, and on gfx950 nothing else in these kernels keeps a value in M0.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_dst)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds_dst)
                 : "memory", "m0");
}
// the same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte offset
__device__ __forceinline__ void dma16_s(uint32_t voff, const void* sbase, uint32_t lds_dst)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds_dst)
                 : "memory", "m0");
}
// Transposing LDS read of 16-bit elements: within each 16-lane group, lane i supplies the
// address of 4 consecutive elements (row i/4 of a 4-row block, elements 4 (i%4) .. +3) and
// receives column i of that 4 x 16 block (its 4 rows).
__device__ __forceinline__ u32x2 ds_read_tr(const uint8_t* p)
{
    const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(p));
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

}  // namespace dsa
