// quantize.hip -- fp8 preparation of the lightning indexer's inputs on gfx950, and the
// decode cache append.
//
// The indexer runs in FP8 (gxzdkb DSA explainer, section 秘密武器：DSA; 《DeepSeek-V3.2-Exp
// 模型优势与 DSA 工作原理》 §3): every 128-wide query or key vector is stored as e4m3fn codes
// with one fp32 scale.  scale = amax / 448 (1 for an all-zero vector); code = the e4m3fn value
// nearest to clamp(x / scale, -448, 448), the quotient rounded to fp32, ties to even.  A
// decode step first appends the new token to the packed caches (gxzdkb explainer, section
// 原始 Attention 的计算逻辑: the cache is updated, then the step attends).
//
// Memory-bound: 16 lanes per vector, each lane 8 consecutive elements (32 or 16 bytes in,
// 8 bytes of codes out, coalesced across the wave); the amax is reduced across the 16 lanes by
// rotations within the lane row, and the codes come from gfx950's pack conversion to OCP
// e4m3fn (round to nearest even), checked against the format's rounding on every fp32 value
// of magnitude at most 448.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int QT = 256;                        // threads per workgroup: 16 vectors

// maximum over the 16 lanes of a lane row (lanes 16r .. 16r + 15): rotations by 8, 4, 2 and 1
// lanes within the row (data-parallel-primitive moves, no LDS)
__device__ __forceinline__ float row16_max(float v)
{
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false)));
    return v;
}

struct Quant8 {
    u32x2 codes;                               // this lane's 8 codes, little-endian
    float scale;
};

// The 16 lanes of a vector group (lane part p holds elements 8p .. 8p + 7) quantise their
// vector together; every lane of the wave must take part (the amax crosses lanes).
__device__ __forceinline__ Quant8 quantize8(const float (&x)[8])
{
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
    amax = row16_max(amax);
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = fminf(fmaxf(x[j] / s, -448.0f), 448.0f);
    // codes of elements 4i .. 4i + 3 in word i, element 4i + m in byte m
    uint32_t w[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * i], y[4 * i + 1], 0, false);
        w[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4 * i + 2], y[4 * i + 3], lo, true);
    }
    return Quant8{u32x2{w[0], w[1]}, s};
}

// elements e0 .. e0 + 7 of x (fp32, or bf16 bits), 16-byte aligned
template <bool BF16>
__device__ __forceinline__ void load8(const void* x, int64_t e0, float (&v)[8])
{
    if constexpr (BF16) {
        const u32x4 r = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + e0);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = __uint_as_float(((r[j >> 1] >> (16 * (j & 1))) & 0xFFFFu) << 16);
    } else {
        const float* p = static_cast<const float*>(x) + e0;
        const v4f a = *reinterpret_cast<const v4f*>(p), b = *reinterpret_cast<const v4f*>(p + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = a[j];
            v[4 + j] = b[j];
        }
    }
}

template <bool BF16>
__global__ __launch_bounds__(QT) void quantize_kernel(const void* __restrict__ x, int64_t n,
                                                      uint8_t* __restrict__ q8,
                                                      float* __restrict__ scale)
{
    const int64_t v = ((int64_t)blockIdx.x * QT + threadIdx.x) >> 4;
    const int p = threadIdx.x & 15;
    float xv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (v < n) load8<BF16>(x, v * 128 + 8 * p, xv);
    const Quant8 r = quantize8(xv);
    if (v < n) {
        *reinterpret_cast<u32x2*>(q8 + v * 128 + 8 * p) = r.codes;
        if (p == 0) scale[v] = r.scale;
    }
}

// One wave per sequence: lanes 0-15 quantise the new key into row r = seq_start[b+1] - 1,
// all lanes copy its 1152-byte latent row.  A sequence without rows (outside the caller's
// contract) is left alone.
template <bool BF16>
__global__ __launch_bounds__(64) void decode_append_kernel(
    const int64_t* __restrict__ seq_start, const void* __restrict__ k_new,
    const uint16_t* __restrict__ kv_new, uint8_t* __restrict__ k8_cache,
    float* __restrict__ ks_cache, uint16_t* __restrict__ kv_cache)
{
    const int b = blockIdx.x, lane = threadIdx.x;
    const int64_t a = seq_start[b], e = seq_start[b + 1];
    if (e <= a) return;                                  // uniform over the wave
    const int64_t r = e - 1;
    float xv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (lane < 16) load8<BF16>(k_new, (int64_t)b * 128 + 8 * lane, xv);
    const Quant8 q = quantize8(xv);
    if (lane < 16) {
        *reinterpret_cast<u32x2*>(k8_cache + r * 128 + 8 * lane) = q.codes;
        if (lane == 0) ks_cache[r] = q.scale;
    }
    const u32x4* src = reinterpret_cast<const u32x4*>(kv_new + (int64_t)b * 576);
    u32x4* dst = reinterpret_cast<u32x4*>(kv_cache + r * 576);
    for (int i = lane; i < 576 * 2 / 16; i += 64) dst[i] = src[i];
}

}  // namespace

hipError_t launch_quantize_fp8(const void* x, bool bf16, int64_t n, uint8_t* q8, float* scale,
                               hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    const dim3 grid((unsigned)((n + QT / 16 - 1) / (QT / 16)));
    if (bf16)
        hipLaunchKernelGGL(quantize_kernel<true>, grid, dim3(QT), 0, stream, x, n, q8, scale);
    else
        hipLaunchKernelGGL(quantize_kernel<false>, grid, dim3(QT), 0, stream, x, n, q8, scale);
    return hipGetLastError();
}

hipError_t launch_decode_append(int B, const int64_t* seq_start, const void* k_new, bool bf16,
                                const uint16_t* kv_new, uint8_t* k8_cache, float* ks_cache,
                                uint16_t* kv_cache, hipStream_t stream)
{
    if (B <= 0) return hipSuccess;
    if (bf16)
        hipLaunchKernelGGL(decode_append_kernel<true>, dim3(B), dim3(64), 0, stream, seq_start,
                           k_new, kv_new, k8_cache, ks_cache, kv_cache);
    else
        hipLaunchKernelGGL(decode_append_kernel<false>, dim3(B), dim3(64), 0, stream, seq_start,
                           k_new, kv_new, k8_cache, ks_cache, kv_cache);
    return hipGetLastError();
}

}  // namespace dsa
