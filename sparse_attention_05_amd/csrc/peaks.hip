// peaks.hip -- what this chip's matrix cores and HBM deliver, measured with streams that have
// no dependencies (a separate library, libdsa_peaks.so, used by the benchmark only: the
// kernels' roofline fractions are reported against both the published and these measured
// peaks).
//
//  * MFMA streams: every wave issues ITER rounds of 8 independent MFMAs (fp8 16x16x128 or
//    bf16 16x16x32) on operands drawn from a per-lane hash (random finite values: the matrix
//    cores draw more power, and the shader clock settles lower, on random data than on zeros),
//    one or two waves per SIMD, all 256 CUs busy.
//  * HBM read stream: a buffer far larger than the last-level cache read once with 16-byte
//    loads, four in flight per lane, the loaded words folded into one register.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa_device.h"

namespace {

using dsa::u32x4;
using dsa::v4f;
using dsa::v8i;

__device__ __forceinline__ uint32_t hash32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    x ^= x >> 16;
    return x;
}

// a finite e4m3fn byte (never 0x7F / 0xFF, the NaN codes) from hash bits
__device__ __forceinline__ uint32_t finite_e4m3x4(uint32_t h)
{
    return h & 0xF7F7F7F7u;          // exponent field below 15: no NaN code
}

// a finite bf16 pair of magnitude near 1 from hash bits
__device__ __forceinline__ uint32_t bf16x2_near_one(uint32_t h)
{
    return (h & 0x807F807Fu) | 0x3F003F00u;
}

// at most two waves per SIMD run it, so the register budget is not squeezed for occupancy
template <bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
void mfma_stream_kernel(int iters, float* __restrict__ sink)
{
    const uint32_t lane = threadIdx.x + 256u * blockIdx.x;
    v4f acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
    if constexpr (FP8) {
        v8i a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (int)finite_e4m3x4(hash32(lane * 16u + i));
            b[i] = (int)finite_e4m3x4(hash32(lane * 16u + 8u + i));
        }
#pragma unroll 1
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = dsa::mfma_f8(a, b, acc[i]);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        u32x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = bf16x2_near_one(hash32(lane * 8u + e));
        const dsa::v8bf av = dsa::as_bf16x8(t);
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = bf16x2_near_one(hash32(lane * 8u + 4u + e));
        const dsa::v8bf bv = dsa::as_bf16x8(t);
        // written as assembly: with the builtin, the compiler rotates these eight chains
        // through extra AGPR copies every iteration; the accumulators are read only after
        // the loop, behind 18 wait states (the MFMA-to-VALU read hazard)
#pragma unroll 1
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i]) : "v"(av), "v"(bv));
        }
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 1" ::: "memory");
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
    if (s == 1.2345678f) sink[lane] = s;       // keeps the stream alive, never true in practice
}

__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                          uint32_t* __restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t x = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        x ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^
             d[0] ^ d[1] ^ d[2] ^ d[3];
    }
    for (; i < n16; i += stride) {
        const u32x4 a = p[i];
        x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    if (x == 0x9E3779B9u) sink[threadIdx.x] = x;
}

}  // namespace

extern "C" {

// MFMA stream: `blocks` workgroups of 256 threads (4 waves), each wave `iters` x 8 MFMAs;
// kind 0 = fp8 16x16x128 (2 * 16 * 16 * 128 flop each), 1 = bf16 16x16x32 (2 * 16 * 16 * 32).
// sink: device float [blocks * 256].  Returns a hipError_t.
int dsa_peak_mfma(int kind, int blocks, int iters, float* sink, hipStream_t stream)
{
    if (kind == 0)
        hipLaunchKernelGGL(mfma_stream_kernel<true>, dim3(blocks), dim3(256), 0, stream, iters,
                           sink);
    else
        hipLaunchKernelGGL(mfma_stream_kernel<false>, dim3(blocks), dim3(256), 0, stream, iters,
                           sink);
    return (int)hipGetLastError();
}

// HBM read stream over `bytes` (a multiple of 16) at device pointer p; sink: device uint32
// [256].  Returns a hipError_t.
int dsa_peak_read(const void* p, int64_t bytes, int blocks, uint32_t* sink, hipStream_t stream)
{
    hipLaunchKernelGGL(read_stream_kernel, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const u32x4*>(p), bytes / 16, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
