// sparse_mla.hip -- attention over the selected latent rows on gfx950.
//
// For query row t and head h: logits l_j = sm_scale * <q[t,h,:576], kv[I_j,:576]> over the
// selected rows I = idx[t,:], softmax within I, output sum_j p_j kv[I_j,:512] with the
// 512-d latent doubling as the value (《DeepSeek-V3.2-Exp模型优势与 DSA 工作原理》 §3 稀疏
// MLA and §4 步骤四; 《狂降75%！…》 §三 第四步).
//
// One workgroup handles one query row for all heads (ceil(H/16) waves, 16 heads each)
// over a contiguous slice of its index list.  Per 32-key tile the workgroup gathers the
// selected 1152-byte rows into LDS twice: row-major (the K operand of S^T = K Q^T, whose
// contraction runs along a row), and, for the 512 latent dims, transposed into 4-key
// groups (the V operand of O = P V, whose contraction runs across rows).  Computing S^T
// rather than S leaves P in registers exactly where the A operand of P V needs it.
// Softmax is online in the exp2 domain with fp32 statistics; P is rounded to bf16.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int MT = 32;                       // keys per tile
constexpr int KROW = 576 * 2 + 16;           // LDS bytes per gathered row (+16 B skew)
constexpr int K_BYTES = MT * KROW;           // row-major tile
constexpr int VT_BYTES = (MT / 4) * 512 * 8; // [key quad][dim][4 keys] bf16
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <int NW>
__global__ __launch_bounds__(NW * 64) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ idx, const int64_t* __restrict__ seq_start, int L, int H, int k,
    float sm_scale, int splits, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse)
{
    constexpr int NT = NW * 64;
    __shared__ __attribute__((aligned(16))) uint8_t s_k[K_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t s_vt[VT_BYTES];
    __shared__ int s_idx[MT];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, c16 = lane & 15;
    const int row = blockIdx.x, split = blockIdx.y;
    const int h0 = wave * 16;
    const int head = h0 + c16;                         // this lane's head in S^T / softmax

    int64_t kv_base = 0;
    int Lr = L;
    if (seq_start) {
        kv_base = seq_start[row];
        Lr = (int)(seq_start[row + 1] - kv_base);
    }
    const uint16_t* kvr = kv + kv_base * 576;
    const int per = (k + splits - 1) / splits;
    const int jbeg = split * per;
    const int jend = min(k, jbeg + per);
    const int ntile = jend > jbeg ? (jend - jbeg + MT - 1) / MT : 0;

    // B operand of S^T: Q^T, lane holds head c16, dims [32s + 8g, +8) for s = 0..17
    u32x4 qreg[18];
    {
        const bool hv = head < H;
        const uint16_t* qh = q + ((int64_t)row * H + (hv ? head : 0)) * 576;
#pragma unroll
        for (int s = 0; s < 18; ++s) {
            qreg[s] = hv ? *reinterpret_cast<const u32x4*>(qh + 32 * s + 8 * g)
                         : u32x4{0u, 0u, 0u, 0u};
        }
    }

    v4f O[32];
#pragma unroll
    for (int n = 0; n < 32; ++n) O[n] = v4f{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_huge_valf(), l_run = 0.f;
    const float scale2 = sm_scale * LOG2E;

#pragma unroll 1
    for (int tile = 0; tile < ntile; ++tile) {
        const int j0 = jbeg + tile * MT;
        if (tid < MT) {
            int s = -1;
            if (j0 + tid < jend) s = idx[(int64_t)row * k + j0 + tid];
            s_idx[tid] = (s >= 0 && s < Lr) ? s : -1;
        }
        __syncthreads();
        // gather: item = (key quad, 16-byte chunk of the 512 latent dims) -> 4 rows' chunks,
        // stored row-major and transposed; then the 64 rope dims row-major only.
        for (int it = tid; it < (MT / 4) * 64; it += NT) {
            const int quad = it >> 6, ch = it & 63;
            u32x4 v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = s_idx[quad * 4 + e];
                v[e] = s >= 0 ? *reinterpret_cast<const u32x4*>(kvr + (int64_t)s * 576 + ch * 8)
                              : u32x4{0u, 0u, 0u, 0u};
                *reinterpret_cast<u32x4*>(&s_k[(quad * 4 + e) * KROW + ch * 16]) = v[e];
            }
            // transpose 4 keys x 8 dims -> 8 dims x 4 keys (one 8-byte word per dim)
#pragma unroll
            for (int dd = 0; dd < 8; ++dd) {
                const int wsel = dd >> 1;
                const bool hi = dd & 1;
                auto pick = [&](const u32x4& x) -> uint32_t {
                    return hi ? (x[wsel] >> 16) : (x[wsel] & 0xFFFFu);
                };
                u32x2 word;
                word[0] = pick(v[0]) | (pick(v[1]) << 16);
                word[1] = pick(v[2]) | (pick(v[3]) << 16);
                *reinterpret_cast<u32x2*>(&s_vt[(quad * 512 + ch * 8 + dd) * 8]) = word;
            }
        }
        for (int it = tid; it < MT * 8; it += NT) {
            const int key = it >> 3, ch = 64 + (it & 7);
            const int s = s_idx[key];
            const u32x4 v = s >= 0 ? *reinterpret_cast<const u32x4*>(kvr + (int64_t)s * 576 + ch * 8)
                                   : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(&s_k[key * KROW + ch * 16]) = v;
        }
        __syncthreads();

        if (h0 < H) {
            // S^T[key][head] for two 16-key halves: A = gathered rows, B = Q^T
            v4f S[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                S[kt] = v4f{0.f, 0.f, 0.f, 0.f};
                const uint8_t* krow = &s_k[(kt * 16 + c16) * KROW];
#pragma unroll
                for (int s = 0; s < 18; ++s) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(krow + (32 * s + 8 * g) * 2);
                    S[kt] = mfma_bf16(as_bf16x8(a), as_bf16x8(qreg[s]), S[kt]);
                }
            }
            // lane: head c16, keys kt*16 + 4g + r
            float x[2][4];
            float mloc = -__builtin_huge_valf();
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool valid = s_idx[kt * 16 + 4 * g + r] >= 0;
                    x[kt][r] = valid ? S[kt][r] * scale2 : -__builtin_huge_valf();
                    mloc = fmaxf(mloc, x[kt][r]);
                }
            mloc = fmaxf(mloc, shfl_xor_f(mloc, 16));
            mloc = fmaxf(mloc, shfl_xor_f(mloc, 32));
            const float m_new = fmaxf(m_run, mloc);
            const bool any = m_new != -__builtin_huge_valf();
            const float alpha = any ? exp2f(m_run - m_new) : 1.f;
            float p[2][4];
            float psum = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    p[kt][r] = any ? exp2f(x[kt][r] - m_new) : 0.f;
                    psum += p[kt][r];
                }
            l_run = l_run * alpha + psum;
            m_run = m_new;
            // O rows are heads 4g + r: fetch their rescale factors
            float ar[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g + r, 64);
#pragma unroll
            for (int n = 0; n < 32; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) O[n][r] *= ar[r];
            // A operand of P V: head c16, K = keys {4g..4g+3} of each half
            u32x4 pa;
            pa[0] = pack_bf16x2(p[0][0], p[0][1]);
            pa[1] = pack_bf16x2(p[0][2], p[0][3]);
            pa[2] = pack_bf16x2(p[1][0], p[1][1]);
            pa[3] = pack_bf16x2(p[1][2], p[1][3]);
            const v8bf pav = as_bf16x8(pa);
#pragma unroll
            for (int n = 0; n < 32; ++n) {
                const int d = 16 * n + c16;
                const u32x2 lo = *reinterpret_cast<const u32x2*>(&s_vt[(g * 512 + d) * 8]);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(&s_vt[((4 + g) * 512 + d) * 8]);
                u32x4 vb;
                vb[0] = lo[0]; vb[1] = lo[1]; vb[2] = hi[0]; vb[3] = hi[1];
                O[n] = mfma_bf16(pav, as_bf16x8(vb), O[n]);
            }
        }
        __syncthreads();
    }

    if (h0 >= H) return;
    // totals per head c16, then per O row (head 4g + r)
    float l_tot = l_run + shfl_xor_f(l_run, 16);
    l_tot += shfl_xor_f(l_tot, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float my_lse = l_tot > 0.f ? m_run * LN2 + logf(l_tot) : -__builtin_huge_valf();
    float ir[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ir[r] = __shfl(inv, 4 * g + r, 64);

    if (splits == 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int hh = h0 + 4 * g + r;
            if (hh >= H) continue;
            uint16_t* orow = out + ((int64_t)row * H + hh) * 512;
#pragma unroll
            for (int n = 0; n < 32; ++n) orow[16 * n + c16] = (uint16_t)bf16_bits(O[n][r] * ir[r]);
        }
        if (lse && g == 0 && head < H) lse[(int64_t)row * H + head] = my_lse;
    } else {
        const int64_t pb = ((int64_t)row * splits + split) * H;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int hh = h0 + 4 * g + r;
            if (hh >= H) continue;
            float* orow = part_o + (pb + hh) * 512;
#pragma unroll
            for (int n = 0; n < 32; ++n) orow[16 * n + c16] = O[n][r] * ir[r];
        }
        if (g == 0 && head < H) part_lse[pb + head] = my_lse;
    }
}

// Merge split partials: out = sum_s exp(lse_s - lse) o_s with lse = log sum_s exp(lse_s).
__global__ __launch_bounds__(128) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          int H, int splits,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse)
{
    const int row = blockIdx.x / H, hh = blockIdx.x % H;
    const int tid = threadIdx.x;                     // 4 dims per thread
    float mx = -__builtin_huge_valf();
    for (int s = 0; s < splits; ++s)
        mx = fmaxf(mx, part_lse[((int64_t)row * splits + s) * H + hh]);
    float acc[4] = {0.f, 0.f, 0.f, 0.f}, den = 0.f;
    if (mx != -__builtin_huge_valf()) {
        for (int s = 0; s < splits; ++s) {
            const int64_t pb = ((int64_t)row * splits + s) * H + hh;
            const float ls = part_lse[pb];
            if (ls == -__builtin_huge_valf()) continue;
            const float wgt = expf(ls - mx);
            den += wgt;
            const v4f o = *reinterpret_cast<const v4f*>(part_o + pb * 512 + 4 * tid);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += wgt * o[e];
        }
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    u32x2 packed;
    packed[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    packed[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<u32x2*>(out + ((int64_t)row * H + hh) * 512 + 4 * tid) = packed;
    if (lse && tid == 0)
        lse[(int64_t)row * H + hh] = den > 0.f ? mx + logf(den) : -__builtin_huge_valf();
}

template <int NW>
hipError_t launch_nw(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                     const int64_t* seq_start, int T, int L, int H, int k, float sm_scale,
                     int splits, uint16_t* out, float* lse, float* part_o, float* part_lse,
                     hipStream_t stream)
{
    hipLaunchKernelGGL(sparse_mla_kernel<NW>, dim3(T, splits), dim3(NW * 64), 0, stream, q, kv,
                       idx, seq_start, L, H, k, sm_scale, splits, out, lse, part_o, part_lse);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                             const int64_t* seq_start, int T, int L, int H, int k,
                             float sm_scale, int splits, uint16_t* out, float* lse,
                             float* part_o, float* part_lse, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    const int nw = (H + 15) / 16;
#define DSA_MLA_CASE(NW) \
    case NW: return launch_nw<NW>(q, kv, idx, seq_start, T, L, H, k, sm_scale, splits, out, lse, part_o, part_lse, stream);
    switch (nw) {
        DSA_MLA_CASE(1) DSA_MLA_CASE(2) DSA_MLA_CASE(3) DSA_MLA_CASE(4)
        DSA_MLA_CASE(5) DSA_MLA_CASE(6) DSA_MLA_CASE(7) DSA_MLA_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef DSA_MLA_CASE
}

hipError_t launch_mla_combine(const float* part_o, const float* part_lse, int T, int H,
                              int splits, uint16_t* out, float* lse, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(mla_combine_kernel, dim3(T * H), dim3(128), 0, stream, part_o, part_lse,
                       H, splits, out, lse);
    return hipGetLastError();
}

}  // namespace dsa
