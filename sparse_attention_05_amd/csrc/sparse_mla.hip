// sparse_mla.hip -- attention over the selected latent rows on gfx950.
//
// For query row t and head h: logits l_j = sm_scale * <q[t,h,:576], kv[I_j,:576]> over the
// selected rows I = idx[t,:], softmax within I, output sum_j p_j kv[I_j,:512] with the
// 512-d latent doubling as the value (《DeepSeek-V3.2-Exp模型优势与 DSA 工作原理》 §3 稀疏
// MLA and §4 步骤四; 《狂降75%！…》 §三 第四步).
//
// One workgroup handles one query row for all heads (ceil(H/16) waves, 16 heads each) over
// a contiguous slice of its index list.  The slice's indices are staged in LDS; the selected
// 1152-byte rows are gathered 64 at a time by direct global->LDS loads into a double-buffered
// tile (16-byte chunks XOR-swizzled by row), so the next tile streams in while the current
// one is used.  Per 32-key half: S^T = K Q^T on bf16 MFMA (A = gathered rows, B = Q^T held in
// registers), softmax in the exp2 domain with fp32 statistics against a per-head reference
// max that moves only when exceeded by 2^8, then O += P V with P
// already in the A-operand layout and V read from the same row-major tile through the LDS
// transpose read (ds_read_b64_tr_b16), so no transposed copy of V is ever built.  Both
// contractions are software-pipelined: LDS operands are read several MFMAs ahead and QK runs
// as four independent accumulation chains, since two waves per SIMD alone cannot hide LDS
// latency at this register budget (Q^T 72 + O 128 of 256 VGPRs).
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int MT = 64;                       // keys per tile
constexpr int CH = 72;                       // 16-byte chunks per 1152-byte row
constexpr int TILE_BYTES = MT * CH * 16;     // 73,728
constexpr int IDX_SEG = 2048;                // indices staged in LDS at a time
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4s lds_v4s_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

__device__ __forceinline__ u32x2 ds_read_tr(const uint8_t* p)
{
    const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(p));
    return __builtin_bit_cast(u32x2, v);
}

// tile byte offset of dims [8c, 8c + 8) of row r (chunk c of the 72 per row).  The XOR only
// touches the low three chunk bits, so for c = 8a + b: offset = row_base(r) + 128 a +
// 16 (b ^ (r & 7)) -- a per-lane base plus an immediate.
__device__ __forceinline__ int row_base(int r) { return r * CH * 16; }
__device__ __forceinline__ int sub_off(int r, int b) { return (b ^ (r & 7)) << 4; }

// Headroom of the softmax reference: a head's reference max m moves (and O is rescaled)
// only when a logit exceeds it by more than REF_SLACK in log2 units, so p = 2^(x - m) stays
// below 2^REF_SLACK -- far inside bf16/fp32 range -- and O is rescaled a handful of times
// per row instead of whenever some head's running max creeps up.
constexpr float REF_SLACK = 8.f;

// NW waves per workgroup, 16 heads per wave.
template <int NW>
__global__ __launch_bounds__(NW * 64) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ idx, const int64_t* __restrict__ seq_start, int L, int H, int k,
    float sm_scale, int splits, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse)
{
    constexpr int NT = NW * 64;
    __shared__ __attribute__((aligned(16))) uint8_t s_tile[2][TILE_BYTES];
    __shared__ int s_idx[IDX_SEG];

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

    // B operand of S^T: Q^T, lane holds head c16, dims [32s + 8g, +8) for s = 0..17
    u32x4 qreg[18];
    {
        const bool hv = head < H;
        const uint16_t* qh = q + ((int64_t)row * H + (hv ? head : 0)) * 576;
#pragma unroll
        for (int s = 0; s < 18; ++s)
            qreg[s] = hv ? *reinterpret_cast<const u32x4*>(qh + 32 * s + 8 * g)
                         : u32x4{0u, 0u, 0u, 0u};
    }

    v4f O[32];                                         // O[n]: heads 4g + r, dim 16n + c16
#pragma unroll
    for (int n = 0; n < 32; ++n) O[n] = v4f{0.f, 0.f, 0.f, 0.f};
    float m_ref = -__builtin_huge_valf(), l_run = 0.f;
    const float scale2 = sm_scale * LOG2E;

    // gather of tile t: 72 wave-instructions of 64 x 16 B; instruction qi fills tile bytes
    // [1024 qi, +1024), lane l the chunk slot 64 qi + l
    auto issue = [&](int seg_n, int t, int buf) {
        for (int qi = wave; qi < MT * CH / 64; qi += NW) {
            const int slot = qi * 64 + lane;
            const int r = slot / CH, cs = slot - r * CH;
            const int c = cs ^ (r & 7);
            const int j = t * MT + r;
            const int s = j < seg_n ? s_idx[j] : -1;
            const uint16_t* src = kvr + (int64_t)(s >= 0 ? s : 0) * 576 + c * 8;
            __builtin_amdgcn_global_load_lds((gbl_void_t*)src,
                                             (lds_void_t*)(&s_tile[buf][qi * 1024]), 16, 0, 0);
        }
    };

#pragma unroll 1
    for (int seg0 = jbeg; seg0 < jend; seg0 += IDX_SEG) {
        const int seg_n = min(IDX_SEG, jend - seg0);
        __syncthreads();                               // previous segment fully consumed
        for (int j = tid; j < seg_n; j += NT) {
            const int s = idx[(int64_t)row * k + seg0 + j];
            s_idx[j] = (s >= 0 && s < Lr) ? s : -1;
        }
        __syncthreads();
        const int ntile = (seg_n + MT - 1) / MT;
        issue(seg_n, 0, 0);
#pragma unroll 1
        for (int t = 0; t < ntile; ++t) {
            __builtin_amdgcn_s_waitcnt(0);             // this wave's part of tile t landed
            __syncthreads();                           // everyone's part; tile t-1 consumed
            if (t + 1 < ntile) issue(seg_n, t + 1, (t + 1) & 1);
            const uint8_t* tb = s_tile[t & 1];
            // validity of the tile's 64 keys as one wave-uniform mask
            const int jt = t * MT + lane;
            const uint64_t vmask = __ballot(jt < seg_n && s_idx[jt] >= 0);
#pragma unroll 1
            for (int half = 0; half < 2; ++half) {
                // S^T[key][head] for keys 32 half + 16 kt + (4g + r);
                // A = row 32 half + 16 kt + c16, dims [32s + 8g, +8): chunk 4s + g
                // four independent accumulation chains (2 key groups x even/odd K steps),
                // A operands read QD steps ahead
                v4f S[2], S2[2];
                const uint8_t* rb[2];
                int oo[2][2];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    const int r = half * 32 + kt * 16 + c16;
                    rb[kt] = tb + row_base(r);
                    oo[kt][0] = sub_off(r, g);
                    oo[kt][1] = sub_off(r, 4 + g);
                    S[kt] = v4f{0.f, 0.f, 0.f, 0.f};
                    S2[kt] = v4f{0.f, 0.f, 0.f, 0.f};
                }
                constexpr int QD = 3;
                u32x4 abuf[QD][2];
#pragma unroll
                for (int s = 0; s < QD; ++s)
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
                        abuf[s][kt] = *reinterpret_cast<const u32x4*>(rb[kt] + 128 * (s >> 1) + oo[kt][s & 1]);
#pragma unroll
                for (int s = 0; s < 18; ++s) {
                    u32x4 a[2] = {abuf[s % QD][0], abuf[s % QD][1]};
                    if (s + QD < 18) {
                        const int m = s + QD;
#pragma unroll
                        for (int kt = 0; kt < 2; ++kt)
                            abuf[s % QD][kt] = *reinterpret_cast<const u32x4*>(rb[kt] + 128 * (m >> 1) + oo[kt][m & 1]);
                    }
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
                        if (s & 1) S2[kt] = mfma_bf16(as_bf16x8(a[kt]), as_bf16x8(qreg[s]), S2[kt]);
                        else S[kt] = mfma_bf16(as_bf16x8(a[kt]), as_bf16x8(qreg[s]), S[kt]);
                    }
                }
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) S[kt] += S2[kt];
                // softmax statistics for head c16 over this half's 32 keys
                float x[2][4];
                float mloc = -__builtin_huge_valf();
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    const uint32_t bits = (uint32_t)(vmask >> (half * 32 + kt * 16 + 4 * g));
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        x[kt][r] = ((bits >> r) & 1u) ? S[kt][r] * scale2 : -__builtin_huge_valf();
                        mloc = fmaxf(mloc, x[kt][r]);
                    }
                }
                mloc = fmaxf(mloc, shfl_xor_f(mloc, 16));
                mloc = fmaxf(mloc, shfl_xor_f(mloc, 32));
                // move the reference only when the new max clears the headroom
                const bool move = mloc > m_ref + REF_SLACK;
                const float m_new = move ? mloc : m_ref;
                const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
                const bool rescale = move && m_ref != -__builtin_huge_valf();
                m_ref = m_new;
                // no valid logit yet: keep exp2(-inf - m) = 0 rather than exp2(-inf + inf)
                const float m_sub = m_new == -__builtin_huge_valf() ? 0.f : m_new;
                float p[2][4];
                float psum = 0.f;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        p[kt][r] = __builtin_amdgcn_exp2f(x[kt][r] - m_sub);
                        psum += p[kt][r];
                    }
                l_run = l_run * alpha + psum;
                if (__any(rescale)) {                  // rare: some head's reference moved
                    float ar[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g + r, 64);
#pragma unroll
                    for (int n = 0; n < 32; ++n)
#pragma unroll
                        for (int r = 0; r < 4; ++r) O[n][r] *= ar[r];
                }
                // A operand of P V: head c16, K = keys {4g..4g+3} of each 16-key group
                const v8bf pav = __builtin_convertvector(
                    (v8f){p[0][0], p[0][1], p[0][2], p[0][3], p[1][0], p[1][1], p[1][2], p[1][3]},
                    v8bf);
                // V operand: column 16n + c16, keys 32 half + 16 kt + 4g + r, by transpose reads:
                // lane (g, i) addresses row 32 half + 16 kt + 4g + i/4, dims 16n + 4(i%4) .. +3,
                // i.e. chunk 2n + (i%4)/2 = 8(n/4) + (2(n%4) + (i%4)/2), byte 8 (i%2) within it
                const int rv0 = half * 32 + 4 * g + (c16 >> 2), rv1 = rv0 + 16;
                const int cpart = (c16 & 3) >> 1, boff = (c16 & 1) * 8;
                const uint8_t* vb0 = tb + row_base(rv0) + boff;
                const uint8_t* vb1 = tb + row_base(rv1) + boff;
                int vo0[4], vo1[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    vo0[m] = sub_off(rv0, 2 * m + cpart);
                    vo1[m] = sub_off(rv1, 2 * m + cpart);
                }
                // software-pipelined: the V operand of MFMA n is read PD MFMAs ahead
                constexpr int PD = 4;
                u32x2 vlo[PD], vhi[PD];
#pragma unroll
                for (int n = 0; n < PD; ++n) {
                    vlo[n] = ds_read_tr(vb0 + 128 * (n >> 2) + vo0[n & 3]);
                    vhi[n] = ds_read_tr(vb1 + 128 * (n >> 2) + vo1[n & 3]);
                }
#pragma unroll
                for (int n = 0; n < 32; ++n) {
                    u32x4 vb;
                    vb[0] = vlo[n % PD][0]; vb[1] = vlo[n % PD][1];
                    vb[2] = vhi[n % PD][0]; vb[3] = vhi[n % PD][1];
                    if (n + PD < 32) {
                        const int m = n + PD;
                        vlo[n % PD] = ds_read_tr(vb0 + 128 * (m >> 2) + vo0[m & 3]);
                        vhi[n % PD] = ds_read_tr(vb1 + 128 * (m >> 2) + vo1[m & 3]);
                    }
                    O[n] = mfma_bf16(pav, as_bf16x8(vb), O[n]);
                }
            }
        }
    }

    // totals per head c16, then per O row (head 4g + r)
    float l_tot = l_run + shfl_xor_f(l_run, 16);
    l_tot += shfl_xor_f(l_tot, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float my_lse = l_tot > 0.f ? m_ref * LN2 + logf(l_tot) : -__builtin_huge_valf();
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
    auto kern = sparse_mla_kernel<NW>;
    hipLaunchKernelGGL(kern, dim3(T, splits), dim3(NW * 64), 0, stream, q, kv, idx, seq_start, L,
                       H, k, sm_scale, splits, out, lse, part_o, part_lse);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                             const int64_t* seq_start, int T, int L, int H, int k,
                             float sm_scale, int splits, uint16_t* out, float* lse,
                             float* part_o, float* part_lse, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    const int nw = (H + 15) / 16;                       // 16 heads per wave
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
