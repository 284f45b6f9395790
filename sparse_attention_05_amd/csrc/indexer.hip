// indexer.hip -- the lightning indexer on gfx950.
//
// score[t,s] = ks[s] * sum_h a'[t,h] * ReLU(q8[t,h,:] . k8[s,:]),  a' = w * qs * c,
// for visible keys s <= q_pos0 + t (《DeepSeek-V3.2-Exp模型优势与 DSA 工作原理》 §4 步骤二:
// dot-product score, mask and scale, then per-head weights; ReLU per the gxzdkb DSA
// explainer, section 秘密武器：DSA).  The fp8 dot products run on
// v_mfma_f32_16x16x128_f8f6f4: one instruction contracts all 128 dims of 16 (token, head)
// rows against 16 keys.  ReLU, the a' weighting, the head sum and the key scale are fused
// on the accumulators in registers; the head sum crosses lane groups with a reduce-scatter
// so every lane ends up owning distinct (token, key) outputs.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {
namespace {

// ---------------------------------------------------------------- prefill geometry
constexpr int IP_WAVES = 8;                // waves per workgroup
// (token, head) rows per wave: 64 (four waves per SIMD, so that one wave's MFMA burst runs
// while others work through their epilogues), except 128 for H_I = 128, whose head sum
// needs a whole token in one wave
template <int HI> constexpr int ip_rows() { return HI >= 128 ? 128 : 64; }
template <int HI> constexpr int ip_waves_per_simd() { return (HI >= 128 || HI <= 2) ? 2 : 4; }
constexpr int IP_KT = 128;                 // keys per LDS tile
// keys per workgroup (grid.y): each workgroup loads its rows' queries once per key range, so
// longer ranges fetch them fewer times (16,384: a quarter of the fetches of 4,096, and 1.5%
// faster on a 128K chunk; 32,768 halves them again at the same speed within the spread
// between runs; 65,536 leaves too few workgroups per launch and is slower)
constexpr int IP_KSPLIT = 32768;
constexpr int IP_CSTAGE = 256;             // candidates staged per wave (MODE 1)

// LDS key tile: 128 keys x 128 B.  16-byte chunk c of key r lives at chunk
// c ^ (r & 7) ^ ((r >> 3) & 1).  A 16-byte LDS read is served 16 lanes at a time, in the lane
// groups {0-7, 24-31} and {8-15, 16-23} (and the same in the upper half-wave), 256 B per clock
// when the group's 16-byte slots (address / 16 mod 16) are distinct.  A B-operand read gives
// lane (g, c16) chunk 2g (or 2g + 1) of key c16 of a 16-key block, so a group pairs keys 0-7
// at chunk 2g with keys 8-15 at chunk 2g + 2; the extra XOR by key bit 3 moves the second
// half to the other chunk parity, and the group's slots are then all distinct.
__device__ __forceinline__ int ktile_off(int key, int chunk)
{
    return key * 128 + ((chunk ^ (key & 7) ^ ((key >> 3) & 1)) << 4);
}

// Head reduction of one 32-key step.  acc[kb][j][r] holds D for tile row 4g + r of tile j
// and key kb*16 + c16.  Calls emit(token_in_wave, kb, value) once per distinct output.
template <int HI, int NT, typename Emit>
__device__ __forceinline__ void reduce_heads(const v4f (&acc)[2][NT],
                                             const float (&wp)[NT][4], int lane,
                                             Emit&& emit)
{
    const int g = lane >> 4;
    const bool odd = (g & 1) != 0;
    if constexpr (HI >= 16) {
        constexpr int TPW = NT * 16 / HI;      // tokens per wave
        constexpr int TPT = HI / 16;           // tiles per token
        constexpr int NO = 2 * TPW;            // (token, key block) partials per lane
        constexpr int N1 = NO / 2;
        float P[NO];
#pragma unroll
        for (int tk = 0; tk < TPW; ++tk) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float s = 0.f;
#pragma unroll
                for (int jj = 0; jj < TPT; ++jj) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        s = fmaf(wp[tk * TPT + jj][r], fmaxf(acc[kb][tk * TPT + jj][r], 0.f), s);
                }
                P[tk * 2 + kb] = s;
            }
        }
        // step 1: lanes 0-31 keep partials [0, N1), lanes 32-63 keep [N1, NO)
        float Q[N1];
#pragma unroll
        for (int i = 0; i < N1; ++i) Q[i] = fold32(P[i], P[N1 + i]);
        if constexpr (N1 >= 2) {
            // step 2: even lane groups keep [0, N2), odd keep [N2, N1) -> group g owns
            // outputs g*N2 .. g*N2 + N2 - 1, each now summed over all four groups
            constexpr int N2 = N1 / 2;
#pragma unroll
            for (int i = 0; i < N2; ++i) {
                const float v = fold16(Q[i], Q[N2 + i]);
                const int o = g * N2 + i;
                emit(o >> 1, o & 1, v);
            }
        } else {
            const float v = fold16(Q[0], Q[0]);
            if (!odd) emit(0, g >> 1, v);
        }
    } else if constexpr (HI == 8) {
        // tile j: rows 0-7 token 2j, rows 8-15 token 2j+1; group g: token 2j + g/2
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            float p0 = 0.f, p1 = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p0 = fmaf(wp[j][r], fmaxf(acc[0][j][r], 0.f), p0);
                p1 = fmaf(wp[j][r], fmaxf(acc[1][j][r], 0.f), p1);
            }
            emit(2 * j + (g >> 1), g & 1, fold16(p0, p1));
        }
    } else {
        // HI in {1, 2, 4}: the lane's four rows hold 4/HI whole tokens
        constexpr int UPL = 4 / HI;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
#pragma unroll
            for (int u = 0; u < UPL; ++u) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    float v = 0.f;
#pragma unroll
                    for (int r = u * HI; r < u * HI + HI; ++r)
                        v = fmaf(wp[j][r], fmaxf(acc[kb][j][r], 0.f), v);
                    emit((16 * j + 4 * g) / HI + u, kb, v);
                }
            }
        }
    }
}

// Grid: x = token blocks of IP_WAVES * ip_rows/HI tokens (heaviest, i.e. latest, first),
//       y = key ranges of IP_KSPLIT keys.  Each wave keeps 128 (token, head) query rows
// in registers as MFMA A operands; the workgroup streams 128-key tiles through a
// double-buffered LDS ring that all eight waves read as B operands.
// MODE 0 writes the scores.  One token per wave (HI >= 64) also allows a key stride (key
// index s reads cache row kstride * s, visible when kstride * s <= the token's position:
// the threshold sample) and a row filter (only[t] == 0: row t is skipped).  MODE 1 (one
// token per wave) keeps, per row, the keys of score >= tau[t] as candidates.
template <int HI, int MODE>
__global__ __launch_bounds__(IP_WAVES * 64, ip_waves_per_simd<HI>()) void indexer_prefill_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks, int T, int q_pos0, float c,
    float* __restrict__ scores, int64_t ld, IdxExtra ex)
{
    constexpr int IP_ROWS = ip_rows<HI>();
    constexpr int IP_NT = IP_ROWS / 16;        // 16-row MFMA tiles per wave
    constexpr int TPW = IP_ROWS / HI;
    constexpr int TB = IP_WAVES * TPW;
    static_assert(MODE == 0 || TPW == 1, "candidates need one token per wave");
    __shared__ __attribute__((aligned(16))) uint8_t s_key[2][IP_KT * 128];
    __shared__ float s_ks[2][IP_KT];
    // MODE 1: each wave stages its row's candidates here and appends them to the row's
    // array a batch at a time (one atomic per batch)
    __shared__ uint2 s_cand[IP_WAVES][MODE == 1 ? IP_CSTAGE : 1];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, c16 = lane & 15;
    const int blk = gridDim.x - 1 - blockIdx.x;
    const int t0 = blk * TB;
    const int t_end = min(T, t0 + TB);
    const int kstride = TPW == 1 ? ex.kstride : 1;
    const int p_last = (q_pos0 + t_end - 1) / kstride;   // last key any row here sees
    const int ksplit = ex.ksplit > 0 ? ex.ksplit : IP_KSPLIT;
    const int kbeg = blockIdx.y * ksplit;
    if (kbeg > p_last) return;                         // uniform over the workgroup
    const int kend = min(kbeg + ksplit, p_last + 1);
    if (TPW == 1 && ex.only) {                         // rows of this block still to score
        bool any = false;
        for (int t = t0; t < t_end; ++t) any |= ex.only[t] != 0;
        if (!any) return;                              // uniform
    }

    const int tw0 = t0 + wave * TPW;                   // first token row of this wave
    const bool wave_active = tw0 < T && (TPW > 1 || !ex.only || ex.only[tw0] != 0);
    const int pw_last = (q_pos0 + min(T, tw0 + TPW) - 1) / kstride;
    const int64_t nrows = (int64_t)T * HI;

    // A operands: row 16j + c16 of the wave's (token, head) rows, bytes [32g, 32g + 32)
    v8i qa[IP_NT];
    float wp[IP_NT][4];
#pragma unroll
    for (int j = 0; j < IP_NT; ++j) {
        const int64_t R = (int64_t)tw0 * HI + 16 * j + c16;
        u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
        if (wave_active && R < nrows) {
            const u32x4* src = reinterpret_cast<const u32x4*>(q8 + R * 128 + 32 * g);
            lo = src[0];
            hi = src[1];
        }
        qa[j] = as_i8(lo, hi);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t R2 = (int64_t)tw0 * HI + 16 * j + 4 * g + r;
            wp[j][r] = (wave_active && R2 < nrows) ? w[R2] * qs[R2] * c : 0.f;
        }
    }

    // cooperative tile load: thread -> key tid/4, bytes [32*(tid%4), +32)
    const int lkey = tid >> 2, lpart = tid & 3;
    u32x4 pre0 = {0u, 0u, 0u, 0u}, pre1 = {0u, 0u, 0u, 0u};
    float pre_s = 0.f;
    auto gload = [&](int tile) {
        const int s = kbeg + tile * IP_KT + lkey;
        if (s < kend) {
            const u32x4* src = reinterpret_cast<const u32x4*>(k8 + (int64_t)s * kstride * 128 + 32 * lpart);
            pre0 = src[0];
            pre1 = src[1];
        } else {
            pre0 = u32x4{0u, 0u, 0u, 0u};
            pre1 = pre0;
        }
        if (tid < IP_KT) {
            const int s2 = kbeg + tile * IP_KT + tid;
            pre_s = s2 < kend ? ks[(int64_t)s2 * kstride] : 0.f;
        }
    };
    // MODE 1: the wave's staged candidates (a wave-uniform count) and its row's threshold
    int nst = 0;
    const uint32_t tau_w = MODE == 1 && wave_active ? ex.tau[tw0] : 0u;
    // the threshold as a float: score_key(v) >= tau exactly when v >= tau_f for finite v (the
    // key is monotonic in v with -0 = +0; thresholds at or below the key of -inf keep every key)
    const float tau_f = tau_w <= 0x007FFFFFu ? -__builtin_huge_valf()
                        : __uint_as_float((tau_w & 0x80000000u) ? (tau_w & 0x7FFFFFFFu) : ~tau_w);
    auto flush = [&]() {
        int base = 0;
        if (lane == 0) base = atomicAdd(&ex.fill[tw0], nst);
        base = __shfl(base, 0, 64);
        uint2* dst = ex.cand + (int64_t)tw0 * ex.capr;
        for (int i = lane; i < nst; i += 64)
            if (base + i < ex.capr) dst[base + i] = s_cand[wave][i];
        nst = 0;
    };
    auto sstore = [&](int buf) {
        *reinterpret_cast<u32x4*>(&s_key[buf][ktile_off(lkey, 2 * lpart)]) = pre0;
        *reinterpret_cast<u32x4*>(&s_key[buf][ktile_off(lkey, 2 * lpart + 1)]) = pre1;
        if (tid < IP_KT) s_ks[buf][tid] = pre_s;
    };

    const int ntiles = (kend - kbeg + IP_KT - 1) / IP_KT;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1;
        if (it + 1 < ntiles) gload(it + 1);
        const int tbase = kbeg + it * IP_KT;
        if constexpr (TPW == 1) {
            // one token per wave: 64-key steps of two 32-key MFMA bursts, each folded into
            // per-16-key-block partials right away; one reduce-scatter then leaves lane group
            // g with the finished sum of key block g, so every lane emits one output
            if (wave_active && tbase <= pw_last) {
                float* srow = scores + (int64_t)tw0 * ld + tbase;   // wave-uniform
#pragma unroll
                for (int step = 0; step < IP_KT / 64; ++step) {
                    const int key0 = tbase + step * 64;
                    if (key0 > pw_last) break;
                    float P[4];
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        v4f acc[2][IP_NT];
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) {
                            const int kl = step * 64 + half * 32 + kb * 16 + c16;
                            const u32x4 lo = *reinterpret_cast<const u32x4*>(&s_key[buf][ktile_off(kl, 2 * g)]);
                            const u32x4 hi = *reinterpret_cast<const u32x4*>(&s_key[buf][ktile_off(kl, 2 * g + 1)]);
                            const v8i bb = as_i8(lo, hi);
#pragma unroll
                            for (int j = 0; j < IP_NT; ++j)
                                acc[kb][j] = mfma_f8(qa[j], bb, v4f{0.f, 0.f, 0.f, 0.f});
                        }
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb) {
                            float sum = 0.f;
#pragma unroll
                            for (int j = 0; j < IP_NT; ++j)
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    sum = fmaf(wp[j][r], fmaxf(acc[kb][j][r], 0.f), sum);
                            P[2 * half + kb] = sum;
                        }
                    }
                    const float v = fold16(fold32(P[0], P[2]), fold32(P[1], P[3]));
                    const int sl = step * 64 + 16 * g + c16;          // key within the tile
                    const bool vis = tbase + sl <= pw_last && tbase + sl < kend;
                    if constexpr (MODE == 0) {
                        if (vis) srow[sl] = v * s_ks[buf][sl];
                    } else {
                        // lanes hold consecutive keys, so ballot order is position order
                        const float sv = v * s_ks[buf][sl];
                        const bool take = vis && sv >= tau_f;
                        const uint64_t m = __ballot(take);
                        if (m) {
                            const int nm = __popcll(m);
                            if (nst + nm > IP_CSTAGE) flush();
                            const int rk = __builtin_amdgcn_mbcnt_hi(
                                (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
                            if (take) s_cand[wave][nst + rk] = make_uint2(__float_as_uint(sv), tbase + sl);
                            nst += nm;
                        }
                    }
                }
            }
        } else if (wave_active && tbase <= pw_last) {
#pragma unroll 1
            for (int step = 0; step < IP_KT / 32; ++step) {
                const int key0 = tbase + step * 32;
                if (key0 > pw_last) break;
                v4f acc[2][IP_NT];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int kl = step * 32 + kb * 16 + c16;
                    const u32x4 lo = *reinterpret_cast<const u32x4*>(&s_key[buf][ktile_off(kl, 2 * g)]);
                    const u32x4 hi = *reinterpret_cast<const u32x4*>(&s_key[buf][ktile_off(kl, 2 * g + 1)]);
                    const v8i bb = as_i8(lo, hi);
#pragma unroll
                    for (int j = 0; j < IP_NT; ++j)
                        acc[kb][j] = mfma_f8(qa[j], bb, v4f{0.f, 0.f, 0.f, 0.f});
                }
                // issue the step's MFMAs as one burst; the epilogue then trails the matrix
                // pipe instead of waiting on each result in turn
                __builtin_amdgcn_sched_barrier(0);
                reduce_heads<HI, IP_NT>(acc, wp, lane, [&](int tok, int kb, float v) {
                    const int t = tw0 + tok;
                    const int s = key0 + kb * 16 + c16;
                    if (t < T && s <= q_pos0 + t && s < kend)
                        scores[(int64_t)t * ld + s] = v * s_ks[buf][s - tbase];
                });
            }
        }
        if (it + 1 < ntiles) sstore(buf ^ 1);
        __syncthreads();
    }
    if constexpr (MODE == 1)
        if (wave_active && nst > 0) flush();
}

__global__ __launch_bounds__(256) void mask_fill_kernel(int L, int q_pos0, float* scores,
                                                        int64_t ld)
{
    const int t = blockIdx.x;
    const float ninf = -__builtin_huge_valf();
    for (int s = q_pos0 + t + 1 + threadIdx.x; s < L; s += blockDim.x)
        scores[(int64_t)t * ld + s] = ninf;
}

// ---------------------------------------------------------------- decode geometry
constexpr int ID_WAVES = 4;
constexpr int ID_KPW = 128;                      // keys per wave
constexpr int ID_KPB = ID_WAVES * ID_KPW;        // keys per workgroup

// Grid: x = key chunks of one sequence's cache, y = sequence.  One query token of HI
// heads is the MFMA A operand (HI/16 tiles, zero-padded below 16 heads); every wave
// streams its own keys straight from HBM as B operands, 64 keys per step.  This is the
// bandwidth-bound shape: 132 bytes of key and scale per scored token.
template <int HI>
__global__ __launch_bounds__(ID_WAVES * 64) void indexer_decode_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const float* __restrict__ w,
    const uint8_t* __restrict__ k8, const float* __restrict__ ks,
    const int64_t* __restrict__ seq_start, float c, float* __restrict__ scores)
{
    constexpr int NTQ = HI >= 16 ? HI / 16 : 1;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, c16 = lane & 15;
    const int b = blockIdx.y;
    const int64_t a = seq_start[b];
    const int Lb = (int)(seq_start[b + 1] - a);
    const int sw0 = blockIdx.x * ID_KPB + wave * ID_KPW;
    if (sw0 >= Lb) return;                            // no barriers in this kernel

    // lane K assignment (A and B alike): 16-byte chunks g and g + 4 of the 128-byte row
    v8i qa[NTQ];
    float wp[NTQ][4];
#pragma unroll
    for (int j = 0; j < NTQ; ++j) {
        const int h = 16 * j + c16;
        u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
        if (h < HI) {
            const uint8_t* src = q8 + ((int64_t)b * HI + h) * 128;
            lo = *reinterpret_cast<const u32x4*>(src + 16 * g);
            hi = *reinterpret_cast<const u32x4*>(src + 64 + 16 * g);
        }
        qa[j] = as_i8(lo, hi);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int hh = 16 * j + 4 * g + r;
            wp[j][r] = hh < HI ? w[b * HI + hh] * qs[b * HI + hh] * c : 0.f;
        }
    }

    // All of the wave's key rows (and their scales) are requested before any is used, so
    // 16 KB per wave are in flight (the loop is bound by HBM latency otherwise); 128 keys per
    // wave leave room for three waves per SIMD (256 keys: two, 2.8% slower per decode step).
    constexpr int NS = ID_KPW / 64;                  // 64-key steps per wave
    u32x4 kd[NS][4][2];
    float ksv[NS];
#pragma unroll
    for (int it = 0; it < NS; ++it) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int key = sw0 + it * 64 + kb * 16 + c16;
            kd[it][kb][0] = u32x4{0u, 0u, 0u, 0u};
            kd[it][kb][1] = u32x4{0u, 0u, 0u, 0u};
            if (key < Lb) {
                const uint8_t* src = k8 + (a + key) * 128;
                kd[it][kb][0] = *reinterpret_cast<const u32x4*>(src + 16 * g);
                kd[it][kb][1] = *reinterpret_cast<const u32x4*>(src + 64 + 16 * g);
            }
        }
        const int key = sw0 + it * 64 + g * 16 + c16;
        ksv[it] = key < Lb ? ks[a + key] : 0.f;
    }
#pragma unroll
    for (int it = 0; it < NS; ++it) {
        const int s0 = sw0 + it * 64;
        if (s0 >= Lb) break;
        float P[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const v8i bb = as_i8(kd[it][kb][0], kd[it][kb][1]);
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < NTQ; ++j) {
                const v4f d = mfma_f8(qa[j], bb, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int r = 0; r < 4; ++r) s = fmaf(wp[j][r], fmaxf(d[r], 0.f), s);
            }
            P[kb] = s;
        }
        // reduce-scatter over the four lane groups: group g ends with key block g
        const float Q0 = fold32(P[0], P[2]), Q1 = fold32(P[1], P[3]);
        const float v = fold16(Q0, Q1);
        const int key = s0 + g * 16 + c16;
        if (key < Lb) scores[a + key] = v * ksv[it];
    }
}

template <int HI, int MODE>
hipError_t launch_prefill_hi(const uint8_t* q8, const float* qs, const float* w,
                             const uint8_t* k8, const float* ks, int T, int L, int q_pos0,
                             float c, float* scores, int64_t ld, const IdxExtra& ex,
                             hipStream_t stream)
{
    constexpr int TB = IP_WAVES * (ip_rows<HI>() / HI);
    const int kstride = ex.kstride > 1 ? ex.kstride : 1;
    // key indices any row can see: s with kstride * s <= q_pos0 + T - 1 (and < L)
    const int keys = min((L - 1) / kstride, (q_pos0 + T - 1) / kstride) + 1;
    const int ksplit = ex.ksplit > 0 ? ex.ksplit : IP_KSPLIT;
    dim3 grid((T + TB - 1) / TB, (keys + ksplit - 1) / ksplit);
    hipLaunchKernelGGL((indexer_prefill_kernel<HI, MODE>), grid, dim3(IP_WAVES * 64), 0,
                       stream, q8, qs, w, k8, ks, T, q_pos0, c, scores, ld, ex);
    return hipGetLastError();
}

template <int HI>
hipError_t launch_decode_hi(const uint8_t* q8, const float* qs, const float* w,
                            const uint8_t* k8, const float* ks, const int64_t* seq_start, int B,
                            int max_len, float c, float* scores, hipStream_t stream)
{
    dim3 grid((max_len + ID_KPB - 1) / ID_KPB, B);
    hipLaunchKernelGGL(indexer_decode_kernel<HI>, grid, dim3(ID_WAVES * 64), 0, stream, q8, qs,
                       w, k8, ks, seq_start, c, scores);
    return hipGetLastError();
}

}  // namespace

bool indexer_supports(int H_I)
{
    return H_I == 1 || H_I == 2 || H_I == 4 || H_I == 8 || H_I == 16 || H_I == 32 ||
           H_I == 64 || H_I == 128;
}

bool indexer_fused_supports(int H_I) { return H_I == 64 || H_I == 128; }

hipError_t launch_indexer_prefill(const uint8_t* q8, const float* qs, const float* w,
                                  const uint8_t* k8, const float* ks, int T, int L, int H_I,
                                  int q_pos0, float c, float* scores, int64_t ld,
                                  hipStream_t stream, const IdxExtra& ex)
{
    if (T <= 0) return hipSuccess;
    if ((ex.kstride > 1 || ex.only) && !indexer_fused_supports(H_I)) return hipErrorInvalidValue;
#define DSA_IDX_CASE(HI) \
    case HI: return launch_prefill_hi<HI, 0>(q8, qs, w, k8, ks, T, L, q_pos0, c, scores, ld, ex, stream);
    switch (H_I) {
        DSA_IDX_CASE(1) DSA_IDX_CASE(2) DSA_IDX_CASE(4) DSA_IDX_CASE(8)
        DSA_IDX_CASE(16) DSA_IDX_CASE(32) DSA_IDX_CASE(64) DSA_IDX_CASE(128)
        default: return hipErrorInvalidValue;
    }
#undef DSA_IDX_CASE
}

hipError_t launch_indexer_candidates(const uint8_t* q8, const float* qs, const float* w,
                                     const uint8_t* k8, const float* ks, int T, int L, int H_I,
                                     int q_pos0, float c, const IdxExtra& ex,
                                     hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    IdxExtra e = ex;
    e.kstride = 1;
    e.only = nullptr;
    if (H_I == 64)
        return launch_prefill_hi<64, 1>(q8, qs, w, k8, ks, T, L, q_pos0, c, nullptr, 0, e, stream);
    if (H_I == 128)
        return launch_prefill_hi<128, 1>(q8, qs, w, k8, ks, T, L, q_pos0, c, nullptr, 0, e, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_mask_fill(int T, int L, int q_pos0, float* scores, int64_t ld,
                            hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(mask_fill_kernel, dim3(T), dim3(256), 0, stream, L, q_pos0, scores, ld);
    return hipGetLastError();
}

hipError_t launch_indexer_decode(const uint8_t* q8, const float* qs, const float* w,
                                 const uint8_t* k8, const float* ks, const int64_t* seq_start,
                                 int B, int max_len, int H_I, float c, float* scores,
                                 hipStream_t stream)
{
    if (B <= 0) return hipSuccess;
#define DSA_IDX_CASE(HI) \
    case HI: return launch_decode_hi<HI>(q8, qs, w, k8, ks, seq_start, B, max_len, c, scores, stream);
    switch (H_I) {
        DSA_IDX_CASE(1) DSA_IDX_CASE(2) DSA_IDX_CASE(4) DSA_IDX_CASE(8)
        DSA_IDX_CASE(16) DSA_IDX_CASE(32) DSA_IDX_CASE(64) DSA_IDX_CASE(128)
        default: return hipErrorInvalidValue;
    }
#undef DSA_IDX_CASE
}

}  // namespace dsa
