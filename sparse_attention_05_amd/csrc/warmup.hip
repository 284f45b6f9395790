// warmup.hip -- the indexer's warm-up objective on gfx950: KL divergence from the frozen
// main attention's head-averaged dense distribution to the indexer's softmax, and its
// gradient with respect to the indexer query vectors, key vectors and head weights
// (ele-yufo.com notes "DeepSeek V3.2-Exp", §四 训练的两步走冷启动, 第一阶段 Warm-up).
//
// For query row t at position p (keys s <= p):
//   teacher  P[t,s] = (1/H) sum_h exp(sm_scale <q[t,h], kv[s]> - lse[t,h])
//   student  I[t,s] = the lightning-indexer score (indexer.hip), Q[t,s] = softmax_s I[t,s]
//   kl[t]    = sum_s P log(P / Q),    G[t,s] = Q[t,s] - P[t,s]  (= dkl/dI)
//   dw[t,h]  = c qs[t,h] sum_s G ks[s] max(D, 0)
//   dq[t,h,:]= c w[t,h] sum_s G ks[s] [D > 0] k8[s,:]          (w.r.t. qs * q8)
//   dk[s,:]  = c sum_t sum_h G w[t,h] qs[t,h] [D > 0] q8[t,h,:] (w.r.t. ks * k8)
// with D[t,h,s] = <q8[t,h], k8[s]> over the fp8 values (the indexer's own product).
//
// Kernels:
//  * teacher_kernel<MODE>: dense causal logits of two query tokens x 128 heads per workgroup
//    (eight waves, two per SIMD: no P V, so a wave fits in half the register file), 64-key
//    tiles of 1152-byte cache rows streamed by direct global->LDS loads into a double buffer.
//    MODE 0 keeps each head's running max and sum (-> lse); MODE 1 sums exp(logit - lse) over
//    the heads of each key (-> P).
//  * row_kernel: one workgroup per row: lse of the scores, G (over P, in place) and kl.
//  * dq_kernel: 256 (token, head) rows per workgroup (eight waves, two per SIMD) held as fp8
//    B operands; 64-key tiles staged in LDS as fp8 (A of D^T) and bf16 (A of dq^T = K^T e^T);
//    e^T = G ks [D > 0] goes from the D^T accumulators straight into the B operand of the bf16
//    MFMA (the contraction takes the keys in the accumulator's order).
//  * dk_kernel: the mirror image: 256 keys x 16 indexer heads per workgroup (eight waves), the
//    keys in registers, 64-row tiles of (token, head) rows streamed; e = G w qs [D > 0];
//    per-head-group partial sums accumulated across query chunks, then summed over the groups.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr float W_LOG2E = 1.4426950408889634f;
constexpr float W_LN2 = 0.6931471805599453f;

// ---------------------------------------------------------------- teacher: dense logits
constexpr int TM = 64;                        // keys per tile
constexpr int T_LROW = 1024;                  // latent bytes per row in a tile
constexpr int T_RROW = 128;                   // rope bytes per row
constexpr int T_ROPE = TM * T_LROW;           // rope part of a tile
constexpr int T_TILE = TM * 1152;             // 73,728 bytes
// 16-byte chunk swizzles of the row-major tile (latent chunk c of row r at slot c ^ 2 (r mod 8),
// rope chunk b at b ^ ((r >> 1) mod 8)): conflict-free K-operand reads
__device__ __forceinline__ int t_latx(int r) { return (r & 7) << 1; }
__device__ __forceinline__ int t_ropex(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ float sum_row16(float v)
{
    // sum over the 16 lanes of a row by rotations (every lane gets the total)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
    return v;
}

// Grid: x = pairs of query tokens, latest (heaviest) first.  Wave w: token 2 pair + w/4,
// heads [32 (w%4), +32).  MODE 0 writes lse[t,h]; MODE 1 reads it and writes P[t, s <= p].
template <int MODE>
__global__ __launch_bounds__(512) void teacher_kernel(const uint16_t* __restrict__ q,
                                                      const uint16_t* __restrict__ kv, int T,
                                                      int H, int q_pos0, float sm_scale,
                                                      float* __restrict__ lse,
                                                      float* __restrict__ P, int64_t ld)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_tile[2][T_TILE];
    __shared__ float s_red[2][2][4][TM];               // [tile parity][token][quarter][key]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tt = wave >> 2, hw = wave & 3;
    const int g = lane >> 4, c16 = lane & 15;
    const int t0 = 2 * (int)(gridDim.x - 1 - blockIdx.x);
    const int t = t0 + tt;
    const bool tok = t < T;
    const int p = q_pos0 + t;                           // this wave's query position
    const int p_last = q_pos0 + min(T, t0 + 2) - 1;     // last key either token sees
    const int ntile = p_last / TM + 1;

    // B operand of S^T = K Q^T: head 32 hw + 16 hq + c16, dims [32 s + 8 g, +8)
    u32x4 qreg[2][18];
    float lse2[2];
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
        const int hh = hw * 32 + hq * 16 + c16;
        const bool hv = tok && hh < H;
        const uint16_t* qh = q + ((int64_t)(hv ? t : 0) * H + (hv ? hh : 0)) * 576;
#pragma unroll
        for (int s = 0; s < 18; ++s)
            qreg[hq][s] = hv ? *reinterpret_cast<const u32x4*>(qh + 32 * s + 8 * g)
                             : u32x4{0u, 0u, 0u, 0u};
        if constexpr (MODE == 1) {
            const float v = lse[hv ? (int64_t)t * H + hh : 0];
            lse2[hq] = hv ? v * W_LOG2E : __builtin_huge_valf();
        } else {
            lse2[hq] = 0.f;
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    const float scale2 = sm_scale * W_LOG2E;
    float m_run[2] = {-__builtin_huge_valf(), -__builtin_huge_valf()}, l_run[2] = {0.f, 0.f};

    // Tile load: wave w moves the latent parts of rows 8w .. 8w+7 (one instruction per row,
    // lane l loading source chunk l ^ t_latx(r)) and the rope parts of the same rows (lane l:
    // row 8w + l/8, slot l%8 <- rope chunk (l%8) ^ t_ropex(row)).  Rows past p_last load
    // row p_last and are masked.
    const uint32_t lds_tiles = __builtin_amdgcn_readfirstlane(lds_addr(s_tile[0]));
    auto issue = [&](int tile, int buf) {
        const uint32_t dst = lds_tiles + (uint32_t)buf * T_TILE;
        const int kb = tile * TM;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = wave * 8 + i;
            const int sr = min(kb + r, p_last);
            dma16_s(16u * (uint32_t)(lane ^ (2 * i)), kv + (int64_t)sr * 576, dst + r * T_LROW);
        }
        const int rr = wave * 8 + (lane >> 3);
        const int sr = min(kb + rr, p_last);
        const uint32_t src = 16u * (64u + (uint32_t)((lane & 7) ^ t_ropex(rr)));
        dma16(reinterpret_cast<const uint8_t*>(kv + (int64_t)sr * 576) + src,
              dst + T_ROPE + wave * 1024);
    };
    // P of the previous tile: the four quarters' head sums of each (token, key)
    auto finish = [&](int tile) {
        if (tid < 2 * TM) {
            const int tk = tid / TM, key = tid % TM;
            const int tq = t0 + tk, s = tile * TM + key;
            if (tq < T && s <= q_pos0 + tq) {
                const float* r = s_red[tile & 1][tk][0];
                const float v = r[key] + r[TM + key] + r[2 * TM + key] + r[3 * TM + key];
                P[(int64_t)tq * ld + s] = v / (float)H;
            }
        }
    };

    issue(0, 0);
#pragma unroll 1
    for (int tile = 0; tile < ntile; ++tile) {
        const uint8_t* tb = s_tile[tile & 1];
        __builtin_amdgcn_s_waitcnt(0);                 // this wave's part of the tile landed
        __syncthreads();                               // all parts; previous tile consumed
        if (tile + 1 < ntile) issue(tile + 1, (tile + 1) & 1);
        if constexpr (MODE == 1)
            if (tile > 0) finish(tile - 1);
        if (!tok) continue;
        const int kb = tile * TM;
#pragma unroll 1
        for (int half = 0; half < 2; ++half) {
            // S^T[key][head] for keys kb + 32 half + 16 kt + 4g + r, heads 16 hq + c16
            v4f S[2][2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int hq = 0; hq < 2; ++hq) S[kt][hq] = v4f{0.f, 0.f, 0.f, 0.f};
            const uint8_t* rb = tb + (half * 32 + c16) * T_LROW;
            const uint8_t* rr = tb + T_ROPE + T_RROW * (half * 32 + c16);
            int qo[4], ro[2];
#pragma unroll
            for (int b = 0; b < 4; ++b) qo[b] = ((4 * b + g) ^ t_latx(c16)) << 4;
#pragma unroll
            for (int b = 0; b < 2; ++b) ro[b] = ((4 * b + g) ^ t_ropex(c16)) << 4;
            constexpr int QD = 3;
            u32x4 abuf[QD][2];
#pragma unroll
            for (int s = 0; s < QD; ++s)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    abuf[s][kt] = *reinterpret_cast<const u32x4*>(rb + kt * 16 * T_LROW + 256 * (s >> 2) + qo[s & 3]);
#pragma unroll
            for (int s = 0; s < 18; ++s) {
                __builtin_amdgcn_sched_barrier(0);
                u32x4 a[2] = {abuf[s % QD][0], abuf[s % QD][1]};
                if (s + QD < 18) {
                    const int m = s + QD;
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
                        abuf[s % QD][kt] = *reinterpret_cast<const u32x4*>(
                            m < 16 ? rb + kt * 16 * T_LROW + 256 * (m >> 2) + qo[m & 3]
                                   : rr + kt * 16 * T_RROW + ro[m & 1]);
                }
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int hq = 0; hq < 2; ++hq)
                        S[kt][hq] = mfma_bf16(as_bf16x8(a[kt]), as_bf16x8(qreg[hq][s]), S[kt][hq]);
            }
            __builtin_amdgcn_sched_barrier(0);
            const int key0 = kb + half * 32 + 4 * g;    // + 16 kt + r
            if constexpr (MODE == 0) {
#pragma unroll
                for (int hq = 0; hq < 2; ++hq) {
                    float x[2][4];
                    float mloc = -__builtin_huge_valf();
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            x[kt][r] = key0 + 16 * kt + r <= p ? S[kt][hq][r] : -__builtin_huge_valf();
                            mloc = fmaxf(mloc, x[kt][r]);
                        }
                    mloc = max_xor32(max_xor16(mloc)) * scale2;
                    if (mloc == -__builtin_huge_valf()) continue;   // no visible key here
                    const float m_new = fmaxf(m_run[hq], mloc);
                    float acc = l_run[hq] * __builtin_amdgcn_exp2f(m_run[hq] - m_new);
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc += __builtin_amdgcn_exp2f(fmaf(x[kt][r], scale2, -m_new));
                    l_run[hq] = acc;
                    m_run[hq] = m_new;
                }
            } else {
                // head sums of exp(logit - lse) for keys key0 + 16 kt + r
                float e[2][4];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float v = 0.f;
                        if (key0 + 16 * kt + r <= p) {
#pragma unroll
                            for (int hq = 0; hq < 2; ++hq)
                                v += __builtin_amdgcn_exp2f(fmaf(S[kt][hq][r], scale2, -lse2[hq]));
                        }
                        e[kt][r] = sum_row16(v);
                    }
                float* red = s_red[tile & 1][tt][hw];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (c16 == 4 * kt + r) red[half * 32 + 16 * kt + 4 * g + r] = e[kt][r];
            }
        }
    }
    if constexpr (MODE == 1) {
        __syncthreads();
        finish(ntile - 1);
    } else if (tok) {
#pragma unroll
        for (int hq = 0; hq < 2; ++hq) {
            float l_tot = l_run[hq] + shfl_xor_f(l_run[hq], 16);
            l_tot += shfl_xor_f(l_tot, 32);
            const int hh = hw * 32 + hq * 16 + c16;
            if (g == 0 && hh < H)
                lse[(int64_t)t * H + hh] = (m_run[hq] + __log2f(l_tot)) * W_LN2;
        }
    }
}

// ------------------------------------------------------------------ row: G and kl
__device__ __forceinline__ float block_reduce(float v, float* sh, bool is_max)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float u = shfl_xor_f(v, o);
        v = is_max ? fmaxf(v, u) : v + u;
    }
    __syncthreads();
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    v = sh[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) v = is_max ? fmaxf(v, sh[w]) : v + sh[w];
    return v;
}

__global__ __launch_bounds__(256) void row_kernel(const float* __restrict__ I, float* __restrict__ PG,
                                                  int64_t ld, int q_pos0, float* __restrict__ kl,
                                                  float* __restrict__ lse_i)
{
    __shared__ float sh[4];
    const int t = blockIdx.x;
    const int n = q_pos0 + t + 1;
    const float* ir = I + (int64_t)t * ld;
    float* pr = PG + (int64_t)t * ld;
    float m = -__builtin_huge_valf();
    for (int s = threadIdx.x; s < n; s += 256) m = fmaxf(m, ir[s]);
    m = block_reduce(m, sh, true);
    float z = 0.f;
    for (int s = threadIdx.x; s < n; s += 256) z += __expf(ir[s] - m);
    z = block_reduce(z, sh, false);
    const float lse = m + __logf(z);
    float acc = 0.f;
    for (int s = threadIdx.x; s < n; s += 256) {
        const float lq = ir[s] - lse;
        const float pv = pr[s];
        pr[s] = __expf(lq) - pv;
        if (pv > 0.f) acc += pv * (__logf(pv) - lq);
    }
    acc = block_reduce(acc, sh, false);
    if (threadIdx.x == 0) {
        kl[t] = acc;
        if (lse_i) lse_i[t] = lse;
    }
}

// ---------------------------------------------------------------- backward through the indexer
constexpr int BK = 64;                        // keys (dq) or rows (dk) per streamed tile
constexpr int F8ROW = 144;                    // fp8 tile row stride (bytes)
constexpr int BFROW = 288;                    // bf16 tile row stride (bytes)

// 16 fp8 bytes -> 16 bf16 (exact), as 8 packed words
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4& v, uint32_t (&o)[8])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
        const v2bf lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[i], 1.0f, false);
        const v2bf hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[i], 1.0f, true);
        o[2 * i] = __builtin_bit_cast(uint32_t, lo);
        o[2 * i + 1] = __builtin_bit_cast(uint32_t, hi);
    }
}

// bf16 A operand of a 16x16x32 MFMA whose K runs over rows of a row-major bf16 tile (stride
// BFROW bytes): row block 32 pr, element 4 kt + r <-> row 32 pr + 16 kt + 4 g + r; M index
// c16 <-> element 16 n + c16 of the row
__device__ __forceinline__ u32x4 tr_operand(const uint8_t* tile, int pr, int n, int g, int c16)
{
    const uint8_t* a = tile + (32 * pr + 4 * g + (c16 >> 2)) * BFROW + 2 * (16 * n + 4 * (c16 & 3));
    const u32x2 lo = ds_read_tr(a);
    const u32x2 hi = ds_read_tr(a + 16 * BFROW);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// e -> bf16 B operand (round to nearest even), elements in the K order of the accumulators
__device__ __forceinline__ u32x4 pack_e(const float (&e)[2][4])
{
    const v8bf b = __builtin_convertvector(
        (v8f){e[0][0], e[0][1], e[0][2], e[0][3], e[1][0], e[1][1], e[1][2], e[1][3]}, v8bf);
    return __builtin_bit_cast(u32x4, b);
}

// dq / dw.  Workgroup: 8 waves (two per SIMD) x 32 rows of the T * H_I (token, head) rows
// (H_I >= 16: a 16-row tile is one token); keys 0 .. p_last in 64-key tiles staged once for
// all eight waves.  G ks is staged per (token, key), so a lane reads the four consecutive keys
// of its accumulator rows in one 16-byte read.
__global__ __launch_bounds__(512) void dq_kernel(const uint8_t* __restrict__ q8,
                                                 const float* __restrict__ qs,
                                                 const float* __restrict__ w,
                                                 const uint8_t* __restrict__ k8,
                                                 const float* __restrict__ ks,
                                                 const float* __restrict__ G, int64_t ld, int T,
                                                 int H_I, int q_pos0, float c,
                                                 float* __restrict__ dq, float* __restrict__ dw)
{
    constexpr int TOKS = 16;
    constexpr int NJ = 2;
    __shared__ __attribute__((aligned(16))) uint8_t s_k8[2][BK * F8ROW];
    __shared__ __attribute__((aligned(16))) uint8_t s_kb[2][BK * BFROW];
    __shared__ __attribute__((aligned(16))) float s_gk[2][TOKS][BK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int shift = 31 - __builtin_clz(H_I);
    const int blk = gridDim.x - 1 - blockIdx.x;
    const int row0 = blk * 256;
    const int64_t nrows = (int64_t)T * H_I;
    const int tok0 = row0 >> shift;
    const int ntok = min(256 >> shift, T - tok0);
    const int p_last = q_pos0 + tok0 + ntok - 1;
    const int ntile = p_last / BK + 1;

    v8i qb[NJ];
    int tokj[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int64_t R = row0 + wave * 32 + 16 * j + c16;
        const u32x4* src = reinterpret_cast<const u32x4*>(q8 + min(R, nrows - 1) * 128 + 32 * g);
        qb[j] = as_i8(src[0], src[1]);
        tokj[j] = min(((row0 + wave * 32 + 16 * j) >> shift) - tok0, TOKS - 1);
    }
    v4f acc[NJ][8];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[j][n] = v4f{0.f, 0.f, 0.f, 0.f};
    float dwp[NJ] = {0.f, 0.f};

    // staging: 64 keys x 8 parts of 16 bytes, one per thread (key tid/8, part tid%8); G ks:
    // 16 tokens x 64 keys, two per thread, both at key tid%64
    const int sk = tid >> 3, sp = tid & 7;
    u32x4 pre;
    float pre_g[2];
    auto gload = [&](int tile) {
        const int kb = tile * BK;
        pre = *reinterpret_cast<const u32x4*>(k8 + (int64_t)min(kb + sk, p_last) * 128 + 16 * sp);
        const int s = kb + (tid & 63);
        const float ksv = ks[min(s, p_last)];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tk = (tid >> 6) + 8 * i;
            pre_g[i] = (tk < ntok && s <= q_pos0 + tok0 + tk)
                           ? G[(int64_t)(tok0 + tk) * ld + s] * ksv : 0.f;
        }
    };
    auto lstore = [&](int buf) {
        *reinterpret_cast<u32x4*>(&s_k8[buf][sk * F8ROW + 16 * sp]) = pre;
        uint32_t o[8];
        fp8x16_to_bf16(pre, o);
        u32x4* d = reinterpret_cast<u32x4*>(&s_kb[buf][sk * BFROW + 32 * sp]);
        d[0] = u32x4{o[0], o[1], o[2], o[3]};
        d[1] = u32x4{o[4], o[5], o[6], o[7]};
#pragma unroll
        for (int i = 0; i < 2; ++i) s_gk[buf][(tid >> 6) + 8 * i][tid & 63] = pre_g[i];
    };

    gload(0);
    lstore(0);
    __syncthreads();
#pragma unroll 1
    for (int tile = 0; tile < ntile; ++tile) {
        const int buf = tile & 1;
        if (tile + 1 < ntile) gload(tile + 1);
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            v4f D[2][NJ];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const u32x4* a = reinterpret_cast<const u32x4*>(
                    &s_k8[buf][(32 * pr + 16 * kt + c16) * F8ROW + 32 * g]);
                const v8i ka = as_i8(a[0], a[1]);
#pragma unroll
                for (int j = 0; j < NJ; ++j) D[kt][j] = mfma_f8(ka, qb[j], v4f{0.f, 0.f, 0.f, 0.f});
            }
            u32x4 eb[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                float e[2][4];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    const v4f gk = *reinterpret_cast<const v4f*>(
                        &s_gk[buf][tokj[j]][32 * pr + 16 * kt + 4 * g]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float d = D[kt][j][r];
                        e[kt][r] = d > 0.f ? gk[r] : 0.f;
                        dwp[j] = fmaf(e[kt][r], d, dwp[j]);
                    }
                }
                eb[j] = pack_e(e);
            }
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const u32x4 ka = tr_operand(s_kb[buf], pr, n, g, c16);
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[j][n] = mfma_bf16(as_bf16x8(ka), as_bf16x8(eb[j]), acc[j][n]);
            }
        }
        if (tile + 1 < ntile) lstore(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int64_t R = row0 + wave * 32 + 16 * j + c16;
        float d = dwp[j] + shfl_xor_f(dwp[j], 16);
        d += shfl_xor_f(d, 32);
        if (R >= nrows) continue;
        const float cw = c * w[R];
        float* o = dq + R * 128;
#pragma unroll
        for (int n = 0; n < 8; ++n)
            *reinterpret_cast<v4f*>(o + 16 * n + 4 * g) = acc[j][n] * cw;
        if (g == 0) dw[R] = c * qs[R] * d;
    }
}

// dk.  Grid: x = blocks of 256 keys, y = groups of 16 indexer heads.  Eight waves (two per
// SIMD) hold 32 keys each as fp8 B operands; the (token, head) rows of the group for the tokens
// that see the block are streamed in 64-row tiles (4 tokens x 16 heads).  Each (group, key) is
// owned by one workgroup per launch, which adds its sum into dkp[group] (accumulated across
// query chunks; dk = the sum over groups, formed once at the end).
__global__ __launch_bounds__(512) void dk_kernel(const uint8_t* __restrict__ q8,
                                                 const float* __restrict__ qs,
                                                 const float* __restrict__ w,
                                                 const uint8_t* __restrict__ k8,
                                                 const float* __restrict__ G, int64_t ld, int T,
                                                 int H_I, int q_pos0, float c, int64_t L,
                                                 float* __restrict__ dkp)
{
    constexpr int TPT = 4;
    constexpr int NK = 2;
    __shared__ __attribute__((aligned(16))) uint8_t s_q8[2][BK * F8ROW];
    __shared__ __attribute__((aligned(16))) uint8_t s_qb[2][BK * BFROW];
    __shared__ __attribute__((aligned(16))) float s_wq[2][BK];
    __shared__ float s_g[2][TPT][256];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int s0 = blockIdx.x * 256;
    const int hg = blockIdx.y;
    const int sw = s0 + wave * 32;
    const int64_t nrows = (int64_t)T * H_I;
    const int tmin = max(0, s0 - q_pos0);
    if (tmin >= T) return;
    const int ntile = (T - tmin + TPT - 1) / TPT;

    v8i kb8[NK];
#pragma unroll
    for (int jk = 0; jk < NK; ++jk) {
        const int s = min(sw + 16 * jk + c16, q_pos0 + T - 1);
        const u32x4* src = reinterpret_cast<const u32x4*>(k8 + (int64_t)s * 128 + 32 * g);
        kb8[jk] = as_i8(src[0], src[1]);
    }
    v4f acc[NK][8];
#pragma unroll
    for (int jk = 0; jk < NK; ++jk)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[jk][n] = v4f{0.f, 0.f, 0.f, 0.f};

    // staging: tile row rl = 16 tk + hl is (token tmin + 4 tile + tk, head 16 hg + hl); one
    // 16-byte part per thread (row tid/8, part tid%8)
    const int sr = tid >> 3, sp = tid & 7;
    auto row_of = [&](int tile, int rl, bool& ok) -> int64_t {
        const int t = tmin + TPT * tile + (rl >> 4);
        ok = t < T;
        return ok ? (int64_t)t * H_I + 16 * hg + (rl & 15) : nrows - 1;
    };
    u32x4 pre;
    float pre_wq = 0.f, pre_g[2];
    auto gload = [&](int tile) {
        bool ok;
        const int64_t R = row_of(tile, sr, ok);
        pre = *reinterpret_cast<const u32x4*>(q8 + R * 128 + 16 * sp);
        if (tid < BK) {
            const int64_t R2 = row_of(tile, tid, ok);
            pre_wq = ok ? w[R2] * qs[R2] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = tid + 512 * i;
            const int t = tmin + TPT * tile + (e >> 8);
            const int key = s0 + (e & 255);
            pre_g[i] = (t < T && key <= q_pos0 + t) ? G[(int64_t)t * ld + key] : 0.f;
        }
    };
    auto lstore = [&](int buf) {
        *reinterpret_cast<u32x4*>(&s_q8[buf][sr * F8ROW + 16 * sp]) = pre;
        uint32_t o[8];
        fp8x16_to_bf16(pre, o);
        u32x4* d = reinterpret_cast<u32x4*>(&s_qb[buf][sr * BFROW + 32 * sp]);
        d[0] = u32x4{o[0], o[1], o[2], o[3]};
        d[1] = u32x4{o[4], o[5], o[6], o[7]};
        if (tid < BK) s_wq[buf][tid] = pre_wq;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = tid + 512 * i;
            s_g[buf][e >> 8][e & 255] = pre_g[i];
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();
#pragma unroll 1
    for (int tile = 0; tile < ntile; ++tile) {
        const int buf = tile & 1;
        if (tile + 1 < ntile) gload(tile + 1);
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            v4f D[2][NK];
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                const u32x4* a = reinterpret_cast<const u32x4*>(
                    &s_q8[buf][(32 * pr + 16 * jt + c16) * F8ROW + 32 * g]);
                const v8i qa = as_i8(a[0], a[1]);
#pragma unroll
                for (int jk = 0; jk < NK; ++jk) D[jt][jk] = mfma_f8(qa, kb8[jk], v4f{0.f, 0.f, 0.f, 0.f});
            }
            v4f wq[2];
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
                wq[jt] = *reinterpret_cast<const v4f*>(&s_wq[buf][32 * pr + 16 * jt + 4 * g]);
            u32x4 eb[NK];
#pragma unroll
            for (int jk = 0; jk < NK; ++jk) {
                float e[2][4];
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
                    const float gv = s_g[buf][2 * pr + jt][wave * 32 + 16 * jk + c16];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        e[jt][r] = D[jt][jk][r] > 0.f ? gv * wq[jt][r] : 0.f;
                }
                eb[jk] = pack_e(e);
            }
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const u32x4 qa = tr_operand(s_qb[buf], pr, n, g, c16);
#pragma unroll
                for (int jk = 0; jk < NK; ++jk)
                    acc[jk][n] = mfma_bf16(as_bf16x8(qa), as_bf16x8(eb[jk]), acc[jk][n]);
            }
        }
        if (tile + 1 < ntile) lstore(buf ^ 1);
        __syncthreads();
    }

    float* part = dkp + (int64_t)hg * L * 128;
#pragma unroll
    for (int jk = 0; jk < NK; ++jk) {
        const int s = sw + 16 * jk + c16;
        if (s > q_pos0 + T - 1) continue;
        float* o = part + (int64_t)s * 128;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            v4f* d = reinterpret_cast<v4f*>(o + 16 * n + 4 * g);
            *d = *d + acc[jk][n] * c;
        }
    }
}

// dk[i] = sum over groups of dkp[group][i]
__global__ void dk_reduce_kernel(const float* __restrict__ dkp, int ngroups, int64_t n,
                                 float* __restrict__ dk)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        float v = 0.f;
        for (int gq = 0; gq < ngroups; ++gq) v += dkp[gq * n + i];
        dk[i] = v;
    }
}

__global__ void zero_kernel(float* __restrict__ p, int64_t n)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

}  // namespace

bool warmup_supports(int H_I, int H)
{
    return (H_I == 16 || H_I == 32 || H_I == 64 || H_I == 128) && H >= 1 && H <= 128;
}

hipError_t launch_attention_lse(const uint16_t* q, const uint16_t* kv, int T, int H, int q_pos0,
                                float sm_scale, float* lse, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(teacher_kernel<0>, dim3((T + 1) / 2), dim3(512), 0, stream, q, kv, T, H,
                       q_pos0, sm_scale, lse, nullptr, (int64_t)0);
    return hipGetLastError();
}

hipError_t launch_attention_dist(const uint16_t* q, const uint16_t* kv, const float* lse, int T,
                                 int H, int q_pos0, float sm_scale, float* P, int64_t ld,
                                 hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(teacher_kernel<1>, dim3((T + 1) / 2), dim3(512), 0, stream, q, kv, T, H,
                       q_pos0, sm_scale, const_cast<float*>(lse), P, ld);
    return hipGetLastError();
}

hipError_t launch_warmup_rows(const float* I, float* PG, int64_t ld, int T, int q_pos0,
                              float* kl, float* lse_i, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(row_kernel, dim3(T), dim3(256), 0, stream, I, PG, ld, q_pos0, kl, lse_i);
    return hipGetLastError();
}

hipError_t launch_warmup_dq(const uint8_t* q8, const float* qs, const float* w, const uint8_t* k8,
                            const float* ks, const float* G, int64_t ld, int T, int H_I,
                            int q_pos0, float c, float* dq, float* dw, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    const int64_t rows = (int64_t)T * H_I;
    hipLaunchKernelGGL(dq_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(512), 0, stream, q8,
                       qs, w, k8, ks, G, ld, T, H_I, q_pos0, c, dq, dw);
    return hipGetLastError();
}

hipError_t launch_warmup_dk(const uint8_t* q8, const float* qs, const float* w, const uint8_t* k8,
                            const float* G, int64_t ld, int T, int H_I, int q_pos0, float c,
                            int64_t L, float* dkp, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    const int keys = q_pos0 + T;                       // keys any row sees
    hipLaunchKernelGGL(dk_kernel, dim3((keys + 255) / 256, H_I / 16), dim3(512), 0, stream, q8,
                       qs, w, k8, G, ld, T, H_I, q_pos0, c, L, dkp);
    return hipGetLastError();
}

hipError_t launch_warmup_dk_reduce(const float* dkp, int ngroups, int64_t n, float* dk,
                                   hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(dk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dkp,
                       ngroups, n, dk);
    return hipGetLastError();
}

hipError_t launch_zero(float* p, int64_t n, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

}  // namespace dsa
