// sparse_mla.hip -- attention over the selected latent rows on gfx950.
//
// For query row t and head h: logits l_j = sm_scale * <q[t,h,:576], kv[I_j,:576]> over the
// selected rows I = idx[t,:], softmax within I, output sum_j p_j kv[I_j,:512] with the
// 512-d latent doubling as the value (《DeepSeek-V3.2-Exp模型优势与 DSA 工作原理》 §3 稀疏
// MLA and §4 步骤四; 《狂降75%！…》 §三 第四步).
//
// One workgroup handles one query row for all heads over a contiguous slice of its index
// list: four waves (128 head slots), one wave per SIMD with the full 512-register file.  The
// selected 1152-byte rows are gathered 64 at a time by direct global->LDS loads into a
// double-buffered tile, so the next tile streams in while the current one is used.  A tile
// holds the rows' 512 latent dims as [64 rows][1024 B] and their 64 rope dims as
// [64 rows][128 B], 16-byte chunks XOR-swizzled by row: one gather instruction moves one
// row's latent part (a wave-uniform scalar base address plus a fixed per-lane chunk offset)
// or the rope parts of eight rows, so issuing the gather costs a few scalar instructions per
// row.  LDS read bandwidth, not MFMA, bounds the arithmetic, so the two contractions split
// the work to minimise LDS reads:
//  * S^T = K Q^T: wave w owns 32 heads (A = gathered rows, each 16-byte operand read feeding
//    two MFMAs; B = Q^T held in registers) and their softmax, and writes P (bf16, already
//    in the A-operand layout of P V) to LDS;
//  * O = P V: wave w owns 128 of the value dims for every head, so each V element is read
//    (by the transposing read ds_read_b64_tr_b16, half the rate of a plain 16-byte read) by
//    one wave only, and P by every wave (plain 16-byte reads).
// Softmax runs in the exp2 domain with fp32 statistics against a per-head reference max
// fixed by the first valid logits of the row; O is never rescaled, which is what lets other
// waves accumulate a head's P V.  Should a later logit exceed the reference by more than
// 2^OVF_SLACK (a logit spread no real attention row reaches), the row is recomputed once
// with the exact per-head max as the reference.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int MT = 64;                       // keys per tile
constexpr int CH = 72;                       // 16-byte chunks per 1152-byte row
constexpr int TILE_BYTES = MT * CH * 16;     // 73,728
constexpr int LROW = 1024;                   // latent bytes per row (dims 0..511)
constexpr int ROPE_OFF = MT * LROW;          // rope part of a tile: [MT rows][128 B]
constexpr int RROW = 128;                    // rope bytes per row (dims 512..575)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
// Headroom of the fixed softmax reference (log2 units): p = 2^(x - m_ref) <= 2^64, so the
// row sum stays below 2^77 for k <= 8192 and fp32 keeps its relative precision throughout.
constexpr float OVF_SLACK = 64.f;

// Tile layout.  Latent dims [8c, 8c + 8) of row r (16-byte chunk c < 64) sit at byte
// row_base(r) + 16 (c ^ lat_x(r)); rope chunk b < 8 (dims 512 + 8b ..) at
// ROPE_OFF + RROW r + 16 (b ^ rope_x(r)).  lat_x only touches chunk bits 1-3, so for
// c = 16a + b the offset is a per-lane part for b plus the immediate 256 a.  With these
// permutations the reads below are free of LDS bank conflicts (measured on gfx950, where a
// 16-byte read serves lanes {0-7, 24-31}, {8-15, 16-23} and likewise in the upper half
// together): the K operand reads (16 rows at one chunk per instruction, latent and rope) and
// the transposing V reads (8-byte pieces of 8 rows, a 32-byte chunk pair per row).
__device__ __forceinline__ int row_base(int r) { return r * LROW; }
__device__ __forceinline__ int lat_x(int r) { return (r & 7) << 1; }
__device__ __forceinline__ int rope_x(int r) { return (r >> 1) & 7; }

// NW waves; wave w: heads [32w, 32w + 32) in S^T / softmax (two 16-head groups hq), 16-dim
// blocks [DPW w, DPW w + DPW) of O for all 2 NW head groups in P V.
template <int NW>
__global__ __launch_bounds__(NW * 64) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ idx, const int64_t* __restrict__ seq_start, int L, int H, int k,
    float sm_scale, int splits, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse, int valid_pos0)
{
    constexpr int NG = 2 * NW;                         // 16-head groups
    constexpr int DPW = 32 / NW;                       // 16-dim blocks of O per wave
    // P of one tile: [head group][32-key step][lane][8 bf16], the PV A-operand layout
    __shared__ __attribute__((aligned(16))) uint8_t s_tile[2][TILE_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t s_p[NG * 2 * 64 * 16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    // prefill rows later in a launch see at least as many keys: start the heaviest first
    const int row = seq_start ? (int)blockIdx.x : (int)(gridDim.x - 1 - blockIdx.x);
    const int split = blockIdx.y;
    const int n0 = wave * DPW;                         // first 16-dim block of O owned here

    int64_t kv_base = 0;
    int Lr = L;
    if (seq_start) {
        kv_base = seq_start[row];
        Lr = (int)(seq_start[row + 1] - kv_base);
    }
    const uint16_t* kvr = kv + kv_base * 576;
    // valid_pos0 >= 0: the row's list is a top-k selection, its valid entries first (min(k,
    // valid_pos0 + row + 1) of them for a prefill row at position valid_pos0 + row, min(k, Lr)
    // for a decode row over its cache), so the padding after them is not visited; otherwise
    // padding may sit anywhere among the k entries
    const int kr = valid_pos0 < 0 ? k : seq_start ? min(k, Lr) : min(k, valid_pos0 + row + 1);
    const int per = (kr + splits - 1) / splits;
    const int jbeg = split * per;
    const int nkeys = max(0, min(kr, jbeg + per) - jbeg);
    const int ntile = (nkeys + MT - 1) / MT;
    const int32_t* idxr = idx + (int64_t)row * k + jbeg;

    // B operand of S^T: Q^T, lane holds head 32 wave + 16 hq + c16, dims [32s + 8g, +8)
    u32x4 qreg[2][18];
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
        const int hh = wave * 32 + hq * 16 + c16;
        const bool hv = hh < H;
        const uint16_t* qh = q + ((int64_t)row * H + (hv ? hh : 0)) * 576;
#pragma unroll
        for (int s = 0; s < 18; ++s)
            qreg[hq][s] = hv ? *reinterpret_cast<const u32x4*>(qh + 32 * s + 8 * g)
                             : u32x4{0u, 0u, 0u, 0u};
    }
    // Q^T complete before the tile loop: the compiler would otherwise place its wait for these
    // loads inside the loop, as a full vector-memory wait that also drains the gathers
    __builtin_amdgcn_s_waitcnt(0);
    const float scale2 = sm_scale * LOG2E;

    // index of key t*MT + lane of the slice: loaded raw (from a clamped, always valid
    // address, so that no wait is forced before the value is used) and checked at use
    // (-1: past the slice, padding or out of range)
    auto load_idx = [&](int t) -> int {
        return idxr[min(t * MT + lane, max(nkeys - 1, 0))];
    };
    auto check_idx = [&](int t, int s) -> int {
        return (t * MT + lane < nkeys && s >= 0 && s < Lr) ? s : -1;
    };
    // Gather of a tile into dst (tidx: lane r holds row r's index, -1 for padding, which loads
    // row 0 and is masked later).  Latent parts: wave w moves rows [RPW w, RPW w + RPW), one
    // instruction per row, lane l loading the source chunk stored in slot l (chunk
    // l ^ lat_x(r)).  Rope parts: instruction j moves rows 8j .. 8j+7, lane l row 8j + l/8,
    // slot l%8, i.e. source chunk 64 + ((l%8) ^ rope_x(8j + l/8)) = 64 + ((l%8) ^ (4 (j%2) + l/16)).
    constexpr int RPW = MT / NW;                       // latent rows per wave
    constexpr int JPW = 8 / NW;                        // rope instructions per wave
    static_assert(JPW % 2 == 0 && RPW % 8 == 0, "rope instruction parity and row groups per wave");
    const uint32_t rope_src[2] = {16u * (64u + (uint32_t)((lane & 7) ^ (lane >> 4))),
                                  16u * (64u + (uint32_t)((lane & 7) ^ (4 + (lane >> 4))))};
    const uint32_t lds_tiles = __builtin_amdgcn_readfirstlane(lds_addr(s_tile[0]));
    auto issue = [&](int buf, int tidx) {
        const uint32_t dst = lds_tiles + (uint32_t)buf * TILE_BYTES;
#pragma unroll 2
        for (int i0 = 0; i0 < RPW; i0 += 8)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = wave * RPW + i0 + i;         // r & 7 == i: lat_x(r) = 2 i
                const int sx = max(__builtin_amdgcn_readlane(tidx, r), 0);
                dma16_s(16u * (uint32_t)(lane ^ (2 * i)), kvr + (int64_t)sx * 576, dst + r * LROW);
            }
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
            const int j = wave * JPW + jj;
            const int sx = max(__builtin_amdgcn_ds_bpermute((8 * j + (lane >> 3)) * 4, tidx), 0);
            dma16(reinterpret_cast<const uint8_t*>(kvr + (int64_t)sx * 576) + rope_src[jj & 1],
                  dst + ROPE_OFF + j * 1024);
        }
    };

    v4f O[NG][DPW];                     // O[hg][d]: heads 16 hg + 4g + r, dims 16 (n0 + d) + c16
    float m_ref[2], m_max[2] = {-__builtin_huge_valf(), -__builtin_huge_valf()}, l_run[2];

#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int hg = 0; hg < NG; ++hg)
#pragma unroll
            for (int d = 0; d < DPW; ++d) O[hg][d] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hq = 0; hq < 2; ++hq) {
            l_run[hq] = 0.f;
            m_ref[hq] = pass ? m_max[hq] : -__builtin_huge_valf();
        }
        bool over = false;
        int idx_cur = 0, idx_nxt = 0;
        if (ntile > 0) {
            idx_cur = check_idx(0, load_idx(0));
            idx_nxt = load_idx(1);
            issue(0, idx_cur);
        }
        // one tile: tb holds it, the other buffer receives the next one
        auto step = [&](int t, const uint8_t* tb) {
            __builtin_amdgcn_s_waitcnt(0);             // this wave's part of tile t landed
            __syncthreads();                           // everyone's part; tile t-1 and P consumed
            const uint64_t vmask = __ballot(idx_cur >= 0);
            idx_nxt = check_idx(t + 1, idx_nxt);
            if (t + 1 < ntile) issue((t + 1) & 1, idx_nxt);
            idx_cur = idx_nxt;
            idx_nxt = load_idx(t + 2);
#pragma unroll 1
            for (int half = 0; half < 2; ++half) {
                // S^T[key][head] for keys 32 half + 16 kt + (4g + r), heads 16 hq + c16;
                // A = row 32 half + 16 kt + c16, dims [32s + 8g, +8): chunk 4s + g, each A
                // read feeding both head groups; A operands read QD steps ahead
                v4f S[2][2];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int hq = 0; hq < 2; ++hq) S[kt][hq] = v4f{0.f, 0.f, 0.f, 0.f};
                const uint8_t* rb = tb + row_base(half * 32 + c16);    // kt adds 16 rows
                const uint8_t* rr = tb + ROPE_OFF + RROW * (half * 32 + c16);
                // latent chunk 4m + g = 16 (m/4) + (4 (m%4) + g): per-lane offsets for m%4,
                // rope chunk 4 (m - 16) + g for m = 16, 17 (row & 7 == c16 & 7 and
                // (row >> 1) & 7 == c16 >> 1 for these rows)
                int qo[4], ro[2];
#pragma unroll
                for (int b = 0; b < 4; ++b) qo[b] = ((4 * b + g) ^ lat_x(c16)) << 4;
#pragma unroll
                for (int b = 0; b < 2; ++b) ro[b] = ((4 * b + g) ^ rope_x(c16)) << 4;
                // Software pipeline with fixed stages: stage s issues the reads of step s + QD
                // and the four MFMAs of step s; the scheduling barriers keep the compiler from
                // collapsing it into read -> wait -> MFMA (one wave per SIMD leaves nothing
                // else to hide LDS latency).
                constexpr int QD = 3;
                u32x4 abuf[QD][2];
#pragma unroll
                for (int s = 0; s < QD; ++s)
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
                        abuf[s][kt] = *reinterpret_cast<const u32x4*>(rb + kt * 16 * LROW + 256 * (s >> 2) + qo[s & 3]);
#pragma unroll
                for (int s = 0; s < 18; ++s) {
                    __builtin_amdgcn_sched_barrier(0);
                    u32x4 a[2] = {abuf[s % QD][0], abuf[s % QD][1]};
                    if (s + QD < 18) {
                        const int m = s + QD;
#pragma unroll
                        for (int kt = 0; kt < 2; ++kt)
                            abuf[s % QD][kt] = *reinterpret_cast<const u32x4*>(
                                m < 16 ? rb + kt * 16 * LROW + 256 * (m >> 2) + qo[m & 3]
                                       : rr + kt * 16 * RROW + ro[m & 1]);
                    }
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int hq = 0; hq < 2; ++hq)
                            S[kt][hq] = mfma_bf16(as_bf16x8(a[kt]), as_bf16x8(qreg[hq][s]), S[kt][hq]);
                }
                __builtin_amdgcn_sched_barrier(0);
                // softmax for heads 16 hq + c16 over this half's 32 keys
#pragma unroll
                for (int hq = 0; hq < 2; ++hq) {
                    // raw logits (masked: -inf); the scale is applied inside the exponent's
                    // fma, and to the maximum once: scale2 > 0 and rounding is monotonic, so
                    // max(x) * scale2 is exactly the maximum of the rounded x * scale2
                    float x[2][4];
                    float mloc = -__builtin_huge_valf();
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
                        const uint32_t bits = (uint32_t)(vmask >> (half * 32 + kt * 16 + 4 * g));
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            x[kt][r] = ((bits >> r) & 1u) ? S[kt][hq][r] : -__builtin_huge_valf();
                            mloc = fmaxf(mloc, x[kt][r]);
                        }
                    }
                    mloc = max_xor32(max_xor16(mloc)) * scale2;
                    m_max[hq] = fmaxf(m_max[hq], mloc);
                    // the first valid logits fix the reference (O and l are still zero then)
                    if (m_ref[hq] == -__builtin_huge_valf()) m_ref[hq] = mloc;
                    over |= mloc > m_ref[hq] + OVF_SLACK;
                    // no valid logit yet: keep exp2(-inf - m) = 0 rather than exp2(-inf + inf)
                    const float m_sub = m_ref[hq] == -__builtin_huge_valf() ? 0.f : m_ref[hq];
                    float p[2][4];
                    float psum = 0.f;
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            p[kt][r] = __builtin_amdgcn_exp2f(fmaf(x[kt][r], scale2, -m_sub));
                            psum += p[kt][r];
                        }
                    l_run[hq] += psum;
                    // A operand of P V: head c16, K = keys {4g..4g+3} of each 16-key group
                    const v8bf pav = __builtin_convertvector(
                        (v8f){p[0][0], p[0][1], p[0][2], p[0][3], p[1][0], p[1][1], p[1][2], p[1][3]},
                        v8bf);
                    *reinterpret_cast<v8bf*>(&s_p[(((2 * wave + hq) * 2 + half) * 64 + lane) * 16]) = pav;
                }
            }
            __syncthreads();                           // P of every head group visible

            // O[hg][d] += P[hg] V[:, dims of block n0 + d] over the tile's two 32-key steps.
            // V operand: column 16n + c16, keys 32 ks + 16 kt + 4g + r, by transpose reads:
            // lane (g, i) addresses row 32 ks + 16 kt + 4g + i/4, dims 16n + 4(i%4) .. +3,
            // i.e. chunk 2n + (i%4)/2 = 8(n/4) + (2(n%4) + (i%4)/2), byte 8 (i%2) within it
            const int cpart = (c16 & 3) >> 1, boff = (c16 & 1) * 8;
            const int rv = 4 * g + (c16 >> 2);         // row within each 16-key group
            // physical chunk (2n + cpart) ^ lat_x(rv) = 8 ((n/4) ^ vq) + 2 ((n%4) ^ (rv%4)) + cpart
            const int vq = (rv >> 2) & 1;
            int vo[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) vo[j] = 32 * (j ^ (rv & 3)) + 16 * cpart;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int vrow = row_base(ks * 32 + rv) + boff;
                // V operands of DC owned blocks held at a time, P streamed per head group
                constexpr int DC = DPW < 8 ? DPW : 8;
#pragma unroll
                for (int d0 = 0; d0 < DPW; d0 += DC) {
                    u32x4 vop[DC];
#pragma unroll
                    for (int d = 0; d < DC; ++d) {
                        const int n = n0 + d0 + d;
                        const int o = vrow + 128 * ((n >> 2) ^ vq) + vo[n & 3];
                        const u32x2 lo = ds_read_tr(tb + o);
                        const u32x2 hi = ds_read_tr(tb + o + 16 * LROW);
                        vop[d] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                    }
                    constexpr int PD = NG < 2 ? NG : 2;
                    u32x4 pbuf[PD];
#pragma unroll
                    for (int hg = 0; hg < PD; ++hg)
                        pbuf[hg] = *reinterpret_cast<const u32x4*>(&s_p[((hg * 2 + ks) * 64 + lane) * 16]);
#pragma unroll
                    for (int hg = 0; hg < NG; ++hg) {
                        __builtin_amdgcn_sched_barrier(0);     // stage hg: P read of hg + PD
                        const u32x4 pa = pbuf[hg % PD];
                        if (hg + PD < NG)
                            pbuf[hg % PD] = *reinterpret_cast<const u32x4*>(&s_p[(((hg + PD) * 2 + ks) * 64 + lane) * 16]);
#pragma unroll
                        for (int d = 0; d < DC; ++d)
                            O[hg][d0 + d] = mfma_bf16(as_bf16x8(pa), as_bf16x8(vop[d]), O[hg][d0 + d]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
#pragma unroll 1
        for (int t = 0; t < ntile; ++t) step(t, s_tile[t & 1]);
        // every wave must agree on a recomputation: flags through LDS
        __syncthreads();                               // last tile's P V done everywhere
        int* s_flag = reinterpret_cast<int*>(s_p);
        const bool wave_over = __any(over);
        if (lane == 0) s_flag[wave] = wave_over ? 1 : 0;
        __syncthreads();
        bool redo = false;
#pragma unroll
        for (int w = 0; w < NW; ++w) redo |= s_flag[w] != 0;
        __syncthreads();                               // flags read before s_p is reused
        if (!redo) break;
    }

    // totals per head (owner wave), shared with the waves holding that head's O columns
    float* s_inv = reinterpret_cast<float*>(s_p);
    float my_lse[2];
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
        float l_tot = l_run[hq] + shfl_xor_f(l_run[hq], 16);
        l_tot += shfl_xor_f(l_tot, 32);
        my_lse[hq] = l_tot > 0.f ? m_ref[hq] * LN2 + logf(l_tot) : -__builtin_huge_valf();
        if (g == 0) s_inv[wave * 32 + hq * 16 + c16] = l_tot > 0.f ? 1.f / l_tot : 0.f;
    }
    __syncthreads();

    if (splits == 1) {
#pragma unroll
        for (int hg = 0; hg < NG; ++hg)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int hh = hg * 16 + 4 * g + r;
                if (hh >= H) continue;
                const float ir = s_inv[hh];
                uint16_t* orow = out + ((int64_t)row * H + hh) * 512;
#pragma unroll
                for (int d = 0; d < DPW; ++d)
                    orow[16 * (n0 + d) + c16] = (uint16_t)bf16_bits(O[hg][d][r] * ir);
            }
        if (lse && g == 0)
#pragma unroll
            for (int hq = 0; hq < 2; ++hq) {
                const int hh = wave * 32 + hq * 16 + c16;
                if (hh < H) lse[(int64_t)row * H + hh] = my_lse[hq];
            }
    } else {
        const int64_t pb = ((int64_t)row * splits + split) * H;
#pragma unroll
        for (int hg = 0; hg < NG; ++hg)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int hh = hg * 16 + 4 * g + r;
                if (hh >= H) continue;
                const float ir = s_inv[hh];
                float* orow = part_o + (pb + hh) * 512;
#pragma unroll
                for (int d = 0; d < DPW; ++d) orow[16 * (n0 + d) + c16] = O[hg][d][r] * ir;
            }
        if (g == 0)
#pragma unroll
            for (int hq = 0; hq < 2; ++hq) {
                const int hh = wave * 32 + hq * 16 + c16;
                if (hh < H) part_lse[pb + hh] = my_lse[hq];
            }
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
                     int valid_pos0, hipStream_t stream)
{
    auto kern = sparse_mla_kernel<NW>;
    hipLaunchKernelGGL(kern, dim3(T, splits), dim3(NW * 64), 0, stream, q, kv, idx, seq_start, L,
                       H, k, sm_scale, splits, out, lse, part_o, part_lse, valid_pos0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                             const int64_t* seq_start, int T, int L, int H, int k,
                             float sm_scale, int splits, uint16_t* out, float* lse,
                             float* part_o, float* part_lse, int valid_pos0, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    // four waves of 32 head slots; fewer heads leave slots empty (their queries read as zero
    // and their outputs are not written): one shape, whose registers fit without spilling
    if (H <= 128)
        return launch_nw<4>(q, kv, idx, seq_start, T, L, H, k, sm_scale, splits, out, lse, part_o,
                            part_lse, valid_pos0, stream);
    return hipErrorInvalidValue;
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
