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
// row.  Wave w owns 32 heads from end to end:
//  * S^T = K Q^T for its heads (A = gathered rows, each 16-byte operand read feeding two
//    MFMAs; B = Q^T held in registers), then their softmax, whose bf16 probabilities come out
//    of the accumulators already in the A-operand layout of P V;
//  * O = P V for its heads over all 512 value dims (V read from the tile by the transposing
//    read ds_read_b64_tr_b16), so P never leaves the wave's registers and the waves meet only
//    once per tile (it has landed; the previous one is consumed).
// Softmax runs in the exp2 domain with fp32 statistics against a per-head reference max
// fixed by the first valid logits of the row, so O is never rescaled.  Should a later logit
// exceed the reference by more than 2^OVF_SLACK (a logit spread no real attention row
// reaches), the row is recomputed once with the exact per-head max as the reference; the test
// uses each lane's running maximum of its raw logits, reduced across lanes once per pass.
// Once the references are fixed, a tile whose 64 keys are all valid runs software-pipelined
// within the wave: the softmax of its first 32 keys is spread over the QK MFMAs of the second
// 32, the softmax of the second over the P V MFMAs of the first (one wave per SIMD keeps
// issuing a few vector instructions under each MFMA), with the arithmetic of each head in
// the same order as the unsplit form, so the results are the same bits.
#include <type_traits>

#include "dsa_device.h"
#include "kernels.h"

namespace dsa {
namespace {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

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

// NW = 4 waves; wave w owns heads [32w, 32w + 32) throughout: S^T = K Q^T for them, their
// softmax, and O = P V over all 512 value dims, so P never leaves the wave's registers and
// the waves meet only once per tile (the tile has landed; the previous one is consumed).
template <int NW>
__global__ __launch_bounds__(NW * 64) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ idx, const int64_t* __restrict__ seq_start, int L, int H, int k,
    float sm_scale, int splits, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse, int valid_pos0)
{
    static_assert(NW == 4, "four waves of 32 heads");
    __shared__ __attribute__((aligned(16))) uint8_t s_tile[2][TILE_BYTES];
    __shared__ int s_flag[NW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    // prefill rows later in a launch see at least as many keys: start the heaviest first
    const int row = seq_start ? (int)blockIdx.x : (int)(gridDim.x - 1 - blockIdx.x);
    const int split = blockIdx.y;

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
    // a gathered row is a 32-bit byte offset from the row's cache (its index times 1152; the
    // launch keeps every cache below 2 GiB, so the offset stays below 2^31), added to the
    // lane's chunk offset: a row's load costs a lane read, one add and the load rather than
    // 64-bit address arithmetic
    auto issue = [&](int buf, int tidx) {
        // the lane's chunk offsets are formed here rather than held across the tile loop
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const uint32_t dst = lds_tiles + (uint32_t)buf * TILE_BYTES;
        const uint32_t roff = (uint32_t)max(tidx, 0) * 1152u;   // lane r: row r's byte offset
#pragma unroll 2
        for (int i0 = 0; i0 < RPW; i0 += 8)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = wave * RPW + i0 + i;         // r & 7 == i: lat_x(r) = 2 i
                dma16_s((uint32_t)__builtin_amdgcn_readlane((int)roff, r) +
                            16u * (uint32_t)(ln ^ (2 * i)), kvr, dst + r * LROW);
            }
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
            const int j = wave * JPW + jj;
            const uint32_t ro = (uint32_t)__builtin_amdgcn_ds_bpermute((8 * j + (lane >> 3)) * 4, (int)roff);
            dma16_s(ro + rope_src[jj & 1], kvr, dst + ROPE_OFF + j * 1024);
        }
    };

    // per-lane offsets of the operand reads (see the tile layout above)
    int qo[4], ro[2];                  // S^T A operand: latent chunk 4m + g, rope chunk 4(m-16) + g
#pragma unroll
    for (int b = 0; b < 4; ++b) qo[b] = ((4 * b + g) ^ lat_x(c16)) << 4;
#pragma unroll
    for (int b = 0; b < 2; ++b) ro[b] = ((4 * b + g) ^ rope_x(c16)) << 4;
    // V operand of P V for dim block n, keys 32 half + 16 kt + 4g + r: transposing reads, lane
    // (g, i) addressing row 32 half + 16 kt + 4g + i/4, dims 16n + 4(i%4) .. +3, i.e. chunk
    // 2n + (i%4)/2 (physical (2n + cpart) ^ lat_x(rv) = 8 ((n/4) ^ vq) + 2 ((n%4) ^ (rv%4)) +
    // cpart), byte 8 (i%2) within it
    const int rv = 4 * g + (c16 >> 2);
    const int vq = (rv >> 2) & 1;
    const int vbase = row_base(rv) + (c16 & 1) * 8;
    int vo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vo[j] = 32 * (j ^ (rv & 3)) + 16 * ((c16 & 3) >> 1);

    v4f O[2][32];                      // O[hq][n]: heads 32 wave + 16 hq + 4g + r, dims 16n + c16
    // m_ref: -inf for the first pass (then fixed by the row's first valid logits); a
    // recomputation pass takes the exact per-head maximum the first pass found
    float m_ref[2] = {-__builtin_huge_valf(), -__builtin_huge_valf()}, l_run[2];
    // each lane's running maximum of its own raw logits (reduced across lanes once per pass)
    float m_lane[2];

    // S^T[key][head] of one half tile (keys 32 half + 16 kt + (4g + r), heads 16 hq + c16):
    // A = row 32 half + 16 kt + c16, dims [32s + 8g, +8) (chunk 4s + g), each A read feeding
    // both head groups, read QD steps ahead; B = Q^T.  The accumulators are pinned in VGPRs
    // (the compiler would place them in AGPRs beside O and shuffle part of O out and back
    // around every half).  between(s) runs inside step s's scheduling region.
    auto qk_half = [&](const uint8_t* tb, int half, v4f (&S)[2][2], auto&& between) {
        const uint8_t* rb = tb + row_base(half * 32 + c16);    // kt adds 16 rows
        const uint8_t* rr = tb + ROPE_OFF + RROW * (half * 32 + c16);
        constexpr int QD = 2;
        u32x4 abuf[QD][2];
#pragma unroll
        for (int s = 0; s < QD; ++s)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                abuf[s][kt] = *reinterpret_cast<const u32x4*>(rb + kt * 16 * LROW + 256 * (s >> 2) + qo[s & 3]);
#pragma unroll
        for (int s = 0; s < 18; ++s) {
            __builtin_amdgcn_sched_barrier(0);
            const u32x4 a[2] = {abuf[s % QD][0], abuf[s % QD][1]};
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
                for (int hq = 0; hq < 2; ++hq) {
                    if (s == 0)
                        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0"
                                     : "=&v"(S[kt][hq]) : "v"(a[kt]), "v"(qreg[hq][s]));
                    else
                        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                                     : "+v"(S[kt][hq]) : "v"(a[kt]), "v"(qreg[hq][s]));
                }
            between(s);
        }
        // no VALU read of the accumulators before the last MFMA has written them: 19 wait
        // states, enough for any MFMA pass count
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2"
                     : "+v"(S[0][0]), "+v"(S[0][1]), "+v"(S[1][0]), "+v"(S[1][1]));
        __builtin_amdgcn_sched_barrier(0);
    };
    // O[hq][n] += P[hq] V[:, 16n .. 16n + 15] over one half's 32 keys, the V operands read VD
    // blocks ahead; between(n) runs inside step n's scheduling region
    auto pv_half = [&](const uint8_t* tb, int half, const u32x4 (&pa)[2], auto&& between) {
        const uint8_t* vb = tb + half * 32 * LROW + vbase;
        constexpr int VD = 4;
        u32x4 vbuf[VD];
        auto vread = [&](int n) -> u32x4 {
            const int o = 128 * ((n >> 2) ^ vq) + vo[n & 3];
            const u32x2 lo = ds_read_tr(vb + o);
            const u32x2 hi = ds_read_tr(vb + o + 16 * LROW);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
#pragma unroll
        for (int n = 0; n < VD; ++n) vbuf[n] = vread(n);
#pragma unroll
        for (int n = 0; n < 32; ++n) {
            __builtin_amdgcn_sched_barrier(0);
            const u32x4 v = vbuf[n % VD];
            if (n + VD < 32) vbuf[n % VD] = vread(n + VD);
#pragma unroll
            for (int hq = 0; hq < 2; ++hq)
                O[hq][n] = mfma_bf16(as_bf16x8(pa[hq]), as_bf16x8(v), O[hq][n]);
            between(n);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // Softmax of one half for heads 16 hq + c16; the bf16 probabilities come out in the A
    // layout of P V (head c16, keys {4g..4g+3} of each 16-key group).  Raw logits, masked to
    // -inf where hbits (the half's 32 key-validity bits) says so; the scale is applied inside
    // the exponent's fma, and to a maximum once: scale2 > 0 and rounding is monotonic, so
    // max(x) * scale2 is exactly the maximum of the rounded x * scale2.
    // FIX: some head still lacks its reference -- the half's per-head maxima across the lanes
    // fix it (the first valid logits; O and l are still zero then).
    auto softmax_half = [&](const v4f (&S)[2][2], uint32_t hbits, bool fix, u32x4 (&pa)[2]) {
#pragma unroll
        for (int hq = 0; hq < 2; ++hq) {
            float x[2][4];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    x[kt][r] = ((hbits >> (kt * 16 + 4 * g + r)) & 1u) ? S[kt][hq][r]
                                                                     : -__builtin_huge_valf();
            const float mx = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                                   fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
            m_lane[hq] = fmaxf(m_lane[hq], mx);
            if (fix) {
                const float mh = max_xor32(max_xor16(mx)) * scale2;   // all lanes take part
                if (m_ref[hq] == -__builtin_huge_valf()) m_ref[hq] = mh;
            }
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
            pa[hq] = __builtin_bit_cast(u32x4, __builtin_convertvector(
                (v8f){p[0][0], p[0][1], p[0][2], p[0][3], p[1][0], p[1][1], p[1][2], p[1][3]}, v8bf));
        }
    };
    // Element e of a half's softmax when every key is valid and the references are fixed
    // (head group e / 8, key group e / 4 % 2, element e % 4): per head the same operations in
    // the same order as softmax_half, so the results are bitwise those of the unsplit form.
    auto softmax_elem = [&](const v4f (&S)[2][2], int e, float (&pb)[2], float (&psum)[2],
                            u32x4 (&pa)[2]) {
        const int hq = e >> 3, kt = (e >> 2) & 1, r = e & 3;
        const float x = S[kt][hq][r];
        m_lane[hq] = fmaxf(m_lane[hq], x);
        const float p = __builtin_amdgcn_exp2f(fmaf(x, scale2, -m_ref[hq]));
        psum[hq] = (e & 7) == 0 ? p : psum[hq] + p;
        if (r & 1)
            pa[hq][(kt * 4 + r) >> 1] =
                __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){pb[hq], p}, v2bf));
        else
            pb[hq] = p;
        if ((e & 7) == 7) l_run[hq] += psum[hq];
    };

#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int hq = 0; hq < 2; ++hq) {
#pragma unroll
            for (int n = 0; n < 32; ++n) O[hq][n] = v4f{0.f, 0.f, 0.f, 0.f};
            l_run[hq] = 0.f;
            m_lane[hq] = -__builtin_huge_valf();
        }
        // a recomputation pass starts with every reference set (-inf only for a head that saw
        // no valid key)
        bool have_ref = __all(m_ref[0] != -__builtin_huge_valf() && m_ref[1] != -__builtin_huge_valf());
        int idx_cur = 0, idx_nxt = 0;
        if (ntile > 0) {
            idx_cur = check_idx(0, load_idx(0));
            idx_nxt = load_idx(1);
            issue(0, idx_cur);
        }
        // One tile: tb holds it, the other buffer receives the next one.  KIND 2: every key
        // valid and the references fixed -- the softmax of the first half runs between the QK
        // MFMAs of the second, that of the second between the P V MFMAs of the first.  KIND 1:
        // references fixed, keys may be masked; KIND 0: some head still lacks its reference.
        auto step = [&](int t, const uint8_t* tb, auto kind_tag) {
            constexpr int KIND = decltype(kind_tag)::value;
            __builtin_amdgcn_s_waitcnt(0);             // this wave's part of tile t landed
            __syncthreads();                           // everyone's part; tile t-1 consumed
            const uint64_t vmask = __ballot(idx_cur >= 0);
            idx_nxt = check_idx(t + 1, idx_nxt);
            if (t + 1 < ntile) issue((t + 1) & 1, idx_nxt);
            idx_cur = idx_nxt;
            idx_nxt = load_idx(t + 2);
            if constexpr (KIND == 2) {
                v4f S0[2][2], S1[2][2];
                u32x4 pa0[2], pa1[2];
                float pb[2], psum[2];
                qk_half(tb, 0, S0, [](int) {});
                qk_half(tb, 1, S1, [&](int s) {
                    if (s < 16) softmax_elem(S0, s, pb, psum, pa0);
                });
                pv_half(tb, 0, pa0, [&](int n) {
                    if ((n & 1) == 0) softmax_elem(S1, n >> 1, pb, psum, pa1);
                });
                pv_half(tb, 1, pa1, [](int) {});
            } else {
#pragma unroll 1
                for (int half = 0; half < 2; ++half) {
                    v4f S[2][2];
                    u32x4 pa[2];
                    qk_half(tb, half, S, [](int) {});
                    softmax_half(S, (uint32_t)(vmask >> (half * 32)), KIND == 0, pa);
                    if (KIND == 0)
                        have_ref = __all(m_ref[0] != -__builtin_huge_valf() &&
                                         m_ref[1] != -__builtin_huge_valf());
                    pv_half(tb, half, pa, [](int) {});
                }
            }
        };
        int t = 0;
#pragma unroll 1
        for (; t < ntile && !have_ref; ++t) step(t, s_tile[t & 1], std::integral_constant<int, 0>{});
#pragma unroll 1
        for (; t < ntile && __ballot(idx_cur >= 0) == ~0ull; ++t)
            step(t, s_tile[t & 1], std::integral_constant<int, 2>{});
#pragma unroll 1
        for (; t < ntile; ++t) step(t, s_tile[t & 1], std::integral_constant<int, 1>{});

        // the heads' maxima over the pass and the overflow test (the halves before a head's
        // reference was fixed held no valid logit, or fixed it, so none of them exceeds it)
        bool over = false;
        float m_max[2];
#pragma unroll
        for (int hq = 0; hq < 2; ++hq) {
            m_max[hq] = max_xor32(max_xor16(m_lane[hq])) * scale2;
            over |= m_max[hq] > m_ref[hq] + OVF_SLACK;
        }
        // every wave must agree on a recomputation (the tile barriers pair up): flags through LDS
        const bool wave_over = __any(over);
        if (lane == 0) s_flag[wave] = wave_over ? 1 : 0;
        __syncthreads();
        bool redo = false;
#pragma unroll
        for (int w = 0; w < NW; ++w) redo |= s_flag[w] != 0;
        __syncthreads();                               // flags read before the next pass
        if (!redo) break;
#pragma unroll
        for (int hq = 0; hq < 2; ++hq) m_ref[hq] = m_max[hq];
    }
    // lane coordinates taken afresh, so that no address of the stores below is formed before
    // the loop and held across it
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    const int ge = lane_e >> 4, ce = lane_e & 15;

    // totals per head (lanes c16 of head group hq), then 1/total for the heads of O's rows
    // (head 16 hq + 4g + r sits in lane 4g + r's column)
    float my_lse[2], inv[2];
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
        float l_tot = l_run[hq] + shfl_xor_f(l_run[hq], 16);
        l_tot += shfl_xor_f(l_tot, 32);
        my_lse[hq] = l_tot > 0.f ? m_ref[hq] * LN2 + logf(l_tot) : -__builtin_huge_valf();
        inv[hq] = l_tot > 0.f ? 1.f / l_tot : 0.f;
    }

    if (splits == 1) {
#pragma unroll
        for (int hq = 0; hq < 2; ++hq)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int hh = wave * 32 + hq * 16 + 4 * ge + r;
                const float ir = __shfl(inv[hq], 4 * ge + r, 64);
                if (hh >= H) continue;
                uint16_t* orow = out + ((int64_t)row * H + hh) * 512;
#pragma unroll
                for (int n = 0; n < 32; ++n)
                    orow[16 * n + ce] = (uint16_t)bf16_bits(O[hq][n][r] * ir);
            }
        if (lse && ge == 0)
#pragma unroll
            for (int hq = 0; hq < 2; ++hq) {
                const int hh = wave * 32 + hq * 16 + ce;
                if (hh < H) lse[(int64_t)row * H + hh] = my_lse[hq];
            }
    } else {
        const int64_t pb = ((int64_t)row * splits + split) * H;
#pragma unroll
        for (int hq = 0; hq < 2; ++hq)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int hh = wave * 32 + hq * 16 + 4 * ge + r;
                const float ir = __shfl(inv[hq], 4 * ge + r, 64);
                if (hh >= H) continue;
                float* orow = part_o + (pb + hh) * 512;
#pragma unroll
                for (int n = 0; n < 32; ++n) orow[16 * n + ce] = O[hq][n][r] * ir;
            }
        if (ge == 0)
#pragma unroll
            for (int hq = 0; hq < 2; ++hq) {
                const int hh = wave * 32 + hq * 16 + ce;
                if (hh < H) part_lse[pb + hh] = my_lse[hq];
            }
    }
}

// Merge split partials: out = sum_s w_s o_s / sum_s w_s, w_s = exp(lse_s - M), M = max_s lse_s,
// lse = M + log sum_s w_s.  One workgroup per (row, 16-head group): its 16 heads' weights go
// to LDS first, then thread i of 256 takes the 16-byte words i, i + 256, .. of the group's
// 16 x 512 fp32 block (head 16 grp + w / 128, dims 4 (w % 128) .. +3) of every split, all of a
// split's loads in flight at once, and writes 8 bytes of bf16 output per word.
constexpr int CB_THREADS = 256;
constexpr int CB_WORDS = 16 * 128 / CB_THREADS;      // 16-byte words per thread and split
constexpr int CB_SMAX = 8;                           // splits at most

__global__ __launch_bounds__(CB_THREADS) void mla_combine_kernel(const float* __restrict__ part_o,
                                                                 const float* __restrict__ part_lse,
                                                                 int H, int splits,
                                                                 uint16_t* __restrict__ out,
                                                                 float* __restrict__ lse)
{
    __shared__ float s_w[CB_SMAX][16];               // weight of split s for head 16 grp + h
    __shared__ float s_inv[16];                      // 1 / sum of the weights
    const int ng = (H + 15) >> 4;
    const int row = blockIdx.x / ng, grp = blockIdx.x % ng;
    const int tid = threadIdx.x;
    if (tid < 16) {
        const int hh = grp * 16 + tid;
        float l[CB_SMAX], M = -__builtin_huge_valf();
#pragma unroll
        for (int sp = 0; sp < CB_SMAX; ++sp) {
            l[sp] = sp < splits && hh < H ? part_lse[((int64_t)row * splits + sp) * H + hh]
                                          : -__builtin_huge_valf();
            M = fmaxf(M, l[sp]);
        }
        const float Mf = M == -__builtin_huge_valf() ? 0.f : M;   // no split has a valid entry
        float den = 0.f;
#pragma unroll
        for (int sp = 0; sp < CB_SMAX; ++sp) {
            const float wgt = expf(l[sp] - Mf);      // 0 for an empty split
            s_w[sp][tid] = wgt;
            den += wgt;
        }
        s_inv[tid] = den > 0.f ? 1.f / den : 0.f;
        if (lse && hh < H) lse[(int64_t)row * H + hh] = den > 0.f ? Mf + logf(den) : -__builtin_huge_valf();
    }
    __syncthreads();
    const int hl0 = tid >> 7;                        // word j: head hl0 + 2j, dims 4 (tid % 128)
    const v4f* src = reinterpret_cast<const v4f*>(part_o) +
                     ((int64_t)row * splits * H + grp * 16) * 128 + (tid & 127);
    v4f acc[CB_WORDS];
#pragma unroll
    for (int j = 0; j < CB_WORDS; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < splits; ++sp) {
        v4f o[CB_WORDS];
#pragma unroll
        for (int j = 0; j < CB_WORDS; ++j) {
            const int hl = hl0 + 2 * j;
            o[j] = grp * 16 + hl < H ? src[((int64_t)sp * H + hl) * 128] : v4f{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < CB_WORDS; ++j) {
            const float wgt = s_w[sp][hl0 + 2 * j];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[j][e] = fmaf(wgt, o[j][e], acc[j][e]);
        }
    }
#pragma unroll
    for (int j = 0; j < CB_WORDS; ++j) {
        const int hl = hl0 + 2 * j, hh = grp * 16 + hl;
        if (hh >= H) continue;
        const float inv = s_inv[hl];
        u32x2 packed;
        packed[0] = pack_bf16x2(acc[j][0] * inv, acc[j][1] * inv);
        packed[1] = pack_bf16x2(acc[j][2] * inv, acc[j][3] * inv);
        *reinterpret_cast<u32x2*>(out + ((int64_t)row * H + hh) * 512 + 4 * (tid & 127)) = packed;
    }
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
    // gathered rows are addressed by byte offsets below 2^31 within a sequence's cache
    if ((int64_t)L * 1152 > 0x7FFFFFFFll) return hipErrorInvalidValue;
    // four waves of 32 head slots; fewer heads leave slots empty (their queries read as zero
    // and their outputs are not written): one shape, which fits its 512 registers without
    // spilling to scratch (checked by the CPU tests on the compiler's resource report)
    if (H <= 128)
        return launch_nw<4>(q, kv, idx, seq_start, T, L, H, k, sm_scale, splits, out, lse, part_o,
                            part_lse, valid_pos0, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_mla_combine(const float* part_o, const float* part_lse, int T, int H,
                              int splits, uint16_t* out, float* lse, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    if (splits > CB_SMAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mla_combine_kernel, dim3(T * ((H + 15) / 16)), dim3(CB_THREADS), 0, stream,
                       part_o, part_lse, H, splits, out, lse);
    return hipGetLastError();
}

}  // namespace dsa
