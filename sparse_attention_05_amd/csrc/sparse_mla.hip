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
// holds nine groups of eight 16-byte chunks (eight groups of 64 latent dims, one of the 64
// rope dims), each group [64 rows][128 B] with its chunks swizzled by row: one gather
// instruction fills 1 KB of a group for eight rows from a per-lane row offset and the
// group's immediate, and a full tile spreads the next tile's gather over its first QK steps.
// Wave w owns 32 heads from end to end:
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
constexpr int GROW = 128;                    // bytes of a row in one chunk group
constexpr int GRP = MT * GROW;               // bytes of one chunk group: 8,192
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
// Headroom of the fixed softmax reference (log2 units): p = 2^(x - m_ref) <= 2^64, so the
// row sum stays below 2^77 for k <= 8192 and fp32 keeps its relative precision throughout.
constexpr float OVF_SLACK = 64.f;

// Tile layout: nine groups of eight 16-byte chunks (group G < 8: latent dims
// [64G, 64G + 64); group 8: the 64 rope dims), each group [64 rows][128 B].  Chunk c of row
// r sits at byte GRP (c / 8) + GROW r + 16 ((c % 8) ^ swz(r)), swz(r) = 2 ((r / 2) % 4).
// One gather instruction fills 1 KB of one group: rows 8j .. 8j + 7, lane l writing row
// 8j + l/8, slot l % 8.  With swz the reads below are free of LDS bank conflicts (gfx950
// serves a 16-byte read in the lane groups {0-7, 24-31}, {8-15, 16-23} and likewise in the
// upper half, an 8-byte read in lanes 0-31 and 32-63): the K operand reads (16 rows at one
// chunk, the four lane groups at chunks 4m .. 4m + 3) and the transposing V reads (8-byte
// pieces of 8 rows, a 32-byte chunk pair per row).
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 3) << 1; }

// s_waitcnt on the LDS counter alone: at most n LDS operations outstanding (n a constant
// once the caller's loop is unrolled: 0, 2, 4 or 6; anything else waits for all).  LDS
// operations complete in order on that counter; no scalar memory load (which shares it and
// may return out of order) is in flight in the tile loop: the kernel's arguments are loaded
// and awaited before it.  Further LDS operations issued after the awaited ones only make
// such a wait stricter.
#define DSA_WAIT_LDS(n) __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | ((n) << 8))
__device__ __forceinline__ void wait_lds(int n)
{
    switch (n) {
    case 6: DSA_WAIT_LDS(6); break;
    case 4: DSA_WAIT_LDS(4); break;
    case 2: DSA_WAIT_LDS(2); break;
    default: DSA_WAIT_LDS(0); break;
    }
}
#undef DSA_WAIT_LDS

// The nine gather instructions of rows 8j .. 8j + 7: lane l loads 16 bytes from sbase + voff
// + 128 G (group G's chunks) into LDS byte lds_rows + GRP G + 16 l.  The instruction's
// offset applies to the LDS address (M0 + offset + 16 l) as well as to the global one, so
// M0 takes lds_rows + (GRP - 128) G; one wait state after each write of M0.
#define DSA_GRP_LOAD(G) "s_add_u32 m0, %2, " #G " * 8064\n\ts_nop 0\n\t" \
                        "global_load_lds_dwordx4 %0, %1 offset:" #G " * 128\n\t"
__device__ __forceinline__ void dma_rows(uint32_t voff, const void* sbase, uint32_t lds_rows)
{
    static_assert(GRP - 128 == 8064, "group stride in the gather's immediates");
    asm volatile(DSA_GRP_LOAD(0) DSA_GRP_LOAD(1) DSA_GRP_LOAD(2) DSA_GRP_LOAD(3) DSA_GRP_LOAD(4)
                 DSA_GRP_LOAD(5) DSA_GRP_LOAD(6) DSA_GRP_LOAD(7) DSA_GRP_LOAD(8)
                 :
                 : "v"(voff), "s"(sbase), "s"(lds_rows)
                 : "memory", "m0", "scc");
}
#undef DSA_GRP_LOAD
// One of those instructions (group G), for issuing them one at a time between other work.
template <int G>
__device__ __forceinline__ void dma_row_group(uint32_t voff, const void* sbase, uint32_t lds_rows)
{
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%4"
                 :
                 : "v"(voff), "s"(sbase), "s"(lds_rows), "i"(G * (GRP - 128)), "i"(128 * G)
                 : "memory", "m0", "scc");
}

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
    // row 0 and is masked later).  Wave w moves rows 8j .. 8j + 7 for j = 2w, 2w + 1 in all
    // nine groups: lane l loads row 8j + l/8's chunk 8G + ((l % 8) ^ swz(l / 8)) (swz(8j + x)
    // = swz(x)).  A row is a 32-bit byte offset from the row's cache (its index times 1152;
    // the launch keeps every cache below 2 GiB, so the offset stays below 2^31), fetched from
    // the lane holding it; the group's chunk offset is the instruction's immediate.
    const uint32_t lds_tiles = __builtin_amdgcn_readfirstlane(lds_addr(s_tile[0]));
    // gather operands of the wave's two row blocks: the lane's source offset v[jj] and the
    // LDS address of the block's rows in group 0, rows[jj]
    struct GatherOps {
        uint32_t v[2];
        uint32_t rows[2];
    };
    auto gather_ops = [&](int buf, int tidx) -> GatherOps {
        // the lane's offsets are formed here rather than held across the tile loop
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const uint32_t dst = lds_tiles + (uint32_t)buf * TILE_BYTES;
        const uint32_t roff = (uint32_t)max(tidx, 0) * 1152u;   // lane r: row r's byte offset
        const uint32_t part = 16u * (uint32_t)((ln & 7) ^ swz(ln >> 3));
        GatherOps o;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * wave + jj;
            o.v[jj] = (uint32_t)__builtin_amdgcn_ds_bpermute((8 * j + (ln >> 3)) * 4, (int)roff) + part;
            o.rows[jj] = dst + (uint32_t)j * 1024u;
        }
        return o;
    };
    auto issue = [&](int buf, int tidx) {
        const GatherOps o = gather_ops(buf, tidx);
        dma_rows(o.v[0], kvr, o.rows[0]);
        dma_rows(o.v[1], kvr, o.rows[1]);
    };
    // the i-th of the wave's 18 gather instructions (row block i / 9, group i % 9)
    auto issue_one = [&](const GatherOps& o, int i) {
        const int jj = i / 9;
        switch (i % 9) {
        case 0: dma_row_group<0>(o.v[jj], kvr, o.rows[jj]); break;
        case 1: dma_row_group<1>(o.v[jj], kvr, o.rows[jj]); break;
        case 2: dma_row_group<2>(o.v[jj], kvr, o.rows[jj]); break;
        case 3: dma_row_group<3>(o.v[jj], kvr, o.rows[jj]); break;
        case 4: dma_row_group<4>(o.v[jj], kvr, o.rows[jj]); break;
        case 5: dma_row_group<5>(o.v[jj], kvr, o.rows[jj]); break;
        case 6: dma_row_group<6>(o.v[jj], kvr, o.rows[jj]); break;
        case 7: dma_row_group<7>(o.v[jj], kvr, o.rows[jj]); break;
        default: dma_row_group<8>(o.v[jj], kvr, o.rows[jj]); break;
        }
    };

    // per-lane offsets of the operand reads (see the tile layout above).  S^T A operand for
    // step m (chunk 4m + g of rows 32 half + 16 kt + c16: group m / 2, slot 4 (m % 2) + g)
    int qo[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) qo[p] = 16 * ((4 * p + g) ^ swz(c16));
    // V operand of P V for dim block n, keys 32 half + 16 kt + 4g + r: transposing reads, lane
    // (g, i) addressing row 32 half + 16 kt + 4g + i/4, dims 16n + 4(i%4) .. +3, i.e. chunk
    // 2n + (i%4)/2 (group n / 4, slot (2 (n % 4) + (i%4)/2) ^ swz(row)), byte 8 (i%2) in it
    const int rv = 4 * g + (c16 >> 2);
    const int vbase = GROW * rv + (c16 & 1) * 8;
    int vo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vo[j] = 16 * ((2 * j + ((c16 & 3) >> 1)) ^ swz(rv));

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
        const uint8_t* rb = tb + GROW * (half * 32 + c16);     // kt adds 16 rows
        constexpr int QD = 4;
        u32x4 abuf[QD][2];
#pragma unroll
        for (int s = 0; s < QD; ++s)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                abuf[s][kt] = *reinterpret_cast<const u32x4*>(rb + kt * 16 * GROW + GRP * (s >> 1) + qo[s & 1]);
#pragma unroll
        for (int s = 0; s < 18; ++s) {
            __builtin_amdgcn_sched_barrier(0);
            // one wait per two steps: both steps' operands (the reads of later steps may stay
            // in flight)
            if ((s & 1) == 0) wait_lds(2 * max(0, min(17, s - 1 + QD) - (s + 1)));
            const u32x4 a[2] = {abuf[s % QD][0], abuf[s % QD][1]};
            if (s + QD < 18) {
                const int m = s + QD;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    abuf[s % QD][kt] = *reinterpret_cast<const u32x4*>(
                        rb + kt * 16 * GROW + GRP * (m >> 1) + qo[m & 1]);
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
        const uint8_t* vb = tb + half * 32 * GROW + vbase;
        constexpr int VD = 4;
        u32x4 vbuf[VD];
        auto vread = [&](int n) -> u32x4 {
            const int o = GRP * (n >> 2) + vo[n & 3];
            const u32x2 lo = ds_read_tr(vb + o);
            const u32x2 hi = ds_read_tr(vb + o + 16 * GROW);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
#pragma unroll
        for (int n = 0; n < VD; ++n) vbuf[n] = vread(n);
#pragma unroll
        for (int n = 0; n < 32; ++n) {
            __builtin_amdgcn_sched_barrier(0);
            if ((n & 1) == 0) wait_lds(2 * max(0, min(31, n - 1 + VD) - (n + 1)));
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
    // (head group e / 8, key group e / 4 % 2, element e % 4), in three stages that the full
    // tile places in successive MFMA steps, so that no vector instruction of a step waits for
    // another of the same step: A, the exponent's argument (and the lane's running maximum);
    // B, the exponential; C, the head's running sum and the bf16 pair.  Per head the same
    // operations in the same order as softmax_half, so the results are bitwise those of the
    // unsplit form.
    auto sm_a = [&](const v4f (&S)[2][2], int e, float (&tv)[16]) {
        const int hq = e >> 3, kt = (e >> 2) & 1, r = e & 3;
        const float x = S[kt][hq][r];
        m_lane[hq] = fmaxf(m_lane[hq], x);
        tv[e] = fmaf(x, scale2, -m_ref[hq]);
    };
    auto sm_b = [&](int e, const float (&tv)[16], float (&pv)[16]) {
        pv[e] = __builtin_amdgcn_exp2f(tv[e]);
    };
    auto sm_c = [&](int e, const float (&pv)[16], float (&psum)[2], u32x4 (&pa)[2]) {
        const int hq = e >> 3, kt = (e >> 2) & 1, r = e & 3;
        psum[hq] = (e & 7) == 0 ? pv[e] : psum[hq] + pv[e];
        if (r & 1)
            pa[hq][(kt * 4 + r) >> 1] =
                __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){pv[e - 1], pv[e]}, v2bf));
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
            GatherOps go;
            if constexpr (KIND == 2)                   // a next tile exists: issued below
                go = gather_ops((t + 1) & 1, idx_nxt);
            else if (t + 1 < ntile)
                issue((t + 1) & 1, idx_nxt);
            idx_cur = idx_nxt;
            idx_nxt = load_idx(t + 2);
            if constexpr (KIND == 2) {
                v4f S0[2][2], S1[2][2];
                u32x4 pa0[2], pa1[2];
                float psum[2];
                float tv0[16], pv0[16], tv1[16], pv1[16];
                // the next tile's gather, one instruction per QK step (bunched, the wave's
                // 18 instructions wait for the address unit, which the other waves' fill too)
                qk_half(tb, 0, S0, [&](int s) { issue_one(go, s); });
                // the first half's softmax, stage A of element s, B of s - 1, C of s - 2
                qk_half(tb, 1, S1, [&](int s) {
                    if (s < 16) sm_a(S0, s, tv0);
                    if (s >= 1 && s <= 16) sm_b(s - 1, tv0, pv0);
                    if (s >= 2) sm_c(s - 2, pv0, psum, pa0);
                });
                // the second's, stage A of element n / 2 at even steps, B at odd ones, C a
                // step later
                pv_half(tb, 0, pa0, [&](int n) {
                    if ((n & 1) == 0) {
                        sm_a(S1, n >> 1, tv1);
                        if (n >= 2) sm_c((n >> 1) - 1, pv1, psum, pa1);
                    } else {
                        sm_b(n >> 1, tv1, pv1);
                    }
                });
                sm_c(15, pv1, psum, pa1);
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
        for (; t + 1 < ntile && __ballot(idx_cur >= 0) == ~0ull; ++t)
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
