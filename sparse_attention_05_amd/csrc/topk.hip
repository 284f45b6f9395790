// topk.hip -- per-row top-k selection on gfx950.
//
// Row t keeps the k largest of its n_t visible scores; a row with n_t <= k keeps all of
// 0..n_t-1 (《DeepSeek-V3.2-Exp模型优势与 DSA 工作原理》 §4 步骤三 and §2 风险边界明确).  Ties
// go to the lower position and -0 equals +0, which makes the selected set unique.
//
// Scores map to order-preserving uint32 keys; one 512-thread workgroup per row.
//   short rows (n <= CAND_CAP = 5888): the whole row is staged in LDS once;
//   long rows: 64 contiguous blocks spread over the row (4096 keys, a few KB of reads) give
//     an estimate tau_lo of the key with about 2k keys above it; one ordered pass over the
//     row keeps every key >= tau_lo as an LDS candidate (key, position) in position order.
//   In both cases an exact three-level radix select over the LDS candidates finds the k-th
//   key tau, and an ordered sweep emits the keys above tau and the lowest-position ties, so
//   the output is ascending.  Each long row is read from memory once (plus the sample).
// If the estimate leaves fewer than k or more than CAND_CAP candidates, the row falls back
// to the exact path: a 4096-bin histogram pass, an ordered pass keeping the positions above
// the boundary bin and the boundary bin's candidates, an LDS radix resolve and a co-rank
// merge (two reads of the row; a global multi-level pass if even that bin overflows).
//
// The fused prefill selection replaces the score row by candidates: a threshold per row
// from the scores of its every 32nd key (topk_threshold_kernel, a lower bound of the key
// with about 1.75k keys above it), the indexer keeping the keys at or above it, and
// topk_resolve_kernel deciding the row from those alone.  Any candidate set holding at least
// k keys contains every key at or above the row's k-th largest, ties included, so the exact
// select over it gives the same top-k as the full row; rows short of k candidates, or with
// more than fit, are flagged and go through the full scores and topk_kernel instead.
#include <algorithm>

#include "dsa_device.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int TK_THREADS = 512;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int CAND_CAP = 5888;              // candidates kept in LDS (two workgroups per CU)
constexpr int SAMPLE = 4096;                // sampled keys (64 blocks of 64)
constexpr int FB_BINS = 4096;               // fallback first digit: key bits 31..20
constexpr int FB_CAP = 3072;                // fallback boundary-bin candidates
constexpr int TK_KMAX = 8192;

// LDS carve-up (bytes): the paths never coexist, so they share one buffer.
constexpr int OFF_HIST = 0;                                    // up to 4096 ints
constexpr int OFF_A = OFF_HIST + 4 * FB_BINS;                  // 16 KB
constexpr int LDS_BYTES = OFF_A + 8 * CAND_CAP + 4 * SAMPLE;   // 80 KB
static_assert(4 * TK_KMAX + 8 * FB_CAP <= 8 * CAND_CAP + 4 * SAMPLE, "fallback fits");

struct RowRef {
    const float* p;
    int n;
};

template <bool DECODE>
__device__ __forceinline__ RowRef row_of(int row, const float* scores, int64_t ld,
                                         const int64_t* seq_start, int L, int q_pos0)
{
    if constexpr (DECODE) {
        const int64_t a = seq_start[row];
        return RowRef{scores + a, (int)(seq_start[row + 1] - a)};
    } else {
        return RowRef{scores + (int64_t)row * ld, min(L, q_pos0 + row + 1)};
    }
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts of 1, 2, 4 and 8 lanes within each
// 16-lane row, then the row totals carried forward by the row broadcasts of lane 15 (into rows
// 1 and 3) and lane 31 (into rows 2 and 3).  Data-parallel-primitive moves, no LDS traffic.
__device__ __forceinline__ int wave_incl_scan(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);    // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);    // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);    // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);    // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return x;
}

// Per-wave totals of the block scans, in two alternating slots: a call writes the slot the
// previous call did not use, and every thread finished reading that slot (two calls back)
// before it reached the previous call's barrier, so one barrier per scan suffices.  Every
// thread of the workgroup makes the same sequence of calls.
struct ScanBuf {
    int* w;                                   // 2 * TK_WAVES ints of LDS
    int par;
};

// Block-wide exclusive prefix sum (ascending thread order) and total.
__device__ __forceinline__ int block_excl_scan(int v, ScanBuf& sb, int* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int* w = sb.w + sb.par * TK_WAVES;
    sb.par ^= 1;
    const int x = wave_incl_scan(v);
    if (lane == 63) w[wave] = x;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < TK_WAVES; ++i) {
        const int c = w[i];
        off += (i < wave) ? c : 0;
        tot += c;
    }
    *total = tot;
    return off + x - v;
}

// Boundary bin of a descending histogram of NB bins: the bin B with count(bins > B) < need
// <= count(bins >= B) (requires need <= the histogram's total).  Returns B and stores
// need - count(bins > B) in *rem.  Thread i covers bins NB-1-i*PER downwards.  One barrier:
// after the per-wave totals are exchanged, every wave re-reads the bins of the wave that
// holds the boundary and finds the boundary lane itself.
template <int NB>
__device__ __forceinline__ int boundary_bin(const int* hist, int need, ScanBuf& sb, int* rem)
{
    constexpr int PER = NB / TK_THREADS;
    static_assert(PER * TK_THREADS == NB, "bins per thread");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int sum = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) sum += hist[NB - 1 - tid * PER - q];
    const int x = wave_incl_scan(sum);
    int* w = sb.w + sb.par * TK_WAVES;
    sb.par ^= 1;
    if (lane == 63) w[wave] = x;
    __syncthreads();
    int acc = 0, bw = 0, before = 0;            // the wave holding the boundary, counts before it
#pragma unroll
    for (int i = 0; i < TK_WAVES; ++i) {
        const int c = w[i];
        if (acc < need && need <= acc + c) {
            bw = i;
            before = acc;
        }
        acc += c;
    }
    const int t2 = bw * 64 + lane;
    int cnt[PER], s2 = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        cnt[q] = hist[NB - 1 - t2 * PER - q];
        s2 += cnt[q];
    }
    int a = before + wave_incl_scan(s2) - s2;   // counts in bins above this lane's bins
    const bool mine = a < need && need <= a + s2;
    int b_l = 0, rem_l = need;
    if (mine) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (a < need && need <= a + cnt[q]) {
                b_l = NB - 1 - t2 * PER - q;
                rem_l = need - a;
            }
            a += cnt[q];
        }
    }
    const uint64_t m = __ballot(mine);
    const int src = m ? __builtin_ctzll(m) : 0;
    *rem = __builtin_amdgcn_readlane(rem_l, src);
    return __builtin_amdgcn_readlane(b_l, src);
}

// Running maximum over the 64 lanes of a wave (lane 63 ends with the wave's maximum): the
// same shift-and-broadcast pattern as wave_incl_scan, 0 being the identity of unsigned max.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x)
{
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false));
    x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Keys per thread of the LDS-resident selections and emissions: covers CAND_CAP, SAMPLE and
// FB_CAP.  Thread t owns the contiguous entries [SEL_PT * t, SEL_PT * t + SEL_PT).
constexpr int SEL_PT = 12;
static_assert(SEL_PT * TK_THREADS >= CAND_CAP && SEL_PT * TK_THREADS >= SAMPLE &&
              SEL_PT * TK_THREADS >= FB_CAP, "selection entries per thread");

// This thread's entries [SEL_PT * tid, ...) of an LDS array of n entries; returns how many
// exist (0..SEL_PT).  Whole 16-byte loads when all SEL_PT exist.
template <typename T>
__device__ __forceinline__ int load_own(const T* a, int n, T (&r)[SEL_PT])
{
    static_assert(sizeof(T) == 4, "4-byte entries");
    const int i0 = SEL_PT * (int)threadIdx.x;
    const int cnt = max(0, min(SEL_PT, n - i0));
    if (cnt == SEL_PT) {
#pragma unroll
        for (int q = 0; q < SEL_PT / 4; ++q) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(a + i0 + 4 * q);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t e = v[j];        // a scalar first: bit_cast of a vector element
                r[4 * q + j] = __builtin_bit_cast(T, e);   // reads element 0 with this compiler
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < SEL_PT; ++j) r[j] = j < cnt ? a[i0 + j] : T(0);
    }
    return cnt;
}

// Exact kth-largest key among keys[0..nk) held in LDS (1 <= kth <= nk <= SEL_PT * 512).
// Each thread holds its keys in registers for all levels.  The keys' common high bits (where
// the smallest and largest key agree) are skipped; the bits below are resolved by radix
// levels of up to 11 bits, starting at the highest bit where keys differ, so the first
// histogram spreads the keys over the range they actually span (candidates above a
// threshold share most of their high bits).  Returns the key and stores in *need_eq how many
// keys equal to it belong to the top kth.  With exact = false it stops after two levels and
// returns the lowest key of the bin reached: a lower bound of the kth-largest key that at
// most the keys of one 22-bit-resolved bin exceed beyond it.
// hist: 4096 ints (levels alternate between its halves); s_mm: 2 * TK_WAVES ints.
// select_own takes the keys already in registers: each thread's kr[0 .. cnt), the keys of all
// threads together being the nk keys selected from.
__device__ __forceinline__ uint32_t select_own(const uint32_t (&kr)[SEL_PT], int cnt, int kth,
                                               int* hist, ScanBuf& s_wave, uint32_t* s_mm,
                                               int* need_eq, bool exact = true)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t lmax = 0, lnmin = 0;                 // max of the keys and of their complements
#pragma unroll
    for (int j = 0; j < SEL_PT; ++j) {
        if (j < cnt) {
            lmax = max(lmax, kr[j]);
            lnmin = max(lnmin, ~kr[j]);
        }
    }
    lmax = wave_max_u32(lmax);
    lnmin = wave_max_u32(lnmin);
    if (lane == 0) {
        s_mm[wave] = lmax;
        s_mm[TK_WAVES + wave] = lnmin;
    }
    for (int i = tid; i < 4096; i += TK_THREADS) hist[i] = 0;     // both halves
    __syncthreads();
    uint32_t kmax = 0, knmin = 0;
#pragma unroll
    for (int i = 0; i < TK_WAVES; ++i) {
        kmax = max(kmax, s_mm[i]);
        knmin = max(knmin, s_mm[TK_WAVES + i]);
    }
    const uint32_t diff = kmax ^ ~knmin;
    if (diff == 0) {                              // every key equal
        *need_eq = kth;
        return kmax;
    }
    int hi = 31 - __clz((int)diff);               // highest bit where the keys differ
    uint32_t prefix = (uint32_t)((uint64_t)kmax >> (hi + 1));
    int need = kth;
#pragma unroll 1
    for (int lvl = 0; hi >= 0; ++lvl) {
        if (!exact && lvl == 2) {
            *need_eq = 0;
            return prefix << (hi + 1);            // hi + 1 <= 10 here
        }
        const int width = min(11, hi + 1);
        const int sh = hi + 1 - width;
        int* h = hist + 2048 * (lvl & 1);
        if (lvl >= 2) {                           // this half was used two levels ago
            for (int i = tid; i < 2048; i += TK_THREADS) h[i] = 0;
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < SEL_PT; ++j) {
            // below the first level hi + 1 <= 21, so the shift is in range
            if (j < cnt && (lvl == 0 || (kr[j] >> (hi + 1)) == prefix))
                atomicAdd(&h[(kr[j] >> sh) & ((1u << width) - 1)], 1);
        }
        __syncthreads();
        int rem;
        const int d = boundary_bin<2048>(h, need, s_wave, &rem);
        prefix = (prefix << width) | (uint32_t)d;
        need = rem;
        hi = sh - 1;
    }
    *need_eq = need;
    return prefix;
}

__device__ __forceinline__ uint32_t lds_select(const uint32_t* keys, int nk, int kth, int* hist,
                                               ScanBuf& s_wave, uint32_t* s_mm, int* need_eq,
                                               bool exact = true)
{
    uint32_t kr[SEL_PT];
    const int cnt = load_own(keys, nk, kr);
    return select_own(kr, cnt, kth, hist, s_wave, s_mm, need_eq, exact);
}

// Visit the row in position order.  The 16-byte-aligned body goes in super-rounds of
// RPT * 4 * TK_THREADS positions: thread t owns the RPT * 4 consecutive positions starting at
// RPT * 4 * t of the round and issues all RPT 16-byte loads before using any, so a
// workgroup keeps RPT * 16 KB in flight.  Thread order is position order within a round.
// f(pos0, key[], cnt) is called by every thread in every round with the keys of positions
// pos0 .. pos0 + cnt - 1 (cnt may be 0); rounds are uniform across the workgroup.  The
// unaligned head and the tail (fewer than 4 positions each) come as one-key rounds.
constexpr int RPT = 4;
constexpr int KPT = 4 * RPT;                            // keys per thread per round

// pre() runs once, after the first round's loads are issued and before f is first called
// (work that f depends on but the loads do not, such as finding a threshold).
struct NoPre {
    __device__ void operator()() const {}
};

template <typename F, typename P = NoPre>
__device__ __forceinline__ void for_row_rounds(const RowRef& rr, F&& f, P&& pre = P{})
{
    const int tid = threadIdx.x;
    const int n = rr.n;
    const int mis = (int)((reinterpret_cast<uintptr_t>(rr.p) >> 2) & 3);
    const int head = min(n, (4 - mis) & 3);            // scalars until 16-byte aligned
    const int body = (n - head) & ~3;
    const v4f* p4 = reinterpret_cast<const v4f*>(rr.p + head);
    // The loads of round r + 1 are issued before f runs on round r, so the workgroup's
    // scans and LDS work overlap the memory latency of the next round.
    v4f v[RPT];
    auto fetch = [&](int base) {
        const int e = base + KPT * tid;
        const int c = max(0, min(KPT, body - e));
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            if (4 * i < c) v[i] = p4[(e >> 2) + i];
    };
    if (body > 0) fetch(0);
    pre();
    uint32_t key[KPT] = {};
    if (head > 0) {                                     // uniform
        const int c = tid < head ? 1 : 0;
        key[0] = c ? score_key(rr.p[tid]) : 0u;
        f(tid, key, c);
    }
    for (int base = 0; base < body; base += KPT * TK_THREADS) {
        const int e = base + KPT * tid;                 // first position (in the body)
        const int c = max(0, min(KPT, body - e));       // a multiple of 4
#pragma unroll
        for (int i = 0; i < RPT; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) key[4 * i + j] = 4 * i < c ? score_key(v[i][j]) : 0u;
        if (base + KPT * TK_THREADS < body) fetch(base + KPT * TK_THREADS);
        f(head + e, key, c);
    }
    const int tail = n - head - body;                   // 0..3
    if (tail > 0) {
        const int c = tid < tail ? 1 : 0;
        key[0] = c ? score_key(rr.p[head + body + tid]) : 0u;
        f(head + body + tid, key, c);
    }
}

// Ordered emission from a position-ordered candidate list (cpos null: position = index;
// nc <= SEL_PT * 512): every key > tau, plus the first need_eq keys equal to tau, at
// slot = #(> tau before) + min(#ties before, need_eq).  One block scan: each thread takes
// SEL_PT consecutive candidates.
__device__ __forceinline__ void emit_sorted(const uint32_t* ckey, const int* cpos, int nc,
                                            uint32_t tau, int need_eq, int k, int32_t* out,
                                            ScanBuf& s_wave)
{
    uint32_t ku[SEL_PT];
    int pp[SEL_PT];
    const int cnt = load_own(ckey, nc, ku);
    if (cpos) {
        load_own(cpos, nc, pp);
    } else {
#pragma unroll
        for (int j = 0; j < SEL_PT; ++j) pp[j] = SEL_PT * (int)threadIdx.x + j;
    }
    int ng = 0, ne = 0;
#pragma unroll
    for (int j = 0; j < SEL_PT; ++j) {
        ng += (j < cnt) && ku[j] > tau;
        ne += (j < cnt) && ku[j] == tau;
    }
    int tot;
    const int off = block_excl_scan(ng | (ne << 16), s_wave, &tot);
    int gt_before = off & 0xFFFF;
    int eq_before = off >> 16;
#pragma unroll
    for (int j = 0; j < SEL_PT; ++j) {
        if (j < cnt) {
            if (ku[j] > tau) {
                const int slot = gt_before + min(eq_before, need_eq);
                if (slot < k) out[slot] = pp[j];
                ++gt_before;
            } else if (ku[j] == tau) {
                if (eq_before < need_eq && gt_before + eq_before < k) out[gt_before + eq_before] = pp[j];
                ++eq_before;
            }
        }
    }
}

// The threshold sample of a row of n > CAND_CAP keys: 64 contiguous 64-key blocks spread
// evenly over the row, as keys, into samp[0..SAMPLE).  The caller synchronises.
__device__ __forceinline__ void load_sample(const RowRef& rr, uint32_t* samp)
{
    constexpr int SPT = SAMPLE / TK_THREADS;                      // sampled keys per thread
    const int i0 = threadIdx.x * SPT, blk = i0 >> 6, off = i0 & 63;
    const int start = (int)(((int64_t)blk * (rr.n - 64)) / 63);    // n > CAND_CAP > 4096
#pragma unroll
    for (int j = 0; j < SPT; ++j) samp[i0 + j] = score_key(rr.p[start + off + j]);
}

// Sample rank with about 2k of the row's n keys above it.
__device__ __forceinline__ int sample_rank(int n, int k)
{
    return (int)min<int64_t>(SAMPLE, ((int64_t)2 * k * SAMPLE + n - 1) / n);
}

// One ordered pass over the keys of rr (positions pos_base + 0 .. rr.n - 1): every key >=
// the threshold goes to (ckey, cpos) in position order, the first CAND_CAP of them kept.
// The threshold is the lower bound that lds_select derives from the row's sample (already
// in samp, synchronised) at rank rs; its selection runs while the first loads are in
// flight.  Returns the number of keys at or above it (possibly more than CAND_CAP).
__device__ __forceinline__ int collect_candidates(const RowRef& rr, int pos_base,
                                                  const uint32_t* samp, int rs, int* hist,
                                                  ScanBuf& s_wave, uint32_t* s_mm,
                                                  uint32_t* ckey, int* cpos)
{
    uint32_t tau_lo = 0;
    int nc = 0;
    for_row_rounds(rr, [&](int pos0, const uint32_t* key, int c) {
        int mine = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) mine += (j < c) && key[j] >= tau_lo;
        int tot;
        int o = nc + block_excl_scan(mine, s_wave, &tot);
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            if (j < c && key[j] >= tau_lo) {
                if (o < CAND_CAP) {
                    ckey[o] = key[j];
                    cpos[o] = pos_base + pos0 + j;
                }
                ++o;
            }
        }
        nc += tot;
    }, [&]() {
        int unused_eq;
        tau_lo = lds_select(samp, SAMPLE, rs, hist, s_wave, s_mm, &unused_eq, false);
    });
    return nc;
}

// Candidates of long decode rows gathered by topk_segment_kernel: segment s of row b
// (keys [s * SEG, min(n, (s + 1) * SEG))) left its count in cnt[b * nseg + s] and its first
// min(count, CAND_CAP) candidates, in position order, at key/pos + (b * nseg + s) * CAND_CAP.
// nseg = 0: not used.
constexpr int SEG = 16384;
constexpr int SEG_MAX = 64;                   // rows of up to SEG * SEG_MAX keys are split
struct SegCands {
    const uint32_t* key;
    const int32_t* pos;
    const int32_t* cnt;
    int nseg;
};

template <bool DECODE>
__global__ __launch_bounds__(TK_THREADS) void topk_kernel(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ seq_start, int L,
    int q_pos0, int k, int32_t* __restrict__ idx, SegCands seg, const int* __restrict__ only,
    int only_off)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_buf[LDS_BYTES];
    __shared__ int s_wave_mem[2 * TK_WAVES];
    ScanBuf s_wave{s_wave_mem, 0};
    __shared__ uint32_t s_mm[2 * TK_WAVES];
    int* hist = reinterpret_cast<int*>(s_buf + OFF_HIST);

    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    if (only && (row < only_off || only[row - only_off] == 0)) return;   // uniform
    const RowRef rr = row_of<DECODE>(row, scores, ld, seq_start, L, q_pos0);
    const int n = rr.n;
    int32_t* out = idx + (int64_t)row * k;

    if (DECODE && n > L) {                        // longer than the scored range (L = max_len):
        for (int j = tid; j < k; j += TK_THREADS) out[j] = -1;   // no selection at all
        return;
    }
    if (n <= k) {                                 // short row: every visible position
        for (int j = tid; j < k; j += TK_THREADS) out[j] = j < n ? j : -1;
        return;
    }

    uint32_t* ckey = reinterpret_cast<uint32_t*>(s_buf + OFF_A);
    int* cpos = reinterpret_cast<int*>(s_buf + OFF_A + 4 * CAND_CAP);
    if (n <= CAND_CAP) {
        // ---- the whole row fits: stage it (all loads in flight at once), select, emit
        constexpr int SPL = (CAND_CAP + TK_THREADS - 1) / TK_THREADS;
        float sv[SPL];
#pragma unroll
        for (int j = 0; j < SPL; ++j)
            if (tid + j * TK_THREADS < n) sv[j] = rr.p[tid + j * TK_THREADS];
#pragma unroll
        for (int j = 0; j < SPL; ++j)
            if (tid + j * TK_THREADS < n) ckey[tid + j * TK_THREADS] = score_key(sv[j]);
        __syncthreads();
        int need_eq;
        const uint32_t tau = lds_select(ckey, n, k, hist, s_wave, s_mm, &need_eq);
        emit_sorted(ckey, nullptr, n, tau, need_eq, k, out, s_wave);
        return;
    }

    const int ns = (n + SEG - 1) / SEG;
    if (DECODE && seg.nseg > 0 && ns <= seg.nseg) {
        // ---- a split row: the segments' candidates, concatenated in segment order (a row
        // longer than the split covers -- outside the caller's contract -- takes the exact
        // path below instead)
        int* offs = hist;                                   // exclusive prefix, then total
        int c = 0;
        if (tid < ns) c = seg.cnt[row * seg.nseg + tid];
        const bool over = __syncthreads_or(c > CAND_CAP);
        int tot;
        const int o = block_excl_scan(c, s_wave, &tot);
        if (tid < ns) offs[tid] = o;
        if (tid == 0) offs[ns] = tot;
        __syncthreads();
        if (!over && tot >= k && tot <= CAND_CAP) {
            constexpr int PT = (CAND_CAP + TK_THREADS - 1) / TK_THREADS;
            uint32_t kv[PT];
            int pv[PT];
#pragma unroll
            for (int j = 0; j < PT; ++j) {
                const int i = tid + j * TK_THREADS;
                if (i < tot) {
                    int sg = 0;                             // last segment starting at or before i
                    for (int q = 1; q < ns; ++q) sg += offs[q] <= i;
                    const int64_t src = (int64_t)(row * seg.nseg + sg) * CAND_CAP + (i - offs[sg]);
                    kv[j] = seg.key[src];
                    pv[j] = seg.pos[src];
                }
            }
#pragma unroll
            for (int j = 0; j < PT; ++j) {
                const int i = tid + j * TK_THREADS;
                if (i < tot) {
                    ckey[i] = kv[j];
                    cpos[i] = pv[j];
                }
            }
            __syncthreads();
            int need_eq;
            const uint32_t tau = lds_select(ckey, tot, k, hist, s_wave, s_mm, &need_eq);
            emit_sorted(ckey, cpos, tot, tau, need_eq, k, out, s_wave);
            return;
        }
        __syncthreads();                                    // offs read: hist free again
    } else {
        // ---- threshold from the row's sample, then one ordered pass for the candidates
        uint32_t* samp = reinterpret_cast<uint32_t*>(s_buf + OFF_A + 8 * CAND_CAP);
        load_sample(rr, samp);
        __syncthreads();
        const int nc = collect_candidates(rr, 0, samp, sample_rank(n, k), hist, s_wave, s_mm,
                                          ckey, cpos);
        __syncthreads();
        if (nc >= k && nc <= CAND_CAP) {
            int need_eq;
            const uint32_t tau = lds_select(ckey, nc, k, hist, s_wave, s_mm, &need_eq);
            emit_sorted(ckey, cpos, nc, tau, need_eq, k, out, s_wave);
            return;
        }
    }

    // ---- fallback: exact two-pass path
    int* s_sel = reinterpret_cast<int*>(s_buf + OFF_A);                 // S: 8192 ints
    uint32_t* fkey = reinterpret_cast<uint32_t*>(s_buf + OFF_A + 4 * TK_KMAX);
    int* fpos = reinterpret_cast<int*>(s_buf + OFF_A + 4 * TK_KMAX + 4 * FB_CAP);
    for (int i = tid; i < FB_BINS; i += TK_THREADS) hist[i] = 0;
    __syncthreads();
    for_row_rounds(rr, [&](int, const uint32_t* key, int c) {
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            if (j < c) atomicAdd(&hist[key[j] >> 20], 1);
    });
    __syncthreads();
    int need_b;                                   // keys still needed from the boundary bin
    const uint32_t b = (uint32_t)boundary_bin<FB_BINS>(hist, k, s_wave, &need_b);
    const int n_above = k - need_b;               // keys in bins above b (all selected)
    const int n_cand = hist[b];
    __syncthreads();

    if (n_cand <= FB_CAP) {
        // S (bins above b) and the boundary candidates, both position-ordered
        int base_s = 0, base_c = 0;
        for_row_rounds(rr, [&](int pos0, const uint32_t* key, int c) {
            int ns = 0, ncb = 0;
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                const uint32_t d = key[j] >> 20;
                ns += (j < c) && d > b;
                ncb += (j < c) && d == b;
            }
            int tot;
            const int off = block_excl_scan(ns | (ncb << 16), s_wave, &tot);
            int os = base_s + (off & 0xFFFF), oc = base_c + (off >> 16);
#pragma unroll
            for (int j = 0; j < KPT; ++j) {
                if (j >= c) break;
                const uint32_t d = key[j] >> 20;
                if (d > b) s_sel[os++] = pos0 + j;
                else if (d == b) {
                    fkey[oc] = key[j];
                    fpos[oc++] = pos0 + j;
                }
            }
            base_s += tot & 0xFFFF;
            base_c += tot >> 16;
        });
        __syncthreads();
        int need_eq;
        const uint32_t tau = lds_select(fkey, n_cand, need_b, hist, s_wave, s_mm, &need_eq);
        // chosen candidates -> C (in place over fkey, as positions), position order kept
        int base_g = 0, base_e = 0;
        for (int r0 = 0; r0 < n_cand; r0 += 4 * TK_THREADS) {
            uint32_t ku[4];
            int pp[4], ng = 0, ne = 0;
            for (int j = 0; j < 4; ++j) {
                const int i = r0 + 4 * tid + j;
                ku[j] = i < n_cand ? fkey[i] : 0u;
                pp[j] = i < n_cand ? fpos[i] : -1;
                ng += (i < n_cand) && ku[j] > tau;
                ne += (i < n_cand) && ku[j] == tau;
            }
            int tot;
            const int off = block_excl_scan(ng | (ne << 16), s_wave, &tot);
            int eq_before = base_e + (off >> 16);
            int slot = base_g + (off & 0xFFFF) + min(eq_before, need_eq);
            __syncthreads();                      // all reads of fkey in this round done
            for (int j = 0; j < 4; ++j) {
                const int i = r0 + 4 * tid + j;
                if (i >= n_cand) break;
                if (ku[j] > tau) {
                    reinterpret_cast<int*>(fkey)[slot++] = pp[j];
                } else if (ku[j] == tau) {
                    if (eq_before < need_eq) reinterpret_cast<int*>(fkey)[slot++] = pp[j];
                    ++eq_before;
                }
            }
            base_g += tot & 0xFFFF;
            base_e += tot >> 16;
            __syncthreads();
        }
        // C holds need_b positions, S holds n_above positions, both ascending: co-rank merge
        const int* C = reinterpret_cast<const int*>(fkey);
        for (int i = tid; i < n_above; i += TK_THREADS) {
            const int p = s_sel[i];
            int lo = 0, hi = need_b;
            while (lo < hi) {
                const int m = (lo + hi) >> 1;
                if (C[m] < p) lo = m + 1; else hi = m;
            }
            out[i + lo] = p;
        }
        for (int i = tid; i < need_b; i += TK_THREADS) {
            const int p = C[i];
            int lo = 0, hi = n_above;
            while (lo < hi) {
                const int m = (lo + hi) >> 1;
                if (s_sel[m] < p) lo = m + 1; else hi = m;
            }
            out[i + lo] = p;
        }
        return;
    }

    // boundary bin too large for LDS: two more radix levels over the row in memory
    uint32_t prefix = b;
    int need = need_b;
#pragma unroll 1
    for (int lvl = 0; lvl < 2; ++lvl) {
        const int sh = lvl == 0 ? 10 : 0;
        __syncthreads();                          // the previous boundary search read hist
        for (int i = tid; i < 1024; i += TK_THREADS) hist[i] = 0;
        __syncthreads();
        for_row_rounds(rr, [&](int, const uint32_t* key, int c) {
#pragma unroll
            for (int j = 0; j < KPT; ++j)
                if (j < c && (key[j] >> (sh + 10)) == prefix)
                    atomicAdd(&hist[(key[j] >> sh) & 1023], 1);
        });
        __syncthreads();
        int rem;
        const int d = boundary_bin<1024>(hist, need, s_wave, &rem);
        prefix = (prefix << 10) | (uint32_t)d;
        need = rem;
    }
    const uint32_t tau = prefix;
    const int need_eq = need;
    int base_gt = 0, base_eq = 0;
    for_row_rounds(rr, [&](int pos0, const uint32_t* key, int c) {
        int ng = 0, ne = 0;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            ng += (j < c) && key[j] > tau;
            ne += (j < c) && key[j] == tau;
        }
        int tot;
        const int off = block_excl_scan(ng | (ne << 16), s_wave, &tot);
        int gt_before = base_gt + (off & 0xFFFF);
        int eq_before = base_eq + (off >> 16);
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            if (j >= c) break;
            if (key[j] > tau) {
                const int slot = gt_before + min(eq_before, need_eq);
                if (slot < k) out[slot] = pos0 + j;
                ++gt_before;
            } else if (key[j] == tau) {
                if (eq_before < need_eq && gt_before + eq_before < k)
                    out[gt_before + eq_before] = pos0 + j;
                ++eq_before;
            }
        }
        base_gt += tot & 0xFFFF;
        base_eq += tot >> 16;
    });
}

// Segment sgi of decode row b (rows longer than CAND_CAP only): the row's sample threshold
// (computed alike by every segment of the row), then one ordered pass over the segment's
// keys, its candidates written out for the row kernel (see SegCands).
__global__ __launch_bounds__(TK_THREADS) void topk_segment_kernel(
    const float* __restrict__ scores, const int64_t* __restrict__ seq_start, int k, int nseg,
    uint32_t* __restrict__ key_out, int32_t* __restrict__ pos_out, int32_t* __restrict__ cnt_out)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_buf[LDS_BYTES];
    __shared__ int s_wave_mem[2 * TK_WAVES];
    ScanBuf s_wave{s_wave_mem, 0};
    __shared__ uint32_t s_mm[2 * TK_WAVES];
    int* hist = reinterpret_cast<int*>(s_buf + OFF_HIST);
    uint32_t* ckey = reinterpret_cast<uint32_t*>(s_buf + OFF_A);
    int* cpos = reinterpret_cast<int*>(s_buf + OFF_A + 4 * CAND_CAP);
    uint32_t* samp = reinterpret_cast<uint32_t*>(s_buf + OFF_A + 8 * CAND_CAP);

    const int sgi = blockIdx.x, row = blockIdx.y;
    const RowRef rr = row_of<true>(row, scores, 0, seq_start, 0, 0);
    const int n = rr.n, s0 = sgi * SEG;
    if (n <= CAND_CAP || s0 >= n) return;              // uniform over the workgroup
    load_sample(rr, samp);
    __syncthreads();
    const int nc = collect_candidates(RowRef{rr.p + s0, min(SEG, n - s0)}, s0, samp,
                                      sample_rank(n, k), hist, s_wave, s_mm, ckey, cpos);
    __syncthreads();
    const int64_t slot = (int64_t)row * nseg + sgi;
    if (threadIdx.x == 0) cnt_out[slot] = nc;
    const int keep = min(nc, CAND_CAP);
    for (int i = threadIdx.x; i < keep; i += TK_THREADS) {
        key_out[slot * CAND_CAP + i] = ckey[i];
        pos_out[slot * CAND_CAP + i] = cpos[i];
    }
}

// ---- the fused prefill selection: threshold, then resolve over the indexer's candidates

// Candidates a row aims for: about 1.75k keys above its threshold (on the 128K workload,
// sampling every 32nd key, rows then keep 0.65k .. 1.4k above the k they need, within the
// LDS capacity).
__device__ __forceinline__ int fused_target(int k) { return min(7 * k / 4, (k + CAND_CAP) / 2); }

// Row t (position q_pos0 + t, n = min(L, q_pos0 + t + 1) visible keys): its threshold from
// the scores of the sampled keys 0, S, 2S, .. (samp + t * ld); 0 (every key) when the whole
// row fits the candidate capacity.  Also clears the row's candidate count and fallback flag.
__global__ __launch_bounds__(TK_THREADS) void topk_threshold_kernel(
    const float* __restrict__ samp, int64_t ld, int S, int L, int q_pos0, int k,
    uint32_t* __restrict__ tau, int* __restrict__ fill, int* __restrict__ fb)
{
    __shared__ int s_hist[4096];
    __shared__ int s_wave_mem[2 * TK_WAVES];
    ScanBuf s_wave{s_wave_mem, 0};
    __shared__ uint32_t s_mm[2 * TK_WAVES];
    const int row = blockIdx.x, tid = threadIdx.x;
    const int n = min(L, q_pos0 + row + 1);
    if (tid == 0) {
        fill[row] = 0;
        fb[row] = 0;
    }
    if (n <= CAND_CAP) {
        if (tid == 0) tau[row] = 0u;
        return;
    }
    const int ns = (n - 1) / S + 1;                     // sampled keys this row sees (<= SAMPLE)
    // this thread's sampled keys [SEL_PT tid, SEL_PT tid + SEL_PT), straight into registers
    const float* sr = samp + (int64_t)row * ld + SEL_PT * tid;
    const int cnt = max(0, min(SEL_PT, ns - SEL_PT * tid));
    uint32_t kr[SEL_PT];
#pragma unroll
    for (int j = 0; j < SEL_PT; ++j) kr[j] = j < cnt ? score_key(sr[j]) : 0u;
    const int rs = (int)max<int64_t>(1, min<int64_t>(ns, ((int64_t)fused_target(k) * ns + n - 1) / n));
    int unused_eq;
    const uint32_t t = select_own(kr, cnt, rs, s_hist, s_wave, s_mm, &unused_eq, false);
    if (tid == 0) tau[row] = t;
}

// Row t's top-k from its candidates (fill[t - off] of them, unordered, at cand + (t - off) *
// capr): an exact radix select finds the k-th key tau and how many keys equal to it to keep;
// an LDS bitmap over the row's positions marks the keys above tau and the kept ties (the
// lowest positions among the keys equal to tau), and the selection is emitted in position
// order.  Rows seeing at most k keys take every position.  A row whose candidates are fewer
// than k (the threshold was too high) or more than fit, or that holds more than TIE_CAP keys
// equal to tau, is flagged in fb for the exact path.  The candidates go straight from memory
// to registers (thread t: entries [SEL_PT t, +SEL_PT)), so LDS holds only the histogram, the
// bitmap and the tie list (dynamic: RES_HIST_BYTES + 4 bytes per 32 positions of the longest
// row + RES_TIE_BYTES), and four workgroups share a CU on rows of up to 128K keys.
constexpr int RES_HIST_BYTES = 4 * 4096;
constexpr int TIE_CAP = 256;
constexpr int RES_TIE_BYTES = 4 * TIE_CAP;
__global__ __launch_bounds__(TK_THREADS) void topk_resolve_kernel(
    const uint2* __restrict__ cand, int capr, const int* __restrict__ fill, int L, int q_pos0,
    int k, int off, int32_t* __restrict__ idx, int* __restrict__ fb)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
    __shared__ int s_wave_mem[2 * TK_WAVES];
    ScanBuf s_wave{s_wave_mem, 0};
    __shared__ uint32_t s_mm[2 * TK_WAVES];
    __shared__ int s_ntie;
    int* hist = reinterpret_cast<int*>(s_dyn);

    const int row = blockIdx.x, tid = threadIdx.x;
    const int n = min(L, q_pos0 + row + 1);
    int32_t* out = idx + (int64_t)row * k;
    if (n <= k) {                                       // every visible position
        for (int j = tid; j < k; j += TK_THREADS) out[j] = j < n ? j : -1;
        return;
    }
    const int cr = row - off;
    const int nc = fill[cr];
    if (nc < k || nc > min(capr, CAND_CAP)) {           // uniform
        if (tid == 0) fb[cr] = 1;
        return;
    }
    const uint2* src = cand + (int64_t)cr * capr + SEL_PT * tid;
    const int cnt = max(0, min(SEL_PT, nc - SEL_PT * tid));
    uint32_t kr[SEL_PT];
    int pr[SEL_PT];
    if (cnt == SEL_PT) {                                // 16-byte aligned: capr and SEL_PT even
#pragma unroll
        for (int q = 0; q < SEL_PT / 2; ++q) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(src + 2 * q);
            kr[2 * q] = score_key(__uint_as_float(v[0]));
            pr[2 * q] = (int)v[1];
            kr[2 * q + 1] = score_key(__uint_as_float(v[2]));
            pr[2 * q + 1] = (int)v[3];
        }
    } else {
#pragma unroll
        for (int j = 0; j < SEL_PT; ++j) {
            const uint2 e = j < cnt ? src[j] : make_uint2(0u, 0u);
            kr[j] = score_key(__uint_as_float(e.x));
            pr[j] = (int)e.y;
        }
    }
    // bitmap over positions 0 .. n-1 (nw words) and tie list after the histogram, cleared
    // here: the selection's barriers order the clearing before the marking
    const int nw = (n + 31) >> 5;
    uint32_t* sel = reinterpret_cast<uint32_t*>(s_dyn + RES_HIST_BYTES);
    int* ties = reinterpret_cast<int*>(sel + nw);
    for (int i = tid; i < nw; i += TK_THREADS) sel[i] = 0u;
    if (tid == 0) s_ntie = 0;
    int need_eq;
    const uint32_t tau = select_own(kr, cnt, k, hist, s_wave, s_mm, &need_eq);
#pragma unroll
    for (int j = 0; j < SEL_PT; ++j) {
        if (j < cnt && kr[j] > tau) {
            atomicOr(&sel[pr[j] >> 5], 1u << (pr[j] & 31));
        } else if (j < cnt && kr[j] == tau) {
            const int t = atomicAdd(&s_ntie, 1);
            if (t < TIE_CAP) ties[t] = pr[j];
        }
    }
    __syncthreads();
    const int nt = s_ntie;                              // >= need_eq >= 1
    if (nt > TIE_CAP) {                                 // uniform
        if (tid == 0) fb[cr] = 1;
        return;
    }
    // the need_eq ties of lowest position join the selection (positions are distinct)
    for (int i = tid; i < nt; i += TK_THREADS) {
        const int p = ties[i];
        int rank = 0;
        if (nt > need_eq)
            for (int j = 0; j < nt; ++j) rank += ties[j] < p ? 1 : 0;
        if (rank < need_eq) atomicOr(&sel[p >> 5], 1u << (p & 31));
    }
    __syncthreads();
    // emit in position order: thread t owns words [wpt t, wpt t + wpt)
    const int wpt = (nw + TK_THREADS - 1) / TK_THREADS;
    const int w0 = min(nw, wpt * tid), w1 = min(nw, w0 + wpt);
    int ns = 0;
    for (int i = w0; i < w1; ++i) ns += __popc(sel[i]);
    int tot;
    int slot = block_excl_scan(ns, s_wave, &tot);
    for (int i = w0; i < w1; ++i) {
        uint32_t m = sel[i];
        while (m) {
            const int b = __builtin_ctz(m);
            m &= m - 1u;
            if (slot < k) out[slot] = 32 * i + b;
            ++slot;
        }
    }
}

}  // namespace

// Every 32nd key (at most SAMPLE of them)
int fused_sample_stride(int L) { return std::max(32, (L + SAMPLE - 1) / SAMPLE); }

bool fused_select_supports(int L, int k)
{
    // candidates aim at 2k within CAND_CAP; a row's candidate array (8 bytes each) takes no
    // more room than its fp32 scores would; the resolve's histogram, position bitmap and tie
    // list fit 64 KB of LDS
    static_assert(RES_HIST_BYTES + 4 * CAND_CAP + RES_TIE_BYTES <= 65536,
                  "resolve LDS at the longest row");
    return 2 * k <= CAND_CAP && L >= 2 * CAND_CAP && L <= 32 * CAND_CAP;
}

int fused_cand_cap() { return CAND_CAP; }

int fused_sample_count(int L) { return (L - 1) / fused_sample_stride(L) + 1; }

hipError_t launch_topk_threshold(const float* samp, int64_t ld, int T, int L, int q_pos0,
                                 int k, uint32_t* tau, int* fill, int* fb, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_threshold_kernel, dim3(T), dim3(TK_THREADS), 0, stream, samp, ld,
                       fused_sample_stride(L), L, q_pos0, k, tau, fill, fb);
    return hipGetLastError();
}

hipError_t launch_topk_resolve(const uint2* cand, int capr, const int* fill, int T, int L,
                               int q_pos0, int k, int off, int32_t* idx, int* fb,
                               hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    const int64_t nmax = std::min<int64_t>(L, (int64_t)q_pos0 + T);
    const size_t lds = RES_HIST_BYTES + 4 * (size_t)((nmax + 31) / 32) + RES_TIE_BYTES;
    if (lds > 65536) return hipErrorInvalidValue;       // rows longer than the candidate path takes
    hipLaunchKernelGGL(topk_resolve_kernel, dim3(T), dim3(TK_THREADS), lds, stream, cand, capr,
                       fill, L, q_pos0, k, off, idx, fb);
    return hipGetLastError();
}

hipError_t launch_topk_prefill_only(const float* scores, int64_t ld, int T, int L, int q_pos0,
                                    int k, int32_t* idx, const int* only, int only_off,
                                    hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel<false>, dim3(T), dim3(TK_THREADS), 0, stream, scores, ld,
                       (const int64_t*)nullptr, L, q_pos0, k, idx,
                       SegCands{nullptr, nullptr, nullptr, 0}, only, only_off);
    return hipGetLastError();
}

hipError_t launch_topk_prefill(const float* scores, int64_t ld, int T, int L, int q_pos0,
                               int k, int32_t* idx, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel<false>, dim3(T), dim3(TK_THREADS), 0, stream, scores, ld,
                       (const int64_t*)nullptr, L, q_pos0, k, idx, SegCands{nullptr, nullptr, nullptr, 0},
                       (const int*)nullptr, 0);
    return hipGetLastError();
}

// Rows of more than CAND_CAP keys are split over segments when max_len needs at most
// SEG_MAX of them: key and position buffers of B * nseg * CAND_CAP entries and nseg counts
// per row.
static int decode_nseg(int max_len)
{
    const int nseg = (max_len + SEG - 1) / SEG;
    return (max_len > CAND_CAP && nseg <= SEG_MAX) ? nseg : 0;
}

size_t topk_decode_workspace_bytes(int B, int max_len)
{
    const size_t nseg = (size_t)decode_nseg(max_len);
    if (B <= 0 || nseg == 0) return 0;
    return (size_t)B * nseg * (8 * (size_t)CAND_CAP + 4) + 16;
}

hipError_t launch_topk_decode(const float* scores, const int64_t* seq_start, int B, int max_len,
                              int k, int32_t* idx, void* ws, hipStream_t stream)
{
    if (B <= 0) return hipSuccess;
    SegCands seg{nullptr, nullptr, nullptr, 0};
    const int nseg = decode_nseg(max_len);
    if (nseg > 0 && ws) {
        const size_t n = (size_t)B * nseg * CAND_CAP;
        uint32_t* key = static_cast<uint32_t*>(ws);
        int32_t* pos = reinterpret_cast<int32_t*>(key + n);
        int32_t* cnt = pos + n;
        hipLaunchKernelGGL(topk_segment_kernel, dim3(nseg, B), dim3(TK_THREADS), 0, stream,
                           scores, seq_start, k, nseg, key, pos, cnt);
        seg = SegCands{key, pos, cnt, nseg};
    }
    hipLaunchKernelGGL(topk_kernel<true>, dim3(B), dim3(TK_THREADS), 0, stream, scores,
                       (int64_t)0, seq_start, max_len, 0, k, idx, seg, (const int*)nullptr, 0);
    return hipGetLastError();
}

}  // namespace dsa
