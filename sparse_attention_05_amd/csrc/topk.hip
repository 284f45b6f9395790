// topk.hip -- per-row top-k selection on gfx950.
//
// Row t keeps the k largest of its n_t visible scores; a row with n_t <= k keeps all of
// 0..n_t-1 (《DeepSeek-V3.2-Exp模型优势与 DSA 工作原理》 §4 步骤三 and §2 风险边界明确).  Ties
// go to the lower position and -0 equals +0, which makes the selected set unique.
//
// Scores map to order-preserving uint32 keys.  One workgroup per row:
//   pass 1  streams the row once into a 4096-bin LDS histogram of the top 12 key bits and
//           finds the boundary bin b holding the k-th largest key;
//   pass 2  streams the row again; positions whose bin is above b are final (list S, kept
//           in position order by ballot/scan compaction), and the boundary bin's entries
//           become LDS candidates (key, position), also in position order;
//   resolve two more radix levels (10 + 10 bits) over the candidates in LDS give the exact
//           k-th key tau; the candidates above tau and the lowest-position ties at tau
//           form list C;
//   merge   S and C are both ascending, so each element's output slot is its index plus
//           its rank in the other list (binary search): the output is in ascending order.
// A row whose boundary bin holds more than TK_CAP keys falls back to radix levels over
// the row in global memory and a position-ordered emission sweep.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_BINS = 4096;               // first digit: key bits 31..20
constexpr int TK_CAP = 3072;                // boundary-bin candidates kept in LDS
constexpr int TK_KMAX = 8192;

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

// Block-wide exclusive prefix sum (ascending thread order) and total.
__device__ __forceinline__ int block_excl_scan(int v, int* s_wave, int* total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < TK_WAVES; ++i) {
        const int c = s_wave[i];
        off += (i < wave) ? c : 0;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return off + x - v;
}

// Boundary bin of a descending histogram: the bin B with count(bins > B) < need <=
// count(bins >= B).  Returns B and stores need - count(bins > B) in *rem.  hist has
// nb = per * TK_THREADS bins; thread i covers bins nb-1-i*per downwards.
template <int PER>
__device__ __forceinline__ int boundary_bin(const int* hist, int need, int* s_wave, int* s_res,
                                            int* rem)
{
    constexpr int NB = PER * TK_THREADS;
    const int tid = threadIdx.x;
    int cnt[PER], sum = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        cnt[q] = hist[NB - 1 - tid * PER - q];
        sum += cnt[q];
    }
    int total;
    int above = block_excl_scan(sum, s_wave, &total);
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if (above < need && need <= above + cnt[q]) {
            s_res[0] = NB - 1 - tid * PER - q;
            s_res[1] = need - above;
        }
        above += cnt[q];
    }
    __syncthreads();
    const int b = s_res[0];
    *rem = s_res[1];
    __syncthreads();
    return b;
}

// Visit the row in rounds of up to 4 * TK_THREADS consecutive positions; within a round,
// thread t owns positions [4t, 4t + 4) of the round (fewer in the unaligned head and the
// tail), so thread order is position order.  f(pos[4], key[4], cnt) is called by every
// thread in every round (cnt may be 0); rounds are uniform across the workgroup.
template <typename F>
__device__ __forceinline__ void for_row_rounds(const RowRef& rr, F&& f)
{
    const int tid = threadIdx.x;
    const int n = rr.n;
    const int mis = (int)((reinterpret_cast<uintptr_t>(rr.p) >> 2) & 3);
    const int head = min(n, (4 - mis) & 3);            // scalars until 16-byte aligned
    int pos[4];
    uint32_t key[4];
    if (head > 0) {                                     // uniform
        const int c = tid < head ? 1 : 0;
        pos[0] = tid;
        key[0] = c ? score_key(rr.p[tid]) : 0u;
        f(pos, key, c);
    }
    const int body = (n - head) & ~3;
    const v4f* p4 = reinterpret_cast<const v4f*>(rr.p + head);
    for (int base = 0; base < body; base += 4 * TK_THREADS) {
        const int e = base + 4 * tid;
        int c = 0;
        if (e < body) {
            const v4f v = p4[e >> 2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pos[j] = head + e + j;
                key[j] = score_key(v[j]);
            }
            c = 4;
        }
        f(pos, key, c);
    }
    const int tail = n - head - body;                   // 0..3
    if (tail > 0) {
        const int c = tid < tail ? 1 : 0;
        pos[0] = head + body + tid;
        key[0] = c ? score_key(rr.p[head + body + tid]) : 0u;
        f(pos, key, c);
    }
}

template <bool DECODE>
__global__ __launch_bounds__(TK_THREADS) void topk_kernel(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ seq_start, int L,
    int q_pos0, int k, int32_t* __restrict__ idx)
{
    __shared__ int s_hist[TK_BINS];
    __shared__ int s_sel[TK_KMAX];            // S: final positions above the boundary bin
    __shared__ uint32_t s_ckey[TK_CAP];       // boundary-bin candidates (key, position)
    __shared__ int s_cpos[TK_CAP];
    __shared__ int s_wave[TK_WAVES];
    __shared__ int s_res[4];

    const int row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const RowRef rr = row_of<DECODE>(row, scores, ld, seq_start, L, q_pos0);
    const int n = rr.n;
    int32_t* out = idx + (int64_t)row * k;

    if (n <= k) {                                 // short row: every visible position
        for (int j = tid; j < k; j += TK_THREADS) out[j] = j < n ? j : -1;
        return;
    }

    // ---- pass 1: histogram of key bits 31..20
    for (int i = tid; i < TK_BINS; i += TK_THREADS) s_hist[i] = 0;
    __syncthreads();
    for_row_rounds(rr, [&](const int*, const uint32_t* key, int c) {
        for (int j = 0; j < c; ++j) atomicAdd(&s_hist[key[j] >> 20], 1);
    });
    __syncthreads();
    int need_b;                                   // keys still needed from the boundary bin
    const uint32_t b = (uint32_t)boundary_bin<TK_BINS / TK_THREADS>(s_hist, k, s_wave, s_res,
                                                                    &need_b);
    const int n_above = k - need_b;               // keys in bins above b (all selected)
    const int n_cand = s_hist[b];
    __syncthreads();

    if (n_cand <= TK_CAP) {
        // ---- pass 2: S (bins above b) and the boundary candidates, both position-ordered
        int base_s = 0, base_c = 0;
        for_row_rounds(rr, [&](const int* pos, const uint32_t* key, int c) {
            int ns = 0, nc = 0;
            for (int j = 0; j < c; ++j) {
                const uint32_t d = key[j] >> 20;
                ns += d > b;
                nc += d == b;
            }
            int tot;
            const int off = block_excl_scan(ns | (nc << 16), s_wave, &tot);
            int os = base_s + (off & 0xFFFF), oc = base_c + (off >> 16);
            for (int j = 0; j < c; ++j) {
                const uint32_t d = key[j] >> 20;
                if (d > b) s_sel[os++] = pos[j];
                else if (d == b) {
                    s_ckey[oc] = key[j];
                    s_cpos[oc++] = pos[j];
                }
            }
            base_s += tot & 0xFFFF;
            base_c += tot >> 16;
        });
        __syncthreads();

        // ---- resolve the candidates: key bits 19..10, then 9..0
        uint32_t prefix = b;
        int need = need_b;
#pragma unroll 1
        for (int lvl = 0; lvl < 2; ++lvl) {
            const int sh = lvl == 0 ? 10 : 0;
            for (int i = tid; i < 1024; i += TK_THREADS) s_hist[i] = 0;
            __syncthreads();
            for (int i = tid; i < n_cand; i += TK_THREADS) {
                const uint32_t u = s_ckey[i];
                if ((u >> (sh + 10)) == prefix) atomicAdd(&s_hist[(u >> sh) & 1023], 1);
            }
            __syncthreads();
            int rem;
            const int d = boundary_bin<1>(s_hist, need, s_wave, s_res, &rem);
            prefix = (prefix << 10) | (uint32_t)d;
            need = rem;
        }
        const uint32_t tau = prefix;              // exact k-th largest key
        const int need_eq = need;                 // ties at tau to keep, lowest first

        // chosen candidates (key > tau, or the first need_eq ties) -> list C in s_ckey
        // (reused as int positions), position order kept by an ordered scan
        int base_g = 0, base_e = 0;
        for (int r0 = 0; r0 < n_cand; r0 += 4 * TK_THREADS) {
            uint32_t ku[4];
            int pp[4], ng = 0, ne = 0;
            for (int j = 0; j < 4; ++j) {
                const int i = r0 + 4 * tid + j;
                ku[j] = i < n_cand ? s_ckey[i] : 0u;
                pp[j] = i < n_cand ? s_cpos[i] : -1;
                ng += (i < n_cand) && ku[j] > tau;
                ne += (i < n_cand) && ku[j] == tau;
            }
            int tot;
            const int off = block_excl_scan(ng | (ne << 16), s_wave, &tot);
            int eq_before = base_e + (off >> 16);
            int slot = base_g + (off & 0xFFFF) + min(eq_before, need_eq);
            __syncthreads();                      // all reads of s_ckey in this round done
            for (int j = 0; j < 4; ++j) {
                const int i = r0 + 4 * tid + j;
                if (i >= n_cand) break;
                if (ku[j] > tau) {
                    reinterpret_cast<int*>(s_ckey)[slot++] = pp[j];
                } else if (ku[j] == tau) {
                    if (eq_before < need_eq) reinterpret_cast<int*>(s_ckey)[slot++] = pp[j];
                    ++eq_before;
                }
            }
            base_g += tot & 0xFFFF;
            base_e += tot >> 16;
            __syncthreads();
        }
        // C holds need_b positions, ascending; S holds n_above positions, ascending.
        const int* C = reinterpret_cast<const int*>(s_ckey);
        for (int i = tid; i < n_above; i += TK_THREADS) {
            const int p = s_sel[i];
            int lo = 0, hi = need_b;              // count of C below p
            while (lo < hi) {
                const int m = (lo + hi) >> 1;
                if (C[m] < p) lo = m + 1; else hi = m;
            }
            out[i + lo] = p;
        }
        for (int i = tid; i < need_b; i += TK_THREADS) {
            const int p = C[i];
            int lo = 0, hi = n_above;             // count of S below p
            while (lo < hi) {
                const int m = (lo + hi) >> 1;
                if (s_sel[m] < p) lo = m + 1; else hi = m;
            }
            out[i + lo] = p;
        }
        return;
    }

    // ---- fallback: two more radix levels over the row in global memory
    uint32_t prefix = b;
    int need = need_b;
#pragma unroll 1
    for (int lvl = 0; lvl < 2; ++lvl) {
        const int sh = lvl == 0 ? 10 : 0;
        for (int i = tid; i < 1024; i += TK_THREADS) s_hist[i] = 0;
        __syncthreads();
        for_row_rounds(rr, [&](const int*, const uint32_t* key, int c) {
            for (int j = 0; j < c; ++j)
                if ((key[j] >> (sh + 10)) == prefix) atomicAdd(&s_hist[(key[j] >> sh) & 1023], 1);
        });
        __syncthreads();
        int rem;
        const int d = boundary_bin<1>(s_hist, need, s_wave, s_res, &rem);
        prefix = (prefix << 10) | (uint32_t)d;
        need = rem;
    }
    const uint32_t tau = prefix;
    const int need_eq = need;
    // slot of a selected position = #(key > tau before it) + min(#ties before it, need_eq)
    int base_gt = 0, base_eq = 0;
    (void)lane;
    for_row_rounds(rr, [&](const int* pos, const uint32_t* key, int c) {
        int ng = 0, ne = 0;
        for (int j = 0; j < c; ++j) {
            ng += key[j] > tau;
            ne += key[j] == tau;
        }
        int tot;
        const int off = block_excl_scan(ng | (ne << 16), s_wave, &tot);
        int gt_before = base_gt + (off & 0xFFFF);
        int eq_before = base_eq + (off >> 16);
        for (int j = 0; j < c; ++j) {
            if (key[j] > tau) {
                const int slot = gt_before + min(eq_before, need_eq);
                if (slot < k) out[slot] = pos[j];
                ++gt_before;
            } else if (key[j] == tau) {
                if (eq_before < need_eq && gt_before + eq_before < k)
                    out[gt_before + eq_before] = pos[j];
                ++eq_before;
            }
        }
        base_gt += tot & 0xFFFF;
        base_eq += tot >> 16;
    });
}

}  // namespace

hipError_t launch_topk_prefill(const float* scores, int64_t ld, int T, int L, int q_pos0,
                               int k, int32_t* idx, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel<false>, dim3(T), dim3(TK_THREADS), 0, stream, scores, ld,
                       (const int64_t*)nullptr, L, q_pos0, k, idx);
    return hipGetLastError();
}

hipError_t launch_topk_decode(const float* scores, const int64_t* seq_start, int B, int k,
                              int32_t* idx, hipStream_t stream)
{
    if (B <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel<true>, dim3(B), dim3(TK_THREADS), 0, stream, scores,
                       (int64_t)0, seq_start, 0, 0, k, idx);
    return hipGetLastError();
}

}  // namespace dsa
