// topk.hip -- per-row top-k selection on gfx950.
//
// Row t keeps the k largest of its n_t visible scores; a row with n_t <= k keeps all of
// 0..n_t-1 (《DeepSeek-V3.2-Exp模型优势与 DSA 工作原理》 §4 步骤三 and §2 风险边界明确).  Ties
// go to the lower position and -0 equals +0, which makes the selected set unique.
//
// Method: scores map to order-preserving uint32 keys; a three-level radix select (11, 11
// and 10 bits, LDS histograms) finds the exact k-th key tau and how many ties at tau are
// needed; a final position-ordered sweep emits every key > tau and the lowest-position
// ties, compacted with wave ballots, so the output is in ascending position order.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;

// Block-wide exclusive prefix sum of one int per thread (ascending thread order).
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

// One workgroup per row.
template <bool DECODE>
__global__ __launch_bounds__(TK_THREADS) void topk_radix_kernel(
    const float* __restrict__ scores, int64_t ld, const int64_t* __restrict__ seq_start, int L,
    int q_pos0, int k, int32_t* __restrict__ idx)
{
    __shared__ int s_hist[2048];
    __shared__ int s_wave[TK_WAVES];
    __shared__ int s_res[2];
    __shared__ int s_tot[2][TK_WAVES];

    const int row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const RowRef rr = row_of<DECODE>(row, scores, ld, seq_start, L, q_pos0);
    const int n = rr.n;
    int32_t* out = idx + (int64_t)row * k;

    if (n <= k) {                                   // short row: everything visible
        for (int j = tid; j < k; j += TK_THREADS) out[j] = j < n ? j : -1;
        return;
    }

    // ---- radix select of the k-th largest key
    uint32_t prefix = 0;                            // bits of tau fixed so far
    int k_rem = k;                                  // still needed at or below the prefix
    const int shifts[3] = {21, 10, 0};
    const int widths[3] = {11, 11, 10};
#pragma unroll 1
    for (int lvl = 0; lvl < 3; ++lvl) {
        const int sh = shifts[lvl], nb = 1 << widths[lvl];
        const int hi_sh = sh + widths[lvl];        // bits above this level's digit
        for (int i = tid; i < nb; i += TK_THREADS) s_hist[i] = 0;
        __syncthreads();
        for (int s = tid; s < n; s += TK_THREADS) {
            const uint32_t u = score_key(rr.p[s]);
            const bool match = (lvl == 0) || ((u >> hi_sh) == prefix);
            if (match) atomicAdd(&s_hist[(u >> sh) & (nb - 1)], 1);
        }
        __syncthreads();
        // thread i covers bins nb-1-i*per .. descending; scan gives the count above each
        const int per = nb / TK_THREADS;            // 2 or 1
        int cnt[2] = {0, 0}, sum = 0;
        for (int q = 0; q < per; ++q) {
            cnt[q] = s_hist[nb - 1 - tid * per - q];
            sum += cnt[q];
        }
        int total;
        int above = block_excl_scan(sum, s_wave, &total);
        for (int q = 0; q < per; ++q) {
            if (above < k_rem && k_rem <= above + cnt[q]) {
                s_res[0] = nb - 1 - tid * per - q;
                s_res[1] = k_rem - above;
            }
            above += cnt[q];
        }
        __syncthreads();
        prefix = (prefix << widths[lvl]) | (uint32_t)s_res[0];
        k_rem = s_res[1];
        __syncthreads();
    }
    const uint32_t tau = prefix;
    const int need_eq = k_rem;                       // ties at tau to take, lowest first

    // ---- position-ordered emission: slot = #(key > tau before s) + min(#ties before s, need)
    int base_gt = 0, base_eq = 0;
    const unsigned long long lt = lanemask_lt(lane);
    for (int s0 = 0; s0 < n; s0 += TK_THREADS) {
        const int s = s0 + tid;
        uint32_t u = 0;
        if (s < n) u = score_key(rr.p[s]);
        const bool gt = s < n && u > tau;
        const bool eq = s < n && u == tau;
        const unsigned long long bg = __ballot(gt), be = __ballot(eq);
        if (lane == 0) {
            s_tot[0][wave] = __popcll(bg);
            s_tot[1][wave] = __popcll(be);
        }
        __syncthreads();
        int off_gt = base_gt, off_eq = base_eq, tot_gt = 0, tot_eq = 0;
#pragma unroll
        for (int i = 0; i < TK_WAVES; ++i) {
            const int a = s_tot[0][i], b = s_tot[1][i];
            off_gt += (i < wave) ? a : 0;
            off_eq += (i < wave) ? b : 0;
            tot_gt += a;
            tot_eq += b;
        }
        const int my_gt = off_gt + __popcll(bg & lt);
        const int my_eq = off_eq + __popcll(be & lt);
        const int slot_gt = my_gt + min(my_eq, need_eq), slot_eq = my_gt + my_eq;
        if (gt && slot_gt < k) out[slot_gt] = s;
        if (eq && my_eq < need_eq && slot_eq < k) out[slot_eq] = s;
        base_gt += tot_gt;
        base_eq += tot_eq;
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_topk_prefill(const float* scores, int64_t ld, int T, int L, int q_pos0,
                               int k, int32_t* idx, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_radix_kernel<false>, dim3(T), dim3(TK_THREADS), 0, stream, scores,
                       ld, (const int64_t*)nullptr, L, q_pos0, k, idx);
    return hipGetLastError();
}

hipError_t launch_topk_decode(const float* scores, const int64_t* seq_start, int B, int k,
                              int32_t* idx, hipStream_t stream)
{
    if (B <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_radix_kernel<true>, dim3(B), dim3(TK_THREADS), 0, stream, scores,
                       (int64_t)0, seq_start, 0, 0, k, idx);
    return hipGetLastError();
}

}  // namespace dsa
