// index_rules.hip -- index lists of the alternative rules that feed the sparse MLA.
//
// DSA generalises sliding-window attention (gxzdkb DSA explainer, section 秘密武器：DSA); a
// local window can also be joined by globally chosen tokens (oilbeater.com "DeepSeek Sparse
// Attention", section Sparse Attention).  Both rules are index lists in the layout
// dsa_sparse_mla reads: ascending positions, -1 padding.
//   window W:          row t (position p = q_pos0 + t) keeps max(0, p-W+1) .. p;
//   local + selected:  the ascending union of that window and the row's selected positions.
#include "dsa_device.h"
#include "kernels.h"

namespace dsa {
namespace {

__global__ __launch_bounds__(256) void window_kernel(int T, int q_pos0, int W, int32_t* __restrict__ idx)
{
    const int64_t total = (int64_t)T * W;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * 256) {
        const int t = (int)(e / W), j = (int)(e - (int64_t)t * W);
        const int p = q_pos0 + t, lo = max(0, p - W + 1);
        idx[e] = lo + j <= p ? lo + j : -1;
    }
}

// One wave per row.  The row's valid selected positions (ascending, as the top-k writes
// them; -1 entries anywhere are skipped) below the window are compacted in order, then the
// window follows, then -1 padding up to W + k entries.
__global__ __launch_bounds__(256) void local_selected_kernel(const int32_t* __restrict__ sel, int T,
                                                             int k, int q_pos0, int W,
                                                             int32_t* __restrict__ out)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (t >= T) return;                                      // whole waves; no barriers
    const int p = q_pos0 + t, lo = max(0, p - W + 1), nw = p - lo + 1;
    const int M = W + k;
    const int32_t* s = sel + (int64_t)t * k;
    int32_t* o = out + (int64_t)t * M;
    int c = 0;
    for (int j0 = 0; j0 < k; j0 += 64) {
        const int j = j0 + lane;
        const int v = j < k ? s[j] : -1;
        const bool keep = v >= 0 && v < lo;
        const uint64_t m = __ballot(keep);
        if (keep) o[c + __popcll(m & lanemask_lt(lane))] = v;
        c += __popcll(m);
    }
    for (int i = lane; i < M - c; i += 64) o[c + i] = i < nw ? lo + i : -1;
}

}  // namespace

hipError_t launch_window_indices(int T, int q_pos0, int W, int32_t* idx, hipStream_t stream)
{
    const int64_t total = (int64_t)T * W;
    if (total <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((total + 255) / 256, 1 << 20);
    hipLaunchKernelGGL(window_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, T, q_pos0, W,
                       idx);
    return hipGetLastError();
}

hipError_t launch_local_selected(const int32_t* sel, int T, int k, int q_pos0, int W,
                                 int32_t* out, hipStream_t stream)
{
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(local_selected_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, sel, T, k,
                       q_pos0, W, out);
    return hipGetLastError();
}

}  // namespace dsa
