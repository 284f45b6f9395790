// kernels.h -- host-side launchers of the DSA kernels (internal to libdsa.so).
// Every launcher assumes arguments already validated by the C ABI layer and only
// enqueues work on `stream`.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// ---- lightning indexer --------------------------------------------------------------
// Extra inputs of the prefill indexer passes; the defaults give plain scores.
struct IdxExtra {
    int kstride = 1;                 // key index s reads cache row kstride * s (visible when
                                     // kstride * s <= the row's position): a strided sample
    int ksplit = 0;                  // keys per workgroup (a multiple of 128; 0: the default)
    const int* only = nullptr;       // rows t with only[t] == 0 are not scored
    const uint32_t* tau = nullptr;   // candidates: per-row thresholds (score_key images)
    int* fill = nullptr;             // candidates: per-row counts, 0 before the launch
    uint2* cand = nullptr;           // candidates: (score bits, position) arrays of capr per row
    int capr = 0;
};
// Scores of T query rows (positions q_pos0 + t) against keys 0..L-1; writes only the
// visible entries s <= q_pos0 + t of each row (row t at scores + t * ld).  kstride > 1 and
// only need indexer_fused_supports(H_I).
hipError_t launch_indexer_prefill(const uint8_t* q8, const float* qs, const float* w,
                                  const uint8_t* k8, const float* ks, int T, int L, int H_I,
                                  int q_pos0, float c, float* scores, int64_t ld,
                                  hipStream_t stream, const IdxExtra& ex = IdxExtra{});
// Candidates instead of scores: row t's visible keys with score_key(score) >= tau[t] are
// appended to cand + t * capr as (score bits, position) in no particular order (the score
// compared as a float against tau[t]'s inverse image); fill[t] counts all
// of them (entries past capr are counted, not stored).
bool indexer_fused_supports(int H_I);
hipError_t launch_indexer_candidates(const uint8_t* q8, const float* qs, const float* w,
                                     const uint8_t* k8, const float* ks, int T, int L, int H_I,
                                     int q_pos0, float c, const IdxExtra& ex,
                                     hipStream_t stream);
// Writes -inf to the masked entries q_pos0 + t < s < L of every row.
hipError_t launch_mask_fill(int T, int L, int q_pos0, float* scores, int64_t ld,
                            hipStream_t stream);
// Decode: query b scores every key of its packed cache slice [seq_start[b], seq_start[b+1])
// into scores[seq_start[b] + s].
hipError_t launch_indexer_decode(const uint8_t* q8, const float* qs, const float* w,
                                 const uint8_t* k8, const float* ks, const int64_t* seq_start,
                                 int B, int max_len, int H_I, float c, float* scores,
                                 hipStream_t stream);
bool indexer_supports(int H_I);

// ---- top-k ----------------------------------------------------------------------------
// Prefill rows: row t at scores + t * ld with n_t = min(L, q_pos0 + t + 1) visible scores.
hipError_t launch_topk_prefill(const float* scores, int64_t ld, int T, int L, int q_pos0,
                               int k, int32_t* idx, hipStream_t stream);
// The fused prefill selection (the indexer writes candidates, not scores):
//  1. launch_indexer_prefill with kstride = fused_sample_stride(L) scores the keys 0, S, 2S,
//     .. (fused_sample_count(L) per row at most) into samp;
//  2. launch_topk_threshold derives each row's threshold tau from them and clears fill, fb;
//  3. launch_indexer_candidates keeps the keys at or above tau (capr = fused_cand_cap());
//  4. launch_topk_resolve selects from the candidates, flagging in fb the rows whose
//     candidates cannot decide (fewer than k, more than the capacity, or more ties at the
//     k-th key than its tie list holds);
//  5. the flagged rows are scored (launch_indexer_prefill with only = fb) and selected by
//     launch_topk_prefill_only.
// Rows are relative to the chunk for the resolve (T rows from q_pos0, the first `off` of
// them seeing at most k keys) and to the first scored row for tau, fill and fb.
// Applies when fused_select_supports(L, k) and indexer_fused_supports(H_I).
bool fused_select_supports(int L, int k);
int fused_sample_stride(int L);
int fused_sample_count(int L);
int fused_cand_cap();
hipError_t launch_topk_threshold(const float* samp, int64_t ld, int T, int L, int q_pos0,
                                 int k, uint32_t* tau, int* fill, int* fb, hipStream_t stream);
hipError_t launch_topk_resolve(const uint2* cand, int capr, const int* fill, int T, int L,
                               int q_pos0, int k, int off, int32_t* idx, int* fb,
                               hipStream_t stream);
hipError_t launch_topk_prefill_only(const float* scores, int64_t ld, int T, int L, int q_pos0,
                                    int k, int32_t* idx, const int* only, int only_off,
                                    hipStream_t stream);
// Decode rows: row b at scores + seq_start[b] with seq_start[b+1] - seq_start[b] <= max_len
// scores (a row longer than max_len, outside that contract, selects nothing: all -1).  Long
// rows are split over several workgroups when ws (at least
// topk_decode_workspace_bytes(B, max_len) bytes, 16-byte aligned; may be null when that is
// 0) is given; otherwise each row is selected by one workgroup.
size_t topk_decode_workspace_bytes(int B, int max_len);
hipError_t launch_topk_decode(const float* scores, const int64_t* seq_start, int B, int max_len,
                              int k, int32_t* idx, void* ws, hipStream_t stream);

// ---- sparse MLA -----------------------------------------------------------------------
// Row t attends over kv rows idx[t, :] (entries outside [0, L) skipped).
// seq_start (nullable, device int64 [T+1]): row t's cache is the packed slice
// kv[seq_start[t] .. seq_start[t+1]) and its indices are relative to that slice.
// splits > 1: each split covers a contiguous slice of the index list and writes fp32
// partials (o normalised by its own denominator, lse) that launch_mla_combine merges.
// valid_pos0 >= 0: row t's list is a top-k selection with its valid entries first, min(k,
// valid_pos0 + t + 1) of them (prefill: position valid_pos0 + t) or min(k, L_t) (decode, with
// seq_start), and only those are visited; -1: the whole list of k entries is visited (padding
// anywhere).
hipError_t launch_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                             const int64_t* seq_start, int T, int L, int H, int k,
                             float sm_scale, int splits, uint16_t* out, float* lse,
                             float* part_o, float* part_lse, int valid_pos0, hipStream_t stream);
hipError_t launch_mla_combine(const float* part_o, const float* part_lse, int T, int H,
                              int splits, uint16_t* out, float* lse, hipStream_t stream);

// ---- fp8 preparation of the indexer inputs ------------------------------------------
// x [n,128] fp32 (or bf16 bits) -> q8 [n,128] e4m3fn, scale [n]: scale = amax / 448 (1 if 0),
// code = nearest-even e4m3fn of clamp(x / scale, +-448).  x 16-byte aligned, q8 8-byte.
hipError_t launch_quantize_fp8(const void* x, bool bf16, int64_t n, uint8_t* q8, float* scale,
                               hipStream_t stream);
// Row seq_start[b+1] - 1 of the packed caches gets the new token of sequence b.
hipError_t launch_decode_append(int B, const int64_t* seq_start, const void* k_new, bool bf16,
                                const uint16_t* kv_new, uint8_t* k8_cache, float* ks_cache,
                                uint16_t* kv_cache, hipStream_t stream);

// ---- alternative index rules ----------------------------------------------------------
// window: idx [T, W], row t = max(0, p-W+1) .. p (p = q_pos0 + t), -1 padded.
hipError_t launch_window_indices(int T, int q_pos0, int W, int32_t* idx, hipStream_t stream);
// local + selected: out [T, W + k] = ascending union of the window and sel [T, k].
hipError_t launch_local_selected(const int32_t* sel, int T, int k, int q_pos0, int W,
                                 int32_t* out, hipStream_t stream);

// ---- indexer warm-up (KL to the dense attention distribution) --------------------------
bool warmup_supports(int H_I, int H);
// lse [T,H] of dense causal attention of q [T,H,576] over kv rows 0..q_pos0+t.
hipError_t launch_attention_lse(const uint16_t* q, const uint16_t* kv, int T, int H, int q_pos0,
                                float sm_scale, float* lse, hipStream_t stream);
// P[t, s <= q_pos0 + t] = (1/H) sum_h exp(logit - lse[t,h]); P rows at stride ld.
hipError_t launch_attention_dist(const uint16_t* q, const uint16_t* kv, const float* lse, int T,
                                 int H, int q_pos0, float sm_scale, float* P, int64_t ld,
                                 hipStream_t stream);
// Per row over s <= q_pos0 + t: kl[t], lse_i[t] (nullable) and G = softmax(I) - P over PG.
hipError_t launch_warmup_rows(const float* I, float* PG, int64_t ld, int T, int q_pos0,
                              float* kl, float* lse_i, hipStream_t stream);
hipError_t launch_warmup_dq(const uint8_t* q8, const float* qs, const float* w, const uint8_t* k8,
                            const float* ks, const float* G, int64_t ld, int T, int H_I,
                            int q_pos0, float c, float* dq, float* dw, hipStream_t stream);
// Adds this call's rows' contribution to the per-16-head-group partials dkp [H_I/16][L][128]
// (keys 0 .. q_pos0 + T - 1); dk = their sum over groups (launch_warmup_dk_reduce).
hipError_t launch_warmup_dk(const uint8_t* q8, const float* qs, const float* w, const uint8_t* k8,
                            const float* G, int64_t ld, int T, int H_I, int q_pos0, float c,
                            int64_t L, float* dkp, hipStream_t stream);
hipError_t launch_warmup_dk_reduce(const float* dkp, int ngroups, int64_t n, float* dk,
                                   hipStream_t stream);
hipError_t launch_zero(float* p, int64_t n, hipStream_t stream);

}  // namespace dsa
