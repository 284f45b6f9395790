/*
 * dsa.h -- C ABI of the DeepSeek Sparse Attention (DSA) hot path on AMD MI355X (gfx950).
 *
 * The method (pages cited by title and section):
 *   [csdn-workflow] 《DeepSeek-V3.2-Exp模型优势与 DSA 工作原理,token降价性能不减的背后》
 *                   (agent.csdn.net): §3 两大核心组件 (a 128-d indexer key per token, a
 *                   512-d latent cache for the sparse MLA), §4 四步工作流程 (步骤二 indexer
 *                   score with mask and scale and per-head weights a_h, 步骤三 top-k with
 *                   k = 2048 and select-all for short contexts, 步骤四 sparse MLA).
 *   [devpress-dsa]  《狂降75%！大模型DeepSeek-V3.2 API杀疯了…》 (devpress.csdn.net):
 *                   §三 第二步–第四步 (the same four steps).
 *   [oilbeater-dsa] oilbeater.com "DeepSeek Sparse Attention": section Sparse Attention
 *                   (sliding windows, local windows joined by global tokens).
 *   [yufo-notes]    ele-yufo.com notes "DeepSeek V3.2-Exp": §四 训练的两步走冷启动, 第一阶段
 *                   Warm-up (the frozen main model's dense attention distribution is the
 *                   target the indexer alone is fitted to, by KL divergence).
 *   [gxzdkb-dsa]    gxzdkb.com DSA explainer: 秘密武器：DSA (fp8 indexer, ReLU),
 *                   原始 Attention 的计算逻辑 (decode appends to the cache first),
 *                   致命问题：平方级复杂度拖垮效率 (rollout inference = prefill, which builds
 *                   every token's cache entry and output, then decode).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  Tensors are row-major
 *     and contiguous unless a leading dimension is given.  fp8 = OCP e4m3fn bytes,
 *     bf16 = raw uint16 bits, scales fp32.
 *   - Indexer: one shared 128-byte fp8 key per token (k8[L,128]) with a per-token fp32
 *     scale ks[L]; query row t has H_I fp8 heads q8[t,h,128] with per-(token,head) scales
 *     qs[t,h] and per-head weights w[t,h] (the pages' a_h).
 *   - MLA: one 576-wide bf16 cache row per token, kv[L,576] = 512 latent (also the value)
 *     + 64 rope dims; queries q[T,H,576]; outputs out[T,H,512] bf16 and lse[T,H] fp32
 *     (natural log of the softmax denominator).
 *   - Query row t sits at absolute position p_t = q_pos0 + t and sees keys 0..p_t, itself
 *     included.  Requires q_pos0 >= 0 and q_pos0 + T <= L.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the default stream)
 *     and returns.  Arguments are validated before any HIP call: an invalid call returns
 *     its status and launches nothing.  Launch failures return DSA_ERR_HIP.  The library
 *     allocates no memory; it keeps no global state except the fixed scratch array of
 *     dsa_decode_noalloc (one per GPU, see there).  Calls are thread-safe.  The caller
 *     keeps every buffer alive until the stream has reached the call.
 *   - DSA_LOG=1 in the environment prints one line per call (entry point, sizes, status)
 *     to stderr.
 *   - Not checked on the device (the caller's contract): scales positive and finite, no
 *     NaN fp8 codes (0x7F/0xFF), finite bf16 values, index lists without duplicates.
 *   - Supported shapes: H_I in {1,2,4,8,16,32,64,128}; 1 <= H <= 128;
 *     1 <= k <= 8192 (index lists of dsa_sparse_mla: any k >= 1); L < 2^31;
 *     T * max(L, k) < 2^40; a latent cache an attention call (or a sequence of a batch)
 *     addresses holds at most 1,864,135 rows (2 GiB of 1152-byte rows: L, each varlen
 *     sequence's keys, decode's max_len).  Other shapes return DSA_ERR_UNSUPPORTED.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* dsa_stream_t;   /* identical to hipStream_t */

typedef enum {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARGUMENT = 1,    /* null pointer, negative size, q_pos0 + T > L, ... */
    DSA_ERR_UNSUPPORTED = 2,         /* a shape outside the supported set */
    DSA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below the matching *_workspace_bytes */
    DSA_ERR_HIP = 4                  /* a HIP launch or runtime error */
} dsa_status_t;

/* Static, human-readable name of a status code. */
const char* dsa_status_string(dsa_status_t status);

/* ABI version: major * 100 + minor (1.02: + dsa_quantize_fp8, dsa_decode_append, dsa_window_indices,
 * dsa_local_selected_indices; 1.03: + dsa_prefill_varlen, dsa_prefill_varlen_workspace_bytes;
 * 1.04: + dsa_attention_lse, dsa_attention_distribution, dsa_indexer_warmup,
 * dsa_indexer_warmup_workspace_bytes; 1.05: + dsa_decode_noalloc,
 * dsa_decode_noalloc_scratch_bytes). */
int dsa_version(void);

/* Lightning-indexer scores ([csdn-workflow] §4 步骤二, [devpress-dsa] §三 第二步):
 *   score[t,s] = ks[s] * sum_h (w[t,h] * qs[t,h] * score_scale) * ReLU(sum_d q8[t,h,d] k8[s,d])
 * for s <= q_pos0 + t.  The masked entries q_pos0 + t < s < L receive -inf when write_masked
 * is non-zero and are left untouched otherwise (for callers that only read visible
 * entries, as dsa_topk does).  fp8 products are exact, accumulation and the epilogue fp32.
 *   q8 [T,H_I,128] u8; q_scale [T,H_I] f32; w [T,H_I] f32; k8 [L,128] u8; k_scale [L] f32;
 *   scores [T, ld_scores] f32 with ld_scores >= L (columns >= L are not written). */
dsa_status_t dsa_index_scores(const uint8_t* q8, const float* q_scale, const float* w,
                              const uint8_t* k8, const float* k_scale, int T, int L, int H_I,
                              int q_pos0, float score_scale, float* scores, int64_t ld_scores,
                              int write_masked, dsa_stream_t stream);

/* Per-row top-k ([csdn-workflow] §4 步骤三): row t keeps the k largest of its n_t =
 * q_pos0 + t + 1 visible scores, ties to the lower position, -0 equal to +0; a row with
 * n_t <= k keeps all of 0..n_t-1 without reading its scores.  idx [T,k] int32 receives
 * the positions in ascending order, then -1 padding.  Scores must not be NaN.
 * Uses no workspace (workspace may be NULL when dsa_topk_workspace_bytes returns 0). */
dsa_status_t dsa_topk(const float* scores, int64_t ld_scores, int T, int L, int q_pos0, int k,
                      int32_t* idx, void* workspace, size_t workspace_bytes,
                      dsa_stream_t stream);
size_t dsa_topk_workspace_bytes(int T, int L, int k);

/* Sparse MLA ([csdn-workflow] §4 步骤四, [devpress-dsa] §三 第四步): for each row t, head h
 *   l_j = sm_scale * <q[t,h,0:576], kv[idx[t,j],0:576]>,   out[t,h] = softmax(l) . kv[idx,0:512],
 *   lse[t,h] = log sum_j exp(l_j).
 * Entries of idx outside [0, L) are padding and skipped; a row with no valid entry gives
 * out = 0 and lse = -inf.  q [T,H,576] bf16; kv [L,576] bf16; idx [T,k] int32;
 * out [T,H,512] bf16 (rounded to nearest even); lse [T,H] f32 or NULL. */
dsa_status_t dsa_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int T,
                            int L, int H, int k, float sm_scale, uint16_t* out, float* lse,
                            dsa_stream_t stream);

/* The whole prefill path for T query rows (indexer -> top-k -> sparse MLA), processed in
 * query chunks so the fp32 score rows of one chunk live in the workspace.  Arguments are
 * those of the three calls above; idx_out [T,k] (nullable) receives the selected indices.
 * workspace must be at least dsa_prefill_workspace_bytes(T, L, H_I, H, k) bytes,
 * 256-byte aligned.
 * With H_I in {64, 128}, 11776 <= L <= 188416 and 2k <= 5888 the scores do not make a round
 * trip through memory: each row's threshold comes from the scores of every 32nd key (every
 * ceil(L/4096)-th beyond L = 131072), the indexer keeps only the (key, position) pairs at
 * or above it, and an exact select over those gives the row's top-k; a row whose pairs
 * cannot decide it (fewer than k, more than 5888, or more than 256 tied at the k-th score)
 * is scored in full and selected by the exact top-k.  The indices are the same as the two-pass path's.  DSA_PREFILL_UNFUSED=1 in
 * the environment (read at each call) keeps the two-pass path for every shape. */
dsa_status_t dsa_prefill(const uint8_t* q8, const float* q_scale, const float* w,
                         const uint8_t* k8, const float* k_scale, const uint16_t* q,
                         const uint16_t* kv, int T, int L, int H_I, int H, int k, int q_pos0,
                         float score_scale, float sm_scale, uint16_t* out, float* lse,
                         int32_t* idx_out, void* workspace, size_t workspace_bytes,
                         dsa_stream_t stream);
size_t dsa_prefill_workspace_bytes(int T, int L, int H_I, int H, int k);

/* Query rows per chunk that dsa_prefill uses for (T, L): chunk c covers rows
 * [c * rows, min(T, (c + 1) * rows)), and within a chunk the result is exactly that of
 * dsa_index_scores (write_masked = 0, rows that see more than k tokens only) ->
 * dsa_topk -> dsa_sparse_mla on that chunk.  Returns 0 for invalid sizes. */
int dsa_prefill_chunk_rows(int T, int L);

/* Prefill of a packed batch of B sequences ([gxzdkb-dsa] 致命问题：平方级复杂度拖垮效率:
 * the prefill of many rollouts at once), fresh or continuing an existing cache.
 * Sequence b owns query rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) of q8, q_scale, w, q, out,
 * lse and idx_out, and key rows [cu_seqlens_k[b], cu_seqlens_k[b+1]) of k8, k_scale, kv.
 * With T_b and L_b those counts, its queries are its last T_b tokens: query row t of it sits
 * at position L_b - T_b + t of that sequence and sees that sequence's keys 0 .. L_b - T_b + t
 * only (T_b = L_b is a fresh prefill; T_b < L_b prefills a chunk against a cache of
 * L_b - T_b tokens).  Each sequence is computed exactly as dsa_prefill with q_pos0 =
 * L_b - T_b on its own rows; idx_out (nullable) holds positions within the sequence.
 *   cu_seqlens_q, cu_seqlens_k  HOST int64 [B+1], each starting at 0, with
 *                               0 <= T_b <= L_b for every b (they size the launches).
 * Other tensors and sizes as dsa_prefill.  workspace: at least
 * dsa_prefill_varlen_workspace_bytes(...) bytes (the largest sequence's prefill workspace),
 * 256-byte aligned; shared by the sequences in turn.  B = 0 or no query rows is a no-op;
 * malformed cu_seqlens give DSA_ERR_INVALID_ARGUMENT. */
dsa_status_t dsa_prefill_varlen(int B, const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_k,
                                const uint8_t* q8, const float* q_scale, const float* w,
                                const uint8_t* k8, const float* k_scale, const uint16_t* q,
                                const uint16_t* kv, int H_I, int H, int k, float score_scale,
                                float sm_scale, uint16_t* out, float* lse, int32_t* idx_out,
                                void* workspace, size_t workspace_bytes, dsa_stream_t stream);
/* 0 for malformed cu_seqlens or when no sequence has query rows. */
size_t dsa_prefill_varlen_workspace_bytes(int B, const int64_t* cu_seqlens_q,
                                          const int64_t* cu_seqlens_k, int H_I, int H, int k);

/* Dense causal attention of the (frozen) main model, the warm-up target's source
 * ([yufo-notes] §四 第一阶段 Warm-up): for row t (position p_t) and head h,
 *   l[t,h,s] = sm_scale * <q[t,h,0:576], kv[s,0:576]>  for s <= p_t,
 * dsa_attention_lse:          lse[t,h] = log sum_s exp l[t,h,s]          (lse [T,H] f32);
 * dsa_attention_distribution: P[t,s] = (1/H) sum_h exp(l[t,h,s] - lse[t,h]) for s <= p_t,
 *   the head-averaged attention distribution (rows of P at stride ld >= L; entries s > p_t
 *   are not written).  q [T,H,576] bf16, kv [L,576] bf16, H <= 128; products exact in
 *   fp32, fp32 accumulation and statistics. */
dsa_status_t dsa_attention_lse(const uint16_t* q, const uint16_t* kv, int T, int L, int H,
                               int q_pos0, float sm_scale, float* lse, dsa_stream_t stream);
dsa_status_t dsa_attention_distribution(const uint16_t* q, const uint16_t* kv, const float* lse,
                                        int T, int L, int H, int q_pos0, float sm_scale,
                                        float* P, int64_t ld, dsa_stream_t stream);

/* Indexer warm-up step ([yufo-notes] §四 第一阶段 Warm-up): the KL divergence from the
 * dense distribution P (above) to the indexer's softmax Q[t,s] = softmax_{s <= p_t} I[t,s]
 * (I = dsa_index_scores), and its gradient.  With x[t,h,s] = <QI[t,h], KI[s]> for the
 * dequantised vectors QI = q_scale * q8, KI = k_scale * k8, and G = Q - P:
 *   kl[t]      = sum_s P log(P / Q)                                  kl [T] f32
 *   dw[t,h]    = score_scale * sum_s G max(x, 0)                     dw [T,H_I] f32
 *   dq[t,h,:]  = score_scale * w[t,h] sum_s G [x > 0] KI[s,:]        dq [T,H_I,128] f32
 *   dk[s,:]    = score_scale * sum_t sum_h G w[t,h] [x > 0] QI[t,h,:] dk [L,128] f32
 * i.e. the gradients with respect to QI, KI and w (the fp8 rounding is treated as the
 * identity); dk rows no query sees are 0.  lse_teacher [T,H] and lse_index [T] (both
 * nullable) receive the teacher lse and log sum_s exp I.  The gradient contractions run on
 * bf16 MFMA (G rounded to bf16, fp32 accumulation).  H_I in {16,32,64,128}, H <= 128,
 * T * H_I < 2^31 (DSA_ERR_UNSUPPORTED otherwise); T = 0 only zeroes dk.
 * Other arguments as dsa_prefill; workspace at least dsa_indexer_warmup_workspace_bytes
 * bytes, 256-byte aligned. */
dsa_status_t dsa_indexer_warmup(const uint8_t* q8, const float* q_scale, const float* w,
                                const uint8_t* k8, const float* k_scale, const uint16_t* q,
                                const uint16_t* kv, int T, int L, int H_I, int H, int q_pos0,
                                float score_scale, float sm_scale, float* kl, float* dq,
                                float* dw, float* dk, float* lse_teacher, float* lse_index,
                                void* workspace, size_t workspace_bytes, dsa_stream_t stream);
size_t dsa_indexer_warmup_workspace_bytes(int T, int L, int H_I, int H);

/* One decode step for B sequences ([gxzdkb-dsa] 原始 Attention 的计算逻辑: the new token's
 * cache entries are appended before attending).  Sequence b owns the packed cache rows
 * [seq_start[b], seq_start[b+1]) of k8_cache [N,128], k_scale_cache [N] and kv_cache
 * [N,576], N = total_tokens; its one query sits at position L_b - 1 = seq_start[b+1] -
 * seq_start[b] - 1 and sees its whole cache.
 *   seq_start  DEVICE int64 [B+1], non-decreasing, seq_start[0] = 0, seq_start[B] = N,
 *              every length in [1, max_len] (not checked: the host never reads it; a
 *              sequence longer than max_len selects nothing: out 0 and lse -inf);
 *   q8 [B,H_I,128]; q_scale, w [B,H_I]; q [B,H,576]; out [B,H,512]; lse [B,H] or NULL;
 *   idx_out [B,k] or NULL (positions within the sequence, ascending, -1 padded).
 * workspace >= dsa_decode_workspace_bytes(B, max_len, total_tokens, H_I, H, k) bytes. */
dsa_status_t dsa_decode(int B, const int64_t* seq_start, int max_len, int64_t total_tokens,
                        const uint8_t* q8, const float* q_scale, const float* w,
                        const uint8_t* k8_cache, const float* k_scale_cache,
                        const uint16_t* q, const uint16_t* kv_cache, int H_I, int H, int k,
                        float score_scale, float sm_scale, uint16_t* out, float* lse,
                        int32_t* idx_out, void* workspace, size_t workspace_bytes,
                        dsa_stream_t stream);
size_t dsa_decode_workspace_bytes(int B, int max_len, int64_t total_tokens, int H_I, int H,
                                  int k);

/* dsa_decode for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same arguments without a
 * workspace, the same kernels and results.  Its workspace is a fixed array of
 * DSA_DECODE_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held by each GPU the
 * library runs on until the process ends; the call allocates nothing and needs no prior
 * set-up (the array's device address is looked up on the first call on a device).
 *   - A call whose workspace, dsa_decode_workspace_bytes(B, max_len, total_tokens, H_I, H, k),
 *     exceeds the array returns DSA_ERR_WORKSPACE_TOO_SMALL and launches nothing (128 MiB
 *     covers, e.g., 64 sequences of up to 131,072 tokens and 4.2M cached tokens at k = 2048,
 *     H = 128).  Other errors as dsa_decode.
 *   - Every call on a GPU uses that GPU's one array, which keeps the last call's contents:
 *     calls that overlap on one GPU (other streams, other threads) race and must be
 *     serialised by the caller.  Nothing in the array needs clearing between calls. */
#define DSA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
dsa_status_t dsa_decode_noalloc(int B, const int64_t* seq_start, int max_len,
                                int64_t total_tokens, const uint8_t* q8, const float* q_scale,
                                const float* w, const uint8_t* k8_cache,
                                const float* k_scale_cache, const uint16_t* q,
                                const uint16_t* kv_cache, int H_I, int H, int k,
                                float score_scale, float sm_scale, uint16_t* out, float* lse,
                                int32_t* idx_out, dsa_stream_t stream);
size_t dsa_decode_noalloc_scratch_bytes(void);

/* fp8 preparation of the indexer's inputs, the step upstream of dsa_index_scores (the
 * indexer runs in FP8: [gxzdkb-dsa] 秘密武器：DSA, [csdn-workflow] §3 两大核心组件).  Each
 * 128-wide vector i of x (fp32, or bf16 bits when x_is_bf16 = 1) becomes
 *   scale[i] = amax_i / 448 (fp32; 1 for an all-zero vector) and
 *   q8[i,d]  = the e4m3fn value nearest to clamp(x[i,d] / scale[i], -448, 448), the quotient
 *              rounded to fp32, ties to even, the sign of zero kept,
 * the format dsa_index_scores reads (q8 with q_scale, k8 with k_scale).
 *   x [n,128] 16-byte aligned; q8 [n,128] 8-byte aligned; scale [n] fp32.  x must be finite.
 * n = 0 is a no-op. */
dsa_status_t dsa_quantize_fp8(const void* x, int x_is_bf16, int64_t n, uint8_t* q8,
                              float* scale, dsa_stream_t stream);

/* Decode cache append ([gxzdkb-dsa] 原始 Attention 的计算逻辑: the new token's entries join
 * the cache before the step attends), the step before dsa_decode: for each sequence b, row
 * r = seq_start[b+1] - 1 of the packed caches receives the new token,
 *   k8_cache[r,:], k_scale_cache[r] = the quantisation of k_new[b,:] (as dsa_quantize_fp8),
 *   kv_cache[r,:] = kv_new[b,:].
 *   seq_start DEVICE int64 [B+1] as in dsa_decode, already counting the new tokens (a
 *   sequence with no row is skipped); k_new [B,128] fp32, or bf16 bits when k_is_bf16 = 1,
 *   16-byte aligned; kv_new [B,576] and kv_cache 16-byte aligned; k8_cache 8-byte aligned.
 * B = 0 is a no-op; B <= 65535. */
dsa_status_t dsa_decode_append(int B, const int64_t* seq_start, const void* k_new, int k_is_bf16,
                               const uint16_t* kv_new, uint8_t* k8_cache, float* k_scale_cache,
                               uint16_t* kv_cache, dsa_stream_t stream);

/* Alternative index rules that feed dsa_sparse_mla ([gxzdkb-dsa] 秘密武器：DSA: DSA
 * generalises sliding-window attention; [oilbeater-dsa] Sparse Attention: a local window,
 * alone or joined by globally chosen tokens).  Row t sits at p = q_pos0 + t (q_pos0 + T <= L).
 * dsa_window_indices: idx [T, window] = max(0, p-window+1) .. p ascending, then -1.
 * dsa_local_selected_indices: out [T, window + k] = the ascending union of that window and
 *   the valid entries of sel [T, k] (positions 0 <= s <= p, in ascending order as dsa_topk
 *   writes them; -1 entries anywhere are skipped), then -1.
 * Either list is the idx argument of dsa_sparse_mla with k = its width. */
dsa_status_t dsa_window_indices(int T, int L, int q_pos0, int window, int32_t* idx,
                                dsa_stream_t stream);
dsa_status_t dsa_local_selected_indices(const int32_t* sel, int T, int L, int q_pos0, int k,
                                        int window, int32_t* out, dsa_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
