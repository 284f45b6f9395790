/*
 * oracle.h -- plain CPU oracle for the DeepSeek Sparse Attention (DSA) hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the package's smoke check and the benchmark's
 * CPU-baseline leg are the only callers.  It shares no code, header, table or constant
 * with the HIP library: its own e4m3fn/bf16 decoders, its own loops, fp64 arithmetic.
 *
 * Pages cited (by title; section names as printed on each page):
 *   [csdn-workflow] 《DeepSeek-V3.2-Exp模型优势与 DSA 工作原理,token降价性能不减的背后》
 *                   (agent.csdn.net) -- §2 风险边界明确, §3 两大核心组件, §4 四步工作流程.
 *   [devpress-dsa]  《狂降75%！大模型DeepSeek-V3.2 API杀疯了：性能零衰减的秘密，藏在DSA这两大
 *                   “黑科技”里》 (devpress.csdn.net) -- §二 两大核心武器, §三 四步工作流.
 *   [gxzdkb-dsa]    gxzdkb.com explainer of DSA -- sections 原始 Attention 的计算逻辑,
 *                   秘密武器：DSA, 实测效果.
 *   [yufo-notes]    ele-yufo.com notes "DeepSeek V3.2-Exp" -- §三 两步跑通稀疏路由,
 *                   §四 训练的两步走冷启动 (第一阶段 Warm-up).
 *   [oilbeater-dsa] oilbeater.com "DeepSeek Sparse Attention" -- section Sparse Attention.
 *
 * Conventions shared by every function:
 *   fp8 operands are OCP e4m3fn bytes; bf16 operands are raw uint16 bits.
 *   Query row t sits at absolute position p_t = q_pos0 + t and sees keys s <= p_t
 *   (the causal mask of [csdn-workflow] §4 步骤二; "update the cache first, then
 *   compute" in [gxzdkb-dsa] makes the query see itself).
 *   `rows` lists which query rows to compute (n_rows of them); outputs are packed
 *   in that order.  All functions return 0, or -1 on invalid input.
 */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* Value of one e4m3fn code (NaN for 0x7F / 0xFF) and of one bf16 bit pattern. */
double ora_e4m3fn_value(uint8_t code);
double ora_bf16_value(uint16_t bits);

/* Lightning-indexer scores, [csdn-workflow] §4 步骤二 and [devpress-dsa] §三 第二步:
 *   D[t,h,s]    = sum_d q8[t,h,d] * k8[s,d]          (exact, int64 at scale 2^18)
 *   score[t,s]  = ks[s] * sum_h (w[t,h]*qs[t,h]*c) * max(D[t,h,s], 0)   for s <= p_t
 *               = -inf                                                  for s >  p_t
 *   bound[t,s]  = ks[s] * sum_h |w*qs*c| * sum_d |q8*k8|   (conditioning bound, nullable)
 * q8[T,H_I,128], qs[T,H_I], w[T,H_I], k8[L,128], ks[L]; scores/bound [n_rows, L]. */
int ora_index_scores(const uint8_t* q8, const float* qs, const float* w,
                     const uint8_t* k8, const float* ks, int64_t L, int H_I,
                     int64_t q_pos0, double c, const int64_t* rows, int64_t n_rows,
                     double* scores, double* bound);

/* Top-k, [csdn-workflow] §4 步骤三: the k visible positions with the largest score,
 * ties to the lower position, -0 == +0; all n visible positions when n <= k.
 * scores [n_rows, ld] (entries s < n_vis[r] are read), idx [n_rows, k] int32,
 * ascending positions then -1 padding.  Two independent selectors:
 *   _sort   : full sort of (score desc, position asc), keep the first k;
 *   _select : k-th largest value by quickselect, then a position-ordered sweep. */
int ora_topk_sort(const double* scores, int64_t ld, int64_t n_rows, const int64_t* n_vis,
                  int k, int32_t* idx);
int ora_topk_select(const double* scores, int64_t ld, int64_t n_rows, const int64_t* n_vis,
                    int k, int32_t* idx);

/* Sparse MLA, [csdn-workflow] §4 步骤四 and [devpress-dsa] §三 第四步: for each row t
 * and head h, logits l_j = sm_scale * <q[t,h,0:576], kv[I_j,0:576]> over the selected
 * rows I_j = idx[t,j] (-1 entries skipped), out = softmax(l) . kv[I,0:512],
 * lse = log sum exp l.  A row with no valid index gives out = 0, lse = -inf.
 * q[T,H,576] bf16, kv[L,576] bf16, idx[T,k]; out [n_rows,H,512], lse [n_rows,H]. */
int ora_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int64_t L,
                   int H, int k, double sm_scale, const int64_t* rows, int64_t n_rows,
                   double* out, double* lse);

/* Dense causal MLA over every s <= p_t, no index list: the full attention that DSA
 * equals when a query sees at most k tokens ([csdn-workflow] §2 风险边界明确, §4 步骤三). */
int ora_dense_mla(const uint16_t* q, const uint16_t* kv, int64_t L, int H, int64_t q_pos0,
                  double sm_scale, const int64_t* rows, int64_t n_rows, double* out,
                  double* lse);

/* Threads the OpenMP loops use. */
/* fp8 preparation of the indexer inputs (the step upstream of the lightning indexer, which
 * runs in FP8: [gxzdkb-dsa] 秘密武器：DSA, [csdn-workflow] §3 两大核心组件).  Per 128-wide
 * vector: scale = amax / 448 in fp32 (1 for an all-zero vector); code d = the e4m3fn value
 * nearest to clamp(x[d] / scale, -448, 448), the quotient rounded to fp32, ties to the even
 * code.  x[n,128] fp32, or bf16 bits when x_bf16; q8[n,128]; scale[n]. */
int ora_quantize_e4m3(const void* x, int x_bf16, int64_t n, uint8_t* q8, float* scale);

/* Decode cache append ([gxzdkb-dsa] 原始 Attention 的计算逻辑: the new token's entries join
 * the cache before the step attends): row r = seq_start[b+1] - 1 of the packed caches gets
 * k8_cache[r], k_scale_cache[r] = the quantisation of k_new[b] (as above) and
 * kv_cache[r] = kv_new[b] (576 bf16).  Every sequence must hold at least one row. */
int ora_decode_append(int B, const int64_t* seq_start, const void* k_new, int k_bf16,
                      const uint16_t* kv_new, uint8_t* k8_cache, float* k_scale_cache,
                      uint16_t* kv_cache);

/* Alternative index rules feeding the sparse MLA ([gxzdkb-dsa] 秘密武器：DSA: DSA generalises
 * sliding-window attention; [oilbeater-dsa] oilbeater.com "DeepSeek Sparse Attention", section
 * Sparse Attention: a local sliding window, alone or joined by globally chosen tokens).
 * Window: row t (position p = q_pos0 + t) keeps the W positions max(0, p-W+1) .. p, ascending,
 * -1 padded: idx [T, W].  Local + selected: the ascending union of that window and the valid
 * entries (0 <= s <= p) of sel[t, 0:k], -1 padded: out [T, W + k]. */
int ora_window_indices(int64_t T, int64_t q_pos0, int W, int32_t* idx);
int ora_local_selected(const int32_t* sel, int64_t T, int k, int64_t q_pos0, int W, int32_t* out);

/* Indexer warm-up loss and its gradient ([yufo-notes] §四 训练的两步走冷启动, 第一阶段
 * Warm-up: the frozen main model's dense attention gives each token's weight distribution
 * as the target, and the indexer alone is trained to fit it with a KL divergence).  For a
 * query at position p (n = p + 1 visible keys):
 *   teacher  l_h[s] = sm_scale <q[h,:], kv[s,:]> (576 dims),  lse_t[h] = log sum_s exp l_h[s],
 *            P[s]   = (1/H) sum_h exp(l_h[s] - lse_t[h])        (head-averaged, sums to 1)
 *   student  x_h[s] = <QI[h,:], KI[s,:]>,  I[s] = c sum_h w[h] max(x_h[s], 0),
 *            lse_i  = log sum_s exp I[s],  Q[s] = exp(I[s] - lse_i)
 *   loss     kl = sum_s P[s] (log P[s] - log Q[s])   (terms with P[s] = 0 contribute 0)
 *   gradient G[s] = dkl/dI[s] = Q[s] - P[s];
 *            dw[h]     = c sum_s G[s] max(x_h[s], 0)
 *            dq[h,d]   = c w[h] sum_s G[s] [x_h[s] > 0] KI[s,d]
 *            dk[s,d]  += c G[s] sum_h w[h] [x_h[s] > 0] QI[h,d]     (summed over the rows given)
 * Inputs are real-valued (fp64): QI [n_rows,H_I,128], w [n_rows,H_I], q [n_rows,H,576],
 * pos [n_rows] (each < L), KI [L,128], kv [L,576].  Outputs per row: kl, lse_t [.,H],
 * lse_i, dq [.,H_I,128], dw [.,H_I]; P and G [n_rows, L] (entries s > p are 0) nullable;
 * dk [L,128] nullable.  Magnitude bounds (all nullable), with A[s] = Q[s] + P[s] >= |G[s]|
 * standing for G: kl_bnd = sum_s P (|log P| + |log Q|); dw_bnd[h] = c sum_s A |x_h|;
 * dq_bnd / dk_bnd = the sums of dq / dk with G replaced by A and every other factor by its
 * absolute value; dq_amb / dk_amb = those sums taken only over the (h, s) whose
 * |x_h[s]| <= 2^-16 sum_d |QI[h,d] KI[s,d]| (where a rounded evaluation of x may take the
 * other side of the ReLU). */
int ora_warmup(const double* QI, const double* w, const double* q, const int64_t* pos,
               int64_t n_rows, const double* KI, const double* kv, int64_t L, int H_I, int H,
               double c, double sm_scale, double* kl, double* lse_t, double* lse_i, double* dq,
               double* dw, double* P, double* G, double* dk, double* kl_bnd, double* dw_bnd,
               double* dq_bnd, double* dq_amb, double* dk_bnd, double* dk_amb);

int ora_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
