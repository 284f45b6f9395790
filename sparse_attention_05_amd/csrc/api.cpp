// api.cpp -- the C ABI of libdsa.so (declared in include/dsa.h).
//
// Every entry point validates all of its arguments before touching the HIP runtime, so an
// invalid call returns its status having launched nothing.  Valid calls only enqueue
// kernels on the caller's stream.
#include "dsa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "kernels.h"

namespace {

// ---- host launch log: DSA_LOG=1 in the environment prints one line per entry-point call
// (name, sizes, status) to stderr; read once per process
bool log_on()
{
    static const bool on = [] {
        const char* v = std::getenv("DSA_LOG");
        return v && v[0] && !(v[0] == '0' && v[1] == 0);
    }();
    return on;
}

__attribute__((format(printf, 2, 3))) dsa_status_t logged(dsa_status_t st, const char* fmt, ...)
{
    if (log_on()) {
        char buf[512];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof buf, fmt, ap);
        va_end(ap);
        std::fprintf(stderr, "[dsa] %s -> %s\n", buf, dsa_status_string(st));
    }
    return st;
}

constexpr int64_t kMaxElems = int64_t(1) << 40;   // T * max(L, k) bound
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

hipStream_t as_hip(dsa_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

dsa_status_t from_hip(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool heads_ok(int H) { return H >= 1 && H <= 128; }
bool k_ok(int k) { return k >= 1 && k <= 8192; }
// latent-cache rows one attention call may address: the sparse MLA finds a gathered row by a
// byte offset (1152 bytes per row) below 2^31 within the call's (or sequence's) cache
constexpr int64_t kMaxCacheRows = 0x7FFFFFFFll / 1152;   // 1,864,135
bool cache_ok(int64_t L) { return L <= kMaxCacheRows; }

// rows of the causal triangle: (T, L, q_pos0) consistency shared by the prefill calls
dsa_status_t check_rows(int T, int L, int q_pos0)
{
    if (T < 0 || L <= 0 || q_pos0 < 0) return DSA_ERR_INVALID_ARGUMENT;
    if ((int64_t)q_pos0 + T > L) return DSA_ERR_INVALID_ARGUMENT;
    return DSA_OK;
}

// ---- prefill chunking: rows per chunk so one chunk's fp32 score rows stay bounded
constexpr int64_t kChunkScoreBytes = int64_t(2048) << 20;   // 2 GiB

int prefill_chunk_rows(int T, int L)
{
    int64_t rows = kChunkScoreBytes / (int64_t(L) * 4);
    rows = std::max<int64_t>(64, rows / 64 * 64);
    return (int)std::min<int64_t>(std::max(T, 1), rows);
}

// Workspace of one prefill call: a chunk's fp32 score rows (also the home of the fused
// selection's key sample and candidate arrays, which never need more room), its indices and
// the fused selection's per-row threshold, candidate count and fallback flag.
struct PrefillWs {
    int chunk;
    size_t scores_off, idx_off, sel_off, total;
};

PrefillWs prefill_ws(int T, int L, int k)
{
    PrefillWs w;
    w.chunk = prefill_chunk_rows(T, L);
    w.scores_off = 0;
    w.idx_off = align_up(size_t(w.chunk) * size_t(L) * 4);
    w.sel_off = w.idx_off + align_up(size_t(w.chunk) * size_t(k) * 4);
    w.total = w.sel_off + 3 * align_up(size_t(w.chunk) * 4);
    return w;
}

// The fused selection applies (candidates instead of a score round trip through memory);
// DSA_PREFILL_UNFUSED=1, read at every call, keeps the two-pass path.
bool prefill_fused(int L, int H_I, int k)
{
    const char* v = std::getenv("DSA_PREFILL_UNFUSED");
    const bool off = v && v[0] == '1';
    return !off && dsa::indexer_fused_supports(H_I) && dsa::fused_select_supports(L, k);
}

// ---- decode workspace: packed scores, indices, split-K partials
int decode_splits(int k) { return std::min(8, std::max(1, (k + 511) / 512)); }

struct DecodeWs {
    int splits;
    size_t scores_off, idx_off, po_off, pl_off, tk_off, tk_bytes, total;
};

DecodeWs decode_ws(int B, int max_len, int64_t N, int H, int k)
{
    DecodeWs w;
    w.splits = decode_splits(k);
    w.scores_off = 0;
    w.idx_off = align_up(size_t(N) * 4);
    w.po_off = w.idx_off + align_up(size_t(B) * size_t(k) * 4);
    w.pl_off = w.po_off + align_up(size_t(B) * w.splits * H * 512 * 4);
    w.tk_off = w.pl_off + align_up(size_t(B) * w.splits * H * 4);
    w.tk_bytes = dsa::topk_decode_workspace_bytes(B, max_len);
    w.total = w.tk_off + align_up(w.tk_bytes);
    return w;
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status_t status)
{
    switch (status) {
        case DSA_OK: return "DSA_OK";
        case DSA_ERR_INVALID_ARGUMENT: return "DSA_ERR_INVALID_ARGUMENT";
        case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
        case DSA_ERR_WORKSPACE_TOO_SMALL: return "DSA_ERR_WORKSPACE_TOO_SMALL";
        case DSA_ERR_HIP: return "DSA_ERR_HIP";
    }
    return "DSA_ERR_UNKNOWN";
}

int dsa_version(void) { return 105; }

static dsa_status_t dsa_index_scores_impl(const uint8_t* q8, const float* q_scale, const float* w,
                                          const uint8_t* k8, const float* k_scale, int T, int L,
                                          int H_I, int q_pos0, float score_scale, float* scores,
                                          int64_t ld_scores, int write_masked, dsa_stream_t stream)
{
    if (dsa_status_t st = check_rows(T, L, q_pos0)) return st;
    if (T > 0 && (!q8 || !q_scale || !w || !k8 || !k_scale || !scores))
        return DSA_ERR_INVALID_ARGUMENT;
    if (ld_scores < L) return DSA_ERR_INVALID_ARGUMENT;
    if (!(score_scale > 0.f)) return DSA_ERR_INVALID_ARGUMENT;
    if (!dsa::indexer_supports(H_I)) return DSA_ERR_UNSUPPORTED;
    if ((int64_t)T * ld_scores > kMaxElems) return DSA_ERR_UNSUPPORTED;
    if (!aligned(q8, 16) || !aligned(k8, 16)) return DSA_ERR_INVALID_ARGUMENT;
    if (T == 0) return DSA_OK;
    hipStream_t s = as_hip(stream);
    hipError_t e = dsa::launch_indexer_prefill(q8, q_scale, w, k8, k_scale, T, L, H_I, q_pos0,
                                               score_scale, scores, ld_scores, s);
    if (e == hipSuccess && write_masked)
        e = dsa::launch_mask_fill(T, L, q_pos0, scores, ld_scores, s);
    return from_hip(e);
}

size_t dsa_topk_workspace_bytes(int, int, int) { return 0; }

static dsa_status_t dsa_topk_impl(const float* scores, int64_t ld_scores, int T, int L, int q_pos0,
                                  int k, int32_t* idx, dsa_stream_t stream)
{
    if (dsa_status_t st = check_rows(T, L, q_pos0)) return st;
    if (T > 0 && (!scores || !idx)) return DSA_ERR_INVALID_ARGUMENT;
    if (ld_scores < L) return DSA_ERR_INVALID_ARGUMENT;
    if (!k_ok(k)) return k < 1 ? DSA_ERR_INVALID_ARGUMENT : DSA_ERR_UNSUPPORTED;
    if ((int64_t)T * std::max<int64_t>(ld_scores, k) > kMaxElems) return DSA_ERR_UNSUPPORTED;
    if (T == 0) return DSA_OK;
    return from_hip(dsa::launch_topk_prefill(scores, ld_scores, T, L, q_pos0, k, idx,
                                             as_hip(stream)));
}

static dsa_status_t dsa_sparse_mla_impl(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                                        int T, int L, int H, int k, float sm_scale, uint16_t* out,
                                        float* lse, dsa_stream_t stream)
{
    if (T < 0 || L <= 0 || k < 1) return DSA_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!q || !kv || !idx || !out)) return DSA_ERR_INVALID_ARGUMENT;
    if (!heads_ok(H)) return H < 1 ? DSA_ERR_INVALID_ARGUMENT : DSA_ERR_UNSUPPORTED;
    if (!(sm_scale > 0.f)) return DSA_ERR_INVALID_ARGUMENT;
    if ((int64_t)T * std::max(L, k) > kMaxElems || !cache_ok(L)) return DSA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 4)) return DSA_ERR_INVALID_ARGUMENT;
    if (T == 0) return DSA_OK;
    return from_hip(dsa::launch_sparse_mla(q, kv, idx, nullptr, T, L, H, k, sm_scale, 1, out,
                                           lse, nullptr, nullptr, -1, as_hip(stream)));
}

int dsa_prefill_chunk_rows(int T, int L)
{
    if (T <= 0 || L <= 0) return 0;
    return prefill_chunk_rows(T, L);
}

size_t dsa_prefill_workspace_bytes(int T, int L, int H_I, int H, int k)
{
    (void)H_I;
    (void)H;
    if (T <= 0 || L <= 0 || k < 1) return 0;
    return prefill_ws(T, L, k).total;
}

// One prefill call after validation: query chunks of ws.chunk rows, each indexer (rows that
// see more than k tokens) -> top-k -> sparse MLA.  Pointers are at the call's first row / key.
static dsa_status_t prefill_run(const uint8_t* q8, const float* q_scale, const float* w,
                         const uint8_t* k8, const float* k_scale, const uint16_t* q,
                                const uint16_t* kv, int T, int L, int H_I, int H, int k,
                                int q_pos0, float score_scale, float sm_scale, uint16_t* out,
                                float* lse, int32_t* idx_out, void* workspace, hipStream_t s)
{
    const PrefillWs ws = prefill_ws(T, L, k);
    uint8_t* base = static_cast<uint8_t*>(workspace);
    float* scores = reinterpret_cast<float*>(base + ws.scores_off);
    int32_t* idx_ws = reinterpret_cast<int32_t*>(base + ws.idx_off);
    uint32_t* tau = reinterpret_cast<uint32_t*>(base + ws.sel_off);
    int* fill = reinterpret_cast<int*>(base + ws.sel_off + align_up(size_t(ws.chunk) * 4));
    int* fb = reinterpret_cast<int*>(base + ws.sel_off + 2 * align_up(size_t(ws.chunk) * 4));
    const bool fused = prefill_fused(L, H_I, k);
    // first row that sees more than k tokens (earlier rows select all without scores)
    const int t_sel = std::max(0, k - q_pos0);
    for (int r0 = 0; r0 < T; r0 += ws.chunk) {
        const int rows = std::min(ws.chunk, T - r0);
        const int qp = q_pos0 + r0;
        int32_t* idx = idx_out ? idx_out + (int64_t)r0 * k : idx_ws;
        const int s0 = std::max(r0, t_sel);           // rows needing scores in this chunk
        const int off = std::min(rows, s0 - r0);
        const int nsel = rows - off;
        const uint8_t* q8s = q8 + (int64_t)s0 * H_I * 128;
        const float* qss = q_scale + (int64_t)s0 * H_I;
        const float* ws_ = w + (int64_t)s0 * H_I;
        hipError_t e = hipSuccess;
        if (fused) {
            // threshold sample -> candidates -> resolve; rows the candidates cannot decide
            // are scored and selected exactly (their launches skip every other row)
            dsa::IdxExtra ex;
            ex.kstride = dsa::fused_sample_stride(L);
            ex.ksplit = 2048;                 // sampled keys per workgroup (of at most 4096)
            const int nsamp = dsa::fused_sample_count(L);
            if (nsel > 0)
                e = dsa::launch_indexer_prefill(q8s, qss, ws_, k8, k_scale, nsel, L, H_I,
                                                q_pos0 + s0, score_scale, scores, nsamp, s, ex);
            if (e == hipSuccess)
                e = dsa::launch_topk_threshold(scores, nsamp, nsel, L, q_pos0 + s0, k, tau,
                                               fill, fb, s);
            ex = dsa::IdxExtra{};
            ex.tau = tau;
            ex.fill = fill;
            ex.cand = reinterpret_cast<uint2*>(scores);
            ex.capr = dsa::fused_cand_cap();
            if (e == hipSuccess && nsel > 0)
                e = dsa::launch_indexer_candidates(q8s, qss, ws_, k8, k_scale, nsel, L, H_I,
                                                   q_pos0 + s0, score_scale, ex, s);
            if (e == hipSuccess)
                e = dsa::launch_topk_resolve(ex.cand, ex.capr, fill, rows, L, qp, k, off, idx,
                                             fb, s);
            ex = dsa::IdxExtra{};
            ex.only = fb;
            if (e == hipSuccess && nsel > 0)
                e = dsa::launch_indexer_prefill(q8s, qss, ws_, k8, k_scale, nsel, L, H_I,
                                                q_pos0 + s0, score_scale,
                                                scores + (int64_t)off * L, L, s, ex);
            if (e == hipSuccess)
                e = dsa::launch_topk_prefill_only(scores, L, rows, L, qp, k, idx, fb, off, s);
        } else {
            if (nsel > 0)
                e = dsa::launch_indexer_prefill(q8s, qss, ws_, k8, k_scale, nsel, L, H_I,
                                                q_pos0 + s0, score_scale,
                                                scores + (int64_t)off * L, L, s);
            if (e == hipSuccess) e = dsa::launch_topk_prefill(scores, L, rows, L, qp, k, idx, s);
        }
        if (e == hipSuccess)
            e = dsa::launch_sparse_mla(q + (int64_t)r0 * H * 576, kv, idx, nullptr, rows, L, H,
                                       k, sm_scale, 1, out + (int64_t)r0 * H * 512,
                                       lse ? lse + (int64_t)r0 * H : nullptr, nullptr, nullptr,
                                       qp, s);
        if (e != hipSuccess) return DSA_ERR_HIP;
    }
    return DSA_OK;
}

static dsa_status_t dsa_prefill_impl(const uint8_t* q8, const float* q_scale, const float* w,
                                     const uint8_t* k8, const float* k_scale, const uint16_t* q,
                                     const uint16_t* kv, int T, int L, int H_I, int H, int k,
                                     int q_pos0, float score_scale, float sm_scale, uint16_t* out,
                                     float* lse, int32_t* idx_out, void* workspace,
                                     size_t workspace_bytes, dsa_stream_t stream)
{
    if (dsa_status_t st = check_rows(T, L, q_pos0)) return st;
    if (T > 0 && (!q8 || !q_scale || !w || !k8 || !k_scale || !q || !kv || !out))
        return DSA_ERR_INVALID_ARGUMENT;
    if (k < 1 || H < 1) return DSA_ERR_INVALID_ARGUMENT;
    if (!(score_scale > 0.f) || !(sm_scale > 0.f)) return DSA_ERR_INVALID_ARGUMENT;
    if (!dsa::indexer_supports(H_I) || !heads_ok(H) || !k_ok(k)) return DSA_ERR_UNSUPPORTED;
    if ((int64_t)T * std::max(L, k) > kMaxElems || !cache_ok(L)) return DSA_ERR_UNSUPPORTED;
    if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(q, 16) || !aligned(kv, 16) ||
        !aligned(out, 4))
        return DSA_ERR_INVALID_ARGUMENT;
    if (T == 0) return DSA_OK;
    if (!workspace || workspace_bytes < prefill_ws(T, L, k).total) return DSA_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(workspace, kAlign)) return DSA_ERR_INVALID_ARGUMENT;

    return prefill_run(q8, q_scale, w, k8, k_scale, q, kv, T, L, H_I, H, k, q_pos0, score_scale,
                       sm_scale, out, lse, idx_out, workspace, as_hip(stream));
}

// Validates a packed batch (cu_q[0] = cu_k[0] = 0, 0 <= T_b <= L_b, sizes within the
// single-call limits) and returns the largest per-sequence prefill workspace, or -1.
static int64_t varlen_ws(int B, const int64_t* cu_q, const int64_t* cu_k, int k)
{
    if (B < 0 || k < 1) return -1;
    if (B == 0) return 0;
    if (!cu_q || !cu_k || cu_q[0] != 0 || cu_k[0] != 0) return -1;
    size_t need = 0;
    for (int b = 0; b < B; ++b) {
        const int64_t T = cu_q[b + 1] - cu_q[b], L = cu_k[b + 1] - cu_k[b];
        if (T < 0 || L < T || L > INT32_MAX) return -1;
        if (T == 0) continue;
        if (T * std::max<int64_t>(L, k) > kMaxElems || !cache_ok(L)) return -1;
        need = std::max(need, prefill_ws((int)T, (int)L, k).total);
    }
    return (int64_t)need;
}

size_t dsa_prefill_varlen_workspace_bytes(int B, const int64_t* cu_seqlens_q,
                                          const int64_t* cu_seqlens_k, int H_I, int H, int k)
{
    (void)H_I;
    (void)H;
    const int64_t ws = varlen_ws(B, cu_seqlens_q, cu_seqlens_k, k);
    return ws < 0 ? 0 : (size_t)ws;
}

static dsa_status_t dsa_prefill_varlen_impl(int B, const int64_t* cu_seqlens_q,
                                            const int64_t* cu_seqlens_k, const uint8_t* q8,
                                            const float* q_scale, const float* w, const uint8_t* k8,
                                            const float* k_scale, const uint16_t* q,
                                            const uint16_t* kv, int H_I, int H, int k,
                                            float score_scale, float sm_scale, uint16_t* out,
                                            float* lse, int32_t* idx_out, void* workspace,
                                            size_t workspace_bytes, dsa_stream_t stream)
{
    if (k < 1 || H < 1) return DSA_ERR_INVALID_ARGUMENT;
    const int64_t need = varlen_ws(B, cu_seqlens_q, cu_seqlens_k, k);
    if (need < 0) return DSA_ERR_INVALID_ARGUMENT;
    if (!(score_scale > 0.f) || !(sm_scale > 0.f)) return DSA_ERR_INVALID_ARGUMENT;
    if (!dsa::indexer_supports(H_I) || !heads_ok(H) || !k_ok(k)) return DSA_ERR_UNSUPPORTED;
    if (B == 0 || cu_seqlens_q[B] == 0) return DSA_OK;   // no query rows
    if (!q8 || !q_scale || !w || !k8 || !k_scale || !q || !kv || !out)
        return DSA_ERR_INVALID_ARGUMENT;
    if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(q, 16) || !aligned(kv, 16) ||
        !aligned(out, 4))
        return DSA_ERR_INVALID_ARGUMENT;
    if (!workspace || workspace_bytes < (size_t)need) return DSA_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(workspace, kAlign)) return DSA_ERR_INVALID_ARGUMENT;

    hipStream_t s = as_hip(stream);
    for (int b = 0; b < B; ++b) {
        const int64_t qa = cu_seqlens_q[b], ka = cu_seqlens_k[b];
        const int T = (int)(cu_seqlens_q[b + 1] - qa), L = (int)(cu_seqlens_k[b + 1] - ka);
        if (T == 0) continue;
        // the sequence's queries are its last T tokens
        const dsa_status_t st = prefill_run(
            q8 + qa * H_I * 128, q_scale + qa * H_I, w + qa * H_I, k8 + ka * 128, k_scale + ka,
            q + qa * H * 576, kv + ka * 576, T, L, H_I, H, k, L - T, score_scale, sm_scale,
            out + qa * H * 512, lse ? lse + qa * H : nullptr, idx_out ? idx_out + qa * k : nullptr,
            workspace, s);
        if (st != DSA_OK) return st;
    }
    return DSA_OK;
}

// ---- indexer warm-up: query chunks with two fp32 [rows, L] buffers (P then G, and the
// indexer scores) and the chunk's teacher lse when the caller does not keep it
struct WarmupWs {
    int chunk;
    size_t pg_off, i_off, lse_off, dkp_off, total;
};

// + the key gradient's per-16-head-group partials [H_I/16][L][128]
static WarmupWs warmup_ws(int T, int L, int H_I, int H)
{
    WarmupWs w;
    w.chunk = prefill_chunk_rows(T, L);
    w.pg_off = 0;
    w.i_off = align_up(size_t(w.chunk) * size_t(L) * 4);
    w.lse_off = w.i_off + align_up(size_t(w.chunk) * size_t(L) * 4);
    w.dkp_off = w.lse_off + align_up(size_t(w.chunk) * size_t(H) * 4);
    w.total = w.dkp_off + align_up(size_t(std::max(H_I / 16, 1)) * size_t(L) * 128 * 4);
    return w;
}

static dsa_status_t check_teacher(const uint16_t* q, const uint16_t* kv, int T, int L, int H,
                                  int q_pos0, float sm_scale)
{
    if (dsa_status_t st = check_rows(T, L, q_pos0)) return st;
    if (T > 0 && (!q || !kv)) return DSA_ERR_INVALID_ARGUMENT;
    if (H < 1 || !(sm_scale > 0.f)) return DSA_ERR_INVALID_ARGUMENT;
    if (H > 128) return DSA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(kv, 16)) return DSA_ERR_INVALID_ARGUMENT;
    return DSA_OK;
}

static dsa_status_t dsa_attention_lse_impl(const uint16_t* q, const uint16_t* kv, int T, int L,
                                           int H, int q_pos0, float sm_scale, float* lse,
                                           dsa_stream_t stream)
{
    if (dsa_status_t st = check_teacher(q, kv, T, L, H, q_pos0, sm_scale)) return st;
    if (T == 0) return DSA_OK;
    if (!lse) return DSA_ERR_INVALID_ARGUMENT;
    return from_hip(dsa::launch_attention_lse(q, kv, T, H, q_pos0, sm_scale, lse, as_hip(stream)));
}

static dsa_status_t dsa_attention_distribution_impl(const uint16_t* q, const uint16_t* kv,
                                                    const float* lse, int T, int L, int H,
                                                    int q_pos0, float sm_scale, float* P,
                                                    int64_t ld, dsa_stream_t stream)
{
    if (dsa_status_t st = check_teacher(q, kv, T, L, H, q_pos0, sm_scale)) return st;
    if (ld < L) return DSA_ERR_INVALID_ARGUMENT;
    if ((int64_t)T * ld > kMaxElems) return DSA_ERR_UNSUPPORTED;
    if (T == 0) return DSA_OK;
    if (!lse || !P) return DSA_ERR_INVALID_ARGUMENT;
    return from_hip(dsa::launch_attention_dist(q, kv, lse, T, H, q_pos0, sm_scale, P, ld,
                                               as_hip(stream)));
}

size_t dsa_indexer_warmup_workspace_bytes(int T, int L, int H_I, int H)
{
    if (T <= 0 || L <= 0 || H < 1 || H_I < 1) return 0;
    return warmup_ws(T, L, H_I, H).total;
}

static dsa_status_t dsa_indexer_warmup_impl(const uint8_t* q8, const float* q_scale, const float* w,
                                            const uint8_t* k8, const float* k_scale,
                                            const uint16_t* q, const uint16_t* kv, int T, int L,
                                            int H_I, int H, int q_pos0, float score_scale,
                                            float sm_scale, float* kl, float* dq, float* dw,
                                            float* dk, float* lse_teacher, float* lse_index,
                                            void* workspace, size_t workspace_bytes,
                                            dsa_stream_t stream)
{
    if (dsa_status_t st = check_teacher(q, kv, T, L, H, q_pos0, sm_scale)) return st;
    if (!(score_scale > 0.f)) return DSA_ERR_INVALID_ARGUMENT;
    if (!dsa::warmup_supports(H_I, H)) return DSA_ERR_UNSUPPORTED;
    // (token, head) rows are indexed with 32-bit integers inside the gradient kernels
    if ((int64_t)T * L > kMaxElems || (int64_t)T * H_I >= (int64_t(1) << 31))
        return DSA_ERR_UNSUPPORTED;
    if (!dk) return DSA_ERR_INVALID_ARGUMENT;
    if (T > 0 && (!q8 || !q_scale || !w || !k8 || !k_scale || !kl || !dq || !dw))
        return DSA_ERR_INVALID_ARGUMENT;
    if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(dq, 16) || !aligned(dk, 16))
        return DSA_ERR_INVALID_ARGUMENT;
    hipStream_t s = as_hip(stream);
    if (T == 0)                                       // no rows: the key gradient is zero
        return from_hip(dsa::launch_zero(dk, (int64_t)L * 128, s));
    const WarmupWs ws = warmup_ws(T, L, H_I, H);
    if (!workspace || workspace_bytes < ws.total) return DSA_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(workspace, kAlign)) return DSA_ERR_INVALID_ARGUMENT;

    uint8_t* base = static_cast<uint8_t*>(workspace);
    float* pg = reinterpret_cast<float*>(base + ws.pg_off);
    float* sc = reinterpret_cast<float*>(base + ws.i_off);
    float* lse_ws = reinterpret_cast<float*>(base + ws.lse_off);
    float* dkp = reinterpret_cast<float*>(base + ws.dkp_off);
    const int ngroups = H_I / 16;
    hipError_t e = dsa::launch_zero(dkp, (int64_t)ngroups * L * 128, s);
    for (int r0 = 0; r0 < T && e == hipSuccess; r0 += ws.chunk) {
        const int rows = std::min(ws.chunk, T - r0);
        const int qp = q_pos0 + r0;
        const uint16_t* qc = q + (int64_t)r0 * H * 576;
        float* lt = lse_teacher ? lse_teacher + (int64_t)r0 * H : lse_ws;
        const int64_t o = (int64_t)r0 * H_I;
        e = dsa::launch_attention_lse(qc, kv, rows, H, qp, sm_scale, lt, s);
        if (e == hipSuccess)
            e = dsa::launch_attention_dist(qc, kv, lt, rows, H, qp, sm_scale, pg, L, s);
        if (e == hipSuccess)
            e = dsa::launch_indexer_prefill(q8 + o * 128, q_scale + o, w + o, k8, k_scale, rows, L,
                                            H_I, qp, score_scale, sc, L, s);
        if (e == hipSuccess)
            e = dsa::launch_warmup_rows(sc, pg, L, rows, qp, kl + r0,
                                        lse_index ? lse_index + r0 : nullptr, s);
        if (e == hipSuccess)
            e = dsa::launch_warmup_dq(q8 + o * 128, q_scale + o, w + o, k8, k_scale, pg, L, rows,
                                      H_I, qp, score_scale, dq + o * 128, dw + o, s);
        if (e == hipSuccess)
            e = dsa::launch_warmup_dk(q8 + o * 128, q_scale + o, w + o, k8, pg, L, rows, H_I, qp,
                                      score_scale, L, dkp, s);
    }
    if (e == hipSuccess) e = dsa::launch_warmup_dk_reduce(dkp, ngroups, (int64_t)L * 128, dk, s);
    return from_hip(e);
}

size_t dsa_decode_workspace_bytes(int B, int max_len, int64_t total_tokens, int H_I, int H,
                                  int k)
{
    (void)H_I;
    if (B <= 0 || max_len < 1 || total_tokens <= 0 || H < 1 || k < 1) return 0;
    return decode_ws(B, max_len, total_tokens, H, k).total;
}

// Validation shared by the decode entry points (everything but the workspace).
static dsa_status_t decode_check(int B, const int64_t* seq_start, int max_len,
                                 int64_t total_tokens, const uint8_t* q8, const float* q_scale,
                                 const float* w, const uint8_t* k8_cache,
                                 const float* k_scale_cache, const uint16_t* q,
                                 const uint16_t* kv_cache, int H_I, int H, int k,
                                 float score_scale, float sm_scale, const uint16_t* out)
{
    if (B < 0) return DSA_ERR_INVALID_ARGUMENT;
    if (B == 0) return DSA_OK;                       // nothing to decode
    if (max_len < 1 || total_tokens < 1 || k < 1 || H < 1) return DSA_ERR_INVALID_ARGUMENT;
    if ((int64_t)B * max_len < total_tokens) return DSA_ERR_INVALID_ARGUMENT;
    if ((!seq_start || !q8 || !q_scale || !w || !k8_cache || !k_scale_cache || !q ||
                  !kv_cache || !out))
        return DSA_ERR_INVALID_ARGUMENT;
    if (!(score_scale > 0.f) || !(sm_scale > 0.f)) return DSA_ERR_INVALID_ARGUMENT;
    if (!dsa::indexer_supports(H_I) || !heads_ok(H) || !k_ok(k)) return DSA_ERR_UNSUPPORTED;
    if (total_tokens >= (int64_t(1) << 31) || B > 65535 || !cache_ok(max_len))
        return DSA_ERR_UNSUPPORTED;
    if (!aligned(q8, 16) || !aligned(k8_cache, 16) || !aligned(q, 16) ||
        !aligned(kv_cache, 16) || !aligned(out, 8))
        return DSA_ERR_INVALID_ARGUMENT;
    return DSA_OK;
}

// The decode step after validation, on a workspace laid out by decode_ws.
static dsa_status_t decode_run(int B, const int64_t* seq_start, int max_len, const uint8_t* q8,
                               const float* q_scale, const float* w, const uint8_t* k8_cache,
                               const float* k_scale_cache, const uint16_t* q,
                               const uint16_t* kv_cache, int H_I, int H, int k,
                               float score_scale, float sm_scale, uint16_t* out, float* lse,
                               int32_t* idx_out, uint8_t* base, const DecodeWs& ws,
                               hipStream_t s)
{
    float* scores = reinterpret_cast<float*>(base + ws.scores_off);
    int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(base + ws.idx_off);
    float* po = reinterpret_cast<float*>(base + ws.po_off);
    float* pl = reinterpret_cast<float*>(base + ws.pl_off);
    hipError_t e = dsa::launch_indexer_decode(q8, q_scale, w, k8_cache, k_scale_cache,
                                              seq_start, B, max_len, H_I, score_scale, scores, s);
    if (e == hipSuccess)
        e = dsa::launch_topk_decode(scores, seq_start, B, max_len, k, idx,
                                    ws.tk_bytes ? base + ws.tk_off : nullptr, s);
    if (e == hipSuccess)
        e = dsa::launch_sparse_mla(q, kv_cache, idx, seq_start, B, max_len, H, k, sm_scale,
                                   ws.splits, out, lse, po, pl, 0, s);
    if (e == hipSuccess && ws.splits > 1)
        e = dsa::launch_mla_combine(po, pl, B, H, ws.splits, out, lse, s);
    return from_hip(e);
}

static dsa_status_t dsa_decode_impl(int B, const int64_t* seq_start, int max_len,
                                    int64_t total_tokens, const uint8_t* q8, const float* q_scale,
                                    const float* w, const uint8_t* k8_cache,
                                    const float* k_scale_cache, const uint16_t* q,
                                    const uint16_t* kv_cache, int H_I, int H, int k,
                                    float score_scale, float sm_scale, uint16_t* out, float* lse,
                                    int32_t* idx_out, void* workspace, size_t workspace_bytes,
                                    dsa_stream_t stream)
{
    if (dsa_status_t st = decode_check(B, seq_start, max_len, total_tokens, q8, q_scale, w,
                                       k8_cache, k_scale_cache, q, kv_cache, H_I, H, k,
                                       score_scale, sm_scale, out))
        return st;
    if (B == 0) return DSA_OK;
    const DecodeWs ws = decode_ws(B, max_len, total_tokens, H, k);
    if (!workspace || workspace_bytes < ws.total) return DSA_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned(workspace, kAlign)) return DSA_ERR_INVALID_ARGUMENT;
    return decode_run(B, seq_start, max_len, q8, q_scale, w, k8_cache, k_scale_cache, q,
                      kv_cache, H_I, H, k, score_scale, sm_scale, out, lse, idx_out,
                      static_cast<uint8_t*>(workspace), ws, as_hip(stream));
}

// ---- decode without a caller workspace: the same kernels on a scratch array of this file,
// one copy per GPU (a static device array; the loader places it in each GPU's memory when
// the library's code is loaded there), for callers that cannot allocate.  Host code never
// passes the array's name to a kernel (that is a host-side stand-in, not a device address):
// it asks the runtime for each device's address once, with that device current, and keeps it.
static __device__ __align__(256) uint8_t scratch[DSA_DECODE_NOALLOC_SCRATCH_BYTES];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// this device's scratch address, looked up on its first use (nullptr on failure)
static void* scratch_on(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return nullptr;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

static dsa_status_t dsa_decode_noalloc_impl(int B, const int64_t* seq_start, int max_len,
                                            int64_t total_tokens, const uint8_t* q8,
                                            const float* q_scale, const float* w,
                                            const uint8_t* k8_cache, const float* k_scale_cache,
                                            const uint16_t* q, const uint16_t* kv_cache, int H_I,
                                            int H, int k, float score_scale, float sm_scale,
                                            uint16_t* out, float* lse, int32_t* idx_out,
                                            dsa_stream_t stream)
{
    if (dsa_status_t st = decode_check(B, seq_start, max_len, total_tokens, q8, q_scale, w,
                                       k8_cache, k_scale_cache, q, kv_cache, H_I, H, k,
                                       score_scale, sm_scale, out))
        return st;
    if (B == 0) return DSA_OK;
    const DecodeWs ws = decode_ws(B, max_len, total_tokens, H, k);
    if (ws.total > (size_t)DSA_DECODE_NOALLOC_SCRATCH_BYTES) return DSA_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t s = as_hip(stream);
    int dev = -1;
    if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) return DSA_ERR_HIP;
    uint8_t* base = static_cast<uint8_t*>(scratch_on(dev));
    if (!base) return DSA_ERR_HIP;
    return decode_run(B, seq_start, max_len, q8, q_scale, w, k8_cache, k_scale_cache, q,
                      kv_cache, H_I, H, k, score_scale, sm_scale, out, lse, idx_out, base, ws, s);
}

static dsa_status_t dsa_quantize_fp8_impl(const void* x, int x_is_bf16, int64_t n, uint8_t* q8,
                                          float* scale, dsa_stream_t stream)
{
    if (n < 0 || (x_is_bf16 != 0 && x_is_bf16 != 1)) return DSA_ERR_INVALID_ARGUMENT;
    if (n == 0) return DSA_OK;
    if (!x || !q8 || !scale) return DSA_ERR_INVALID_ARGUMENT;
    if (n > kMaxElems / 128) return DSA_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(q8, 8) || !aligned(scale, 4)) return DSA_ERR_INVALID_ARGUMENT;
    return from_hip(dsa::launch_quantize_fp8(x, x_is_bf16 != 0, n, q8, scale, as_hip(stream)));
}

static dsa_status_t dsa_decode_append_impl(int B, const int64_t* seq_start, const void* k_new,
                                           int k_is_bf16, const uint16_t* kv_new, uint8_t* k8_cache,
                                           float* k_scale_cache, uint16_t* kv_cache,
                                           dsa_stream_t stream)
{
    if (B < 0 || (k_is_bf16 != 0 && k_is_bf16 != 1)) return DSA_ERR_INVALID_ARGUMENT;
    if (B == 0) return DSA_OK;
    if (B > 65535) return DSA_ERR_UNSUPPORTED;
    if (!seq_start || !k_new || !kv_new || !k8_cache || !k_scale_cache || !kv_cache)
        return DSA_ERR_INVALID_ARGUMENT;
    if (!aligned(k_new, 16) || !aligned(kv_new, 16) || !aligned(k8_cache, 8) ||
        !aligned(k_scale_cache, 4) || !aligned(kv_cache, 16))
        return DSA_ERR_INVALID_ARGUMENT;
    return from_hip(dsa::launch_decode_append(B, seq_start, k_new, k_is_bf16 != 0, kv_new,
                                              k8_cache, k_scale_cache, kv_cache,
                                              as_hip(stream)));
}

static dsa_status_t dsa_window_indices_impl(int T, int L, int q_pos0, int window, int32_t* idx,
                                            dsa_stream_t stream)
{
    if (check_rows(T, L, q_pos0) != DSA_OK || window < 1) return DSA_ERR_INVALID_ARGUMENT;
    if (T == 0) return DSA_OK;
    if (!idx) return DSA_ERR_INVALID_ARGUMENT;
    if ((int64_t)T * window > kMaxElems) return DSA_ERR_UNSUPPORTED;
    return from_hip(dsa::launch_window_indices(T, q_pos0, window, idx, as_hip(stream)));
}

static dsa_status_t dsa_local_selected_indices_impl(const int32_t* sel, int T, int L, int q_pos0,
                                                    int k, int window, int32_t* out,
                                                    dsa_stream_t stream)
{
    if (check_rows(T, L, q_pos0) != DSA_OK || window < 1 || k < 1)
        return DSA_ERR_INVALID_ARGUMENT;
    if (T == 0) return DSA_OK;
    if (!sel || !out) return DSA_ERR_INVALID_ARGUMENT;
    if ((int64_t)window + k > (int64_t(1) << 30) ||
        (int64_t)T * (window + k) > kMaxElems)
        return DSA_ERR_UNSUPPORTED;
    return from_hip(dsa::launch_local_selected(sel, T, k, q_pos0, window, out, as_hip(stream)));
}

// ---- the exported entry points: the implementations above, with the DSA_LOG launch log

dsa_status_t dsa_index_scores(const uint8_t* q8, const float* q_scale, const float* w,
                              const uint8_t* k8, const float* k_scale, int T, int L, int H_I,
                              int q_pos0, float score_scale, float* scores, int64_t ld_scores,
                              int write_masked, dsa_stream_t stream)
{
    return logged(dsa_index_scores_impl(q8, q_scale, w, k8, k_scale, T, L, H_I, q_pos0, score_scale,
                  scores, ld_scores, write_masked, stream),
                  "dsa_index_scores T=%d L=%d H_I=%d q_pos0=%d", T, L, H_I, q_pos0);
}

dsa_status_t dsa_topk(const float* scores, int64_t ld_scores, int T, int L, int q_pos0, int k,
                      int32_t* idx, void* workspace, size_t workspace_bytes, dsa_stream_t stream)
{
    (void)workspace;                                 // dsa_topk needs no workspace
    (void)workspace_bytes;
    return logged(dsa_topk_impl(scores, ld_scores, T, L, q_pos0, k, idx, stream),
                  "dsa_topk T=%d L=%d q_pos0=%d k=%d", T, L, q_pos0, k);
}

dsa_status_t dsa_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int T,
                            int L, int H, int k, float sm_scale, uint16_t* out, float* lse,
                            dsa_stream_t stream)
{
    return logged(dsa_sparse_mla_impl(q, kv, idx, T, L, H, k, sm_scale, out, lse, stream),
                  "dsa_sparse_mla T=%d L=%d H=%d k=%d", T, L, H, k);
}

dsa_status_t dsa_prefill(const uint8_t* q8, const float* q_scale, const float* w,
                         const uint8_t* k8, const float* k_scale, const uint16_t* q,
                         const uint16_t* kv, int T, int L, int H_I, int H, int k, int q_pos0,
                         float score_scale, float sm_scale, uint16_t* out, float* lse,
                         int32_t* idx_out, void* workspace, size_t workspace_bytes,
                         dsa_stream_t stream)
{
    return logged(dsa_prefill_impl(q8, q_scale, w, k8, k_scale, q, kv, T, L, H_I, H, k, q_pos0,
                  score_scale, sm_scale, out, lse, idx_out, workspace, workspace_bytes, stream),
                  "dsa_prefill T=%d L=%d H_I=%d H=%d k=%d q_pos0=%d", T, L, H_I, H, k, q_pos0);
}

dsa_status_t dsa_prefill_varlen(int B, const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_k,
                                const uint8_t* q8, const float* q_scale, const float* w,
                                const uint8_t* k8, const float* k_scale, const uint16_t* q,
                                const uint16_t* kv, int H_I, int H, int k, float score_scale,
                                float sm_scale, uint16_t* out, float* lse, int32_t* idx_out,
                                void* workspace, size_t workspace_bytes, dsa_stream_t stream)
{
    return logged(dsa_prefill_varlen_impl(B, cu_seqlens_q, cu_seqlens_k, q8, q_scale, w, k8,
                  k_scale, q, kv, H_I, H, k, score_scale, sm_scale, out, lse, idx_out,
                  workspace, workspace_bytes, stream),
                  "dsa_prefill_varlen B=%d H_I=%d H=%d k=%d", B, H_I, H, k);
}

dsa_status_t dsa_attention_lse(const uint16_t* q, const uint16_t* kv, int T, int L, int H,
                               int q_pos0, float sm_scale, float* lse, dsa_stream_t stream)
{
    return logged(dsa_attention_lse_impl(q, kv, T, L, H, q_pos0, sm_scale, lse, stream),
                  "dsa_attention_lse T=%d L=%d H=%d q_pos0=%d", T, L, H, q_pos0);
}

dsa_status_t dsa_attention_distribution(const uint16_t* q, const uint16_t* kv, const float* lse,
                                        int T, int L, int H, int q_pos0, float sm_scale,
                                        float* P, int64_t ld, dsa_stream_t stream)
{
    return logged(dsa_attention_distribution_impl(q, kv, lse, T, L, H, q_pos0, sm_scale, P, ld,
                  stream),
                  "dsa_attention_distribution T=%d L=%d H=%d q_pos0=%d", T, L, H, q_pos0);
}

dsa_status_t dsa_indexer_warmup(const uint8_t* q8, const float* q_scale, const float* w,
                                const uint8_t* k8, const float* k_scale, const uint16_t* q,
                                const uint16_t* kv, int T, int L, int H_I, int H, int q_pos0,
                                float score_scale, float sm_scale, float* kl, float* dq,
                                float* dw, float* dk, float* lse_teacher, float* lse_index,
                                void* workspace, size_t workspace_bytes, dsa_stream_t stream)
{
    return logged(dsa_indexer_warmup_impl(q8, q_scale, w, k8, k_scale, q, kv, T, L, H_I, H, q_pos0,
                  score_scale, sm_scale, kl, dq, dw, dk, lse_teacher, lse_index, workspace,
                  workspace_bytes, stream),
                  "dsa_indexer_warmup T=%d L=%d H_I=%d H=%d q_pos0=%d", T, L, H_I, H, q_pos0);
}

dsa_status_t dsa_decode(int B, const int64_t* seq_start, int max_len, int64_t total_tokens,
                        const uint8_t* q8, const float* q_scale, const float* w,
                        const uint8_t* k8_cache, const float* k_scale_cache,
                        const uint16_t* q, const uint16_t* kv_cache, int H_I, int H, int k,
                        float score_scale, float sm_scale, uint16_t* out, float* lse,
                        int32_t* idx_out, void* workspace, size_t workspace_bytes,
                        dsa_stream_t stream)
{
    return logged(dsa_decode_impl(B, seq_start, max_len, total_tokens, q8, q_scale, w, k8_cache,
                  k_scale_cache, q, kv_cache, H_I, H, k, score_scale, sm_scale, out, lse,
                  idx_out, workspace, workspace_bytes, stream),
                  "dsa_decode B=%d max_len=%d total_tokens=%lld H_I=%d H=%d k=%d", B, max_len,
                  (long long)total_tokens, H_I, H, k);
}

dsa_status_t dsa_decode_noalloc(int B, const int64_t* seq_start, int max_len,
                                int64_t total_tokens, const uint8_t* q8, const float* q_scale,
                                const float* w, const uint8_t* k8_cache,
                                const float* k_scale_cache, const uint16_t* q,
                                const uint16_t* kv_cache, int H_I, int H, int k,
                                float score_scale, float sm_scale, uint16_t* out, float* lse,
                                int32_t* idx_out, dsa_stream_t stream)
{
    return logged(dsa_decode_noalloc_impl(B, seq_start, max_len, total_tokens, q8, q_scale, w,
                                          k8_cache, k_scale_cache, q, kv_cache, H_I, H, k,
                                          score_scale, sm_scale, out, lse, idx_out, stream),
                  "dsa_decode_noalloc B=%d max_len=%d total_tokens=%lld H_I=%d H=%d k=%d", B,
                  max_len, (long long)total_tokens, H_I, H, k);
}

size_t dsa_decode_noalloc_scratch_bytes(void) { return DSA_DECODE_NOALLOC_SCRATCH_BYTES; }

dsa_status_t dsa_quantize_fp8(const void* x, int x_is_bf16, int64_t n, uint8_t* q8,
                              float* scale, dsa_stream_t stream)
{
    return logged(dsa_quantize_fp8_impl(x, x_is_bf16, n, q8, scale, stream),
                  "dsa_quantize_fp8 n=%lld", (long long)n);
}

dsa_status_t dsa_decode_append(int B, const int64_t* seq_start, const void* k_new, int k_is_bf16,
                               const uint16_t* kv_new, uint8_t* k8_cache, float* k_scale_cache,
                               uint16_t* kv_cache, dsa_stream_t stream)
{
    return logged(dsa_decode_append_impl(B, seq_start, k_new, k_is_bf16, kv_new, k8_cache,
                  k_scale_cache, kv_cache, stream),
                  "dsa_decode_append B=%d", B);
}

dsa_status_t dsa_window_indices(int T, int L, int q_pos0, int window, int32_t* idx,
                                dsa_stream_t stream)
{
    return logged(dsa_window_indices_impl(T, L, q_pos0, window, idx, stream),
                  "dsa_window_indices T=%d L=%d q_pos0=%d window=%d", T, L, q_pos0, window);
}

dsa_status_t dsa_local_selected_indices(const int32_t* sel, int T, int L, int q_pos0, int k,
                                        int window, int32_t* out, dsa_stream_t stream)
{
    return logged(dsa_local_selected_indices_impl(sel, T, L, q_pos0, k, window, out, stream),
                  "dsa_local_selected_indices T=%d L=%d q_pos0=%d k=%d window=%d", T, L, q_pos0,
                  k, window);
}

}  // extern "C"
