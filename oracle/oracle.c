/*
 * oracle.c -- plain CPU oracle for the DSA hot path (TEST INFRASTRUCTURE ONLY).
 * Definitions and page citations are in oracle.h.  Everything is fp64 except the
 * indexer dot products, which are exact int64 sums.  OpenMP parallelises over rows only;
 * every row is an independent, straightforward loop.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- decoders */

/* OCP e4m3fn: sign | 4 exponent bits (bias 7) | 3 mantissa bits; E=15,M=7 is NaN,
 * E=0 is subnormal M * 2^-9; there are no infinities. */
double ora_e4m3fn_value(uint8_t code)
{
    int sign = code >> 7, E = (code >> 3) & 15, M = code & 7;
    double mag;
    if (E == 15 && M == 7) return NAN;
    if (E == 0) mag = ldexp((double)M, -9);
    else        mag = ldexp(1.0 + M / 8.0, E - 7);
    return sign ? -mag : mag;
}

/* The same value times 2^9, which is always an integer of magnitude <= 448*512. */
static int64_t e4m3fn_times_512(uint8_t code)
{
    int sign = code >> 7, E = (code >> 3) & 15, M = code & 7;
    int64_t mag = (E == 0) ? (int64_t)M : ((int64_t)(8 + M) << (E - 1));
    return sign ? -mag : mag;
}

static int e4m3fn_is_nan(uint8_t code) { return (code & 0x7F) == 0x7F; }

/* bf16 is the top half of an IEEE binary32. */
double ora_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int ora_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ----------------------------------------------------------------- indexer */

int ora_index_scores(const uint8_t* q8, const float* qs, const float* w,
                     const uint8_t* k8, const float* ks, int64_t L, int H_I,
                     int64_t q_pos0, double c, const int64_t* rows, int64_t n_rows,
                     double* scores, double* bound)
{
    if (L <= 0 || H_I <= 0 || n_rows < 0 || q_pos0 < 0) return -1;
    for (int64_t s = 0; s < L * 128; ++s)
        if (e4m3fn_is_nan(k8[s])) return -1;

    /* keys decoded once to integers (value * 2^9) */
    int64_t* kint = (int64_t*)malloc(sizeof(int64_t) * (size_t)L * 128);
    if (!kint) return -1;
    for (int64_t s = 0; s < L * 128; ++s) kint[s] = e4m3fn_times_512(k8[s]);

    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t t = rows[r];
        const int64_t p = q_pos0 + t;          /* absolute position of the query */
        int64_t qint[128 * 128];               /* H_I <= 128 */
        double wprime[128];
        if (t < 0 || H_I > 128) { bad = 1; continue; }
        for (int h = 0; h < H_I; ++h) {
            for (int d = 0; d < 128; ++d) {
                uint8_t code = q8[(t * H_I + h) * 128 + d];
                if (e4m3fn_is_nan(code)) bad = 1;
                qint[h * 128 + d] = e4m3fn_times_512(code);
            }
            /* per-head weight a_h carries the query's dequantisation scale and c */
            wprime[h] = (double)w[t * H_I + h] * (double)qs[t * H_I + h] * c;
        }
        for (int64_t s = 0; s < L; ++s) {
            double* out = scores + r * L + s;
            if (s > p) {                         /* future token: masked */
                *out = -INFINITY;
                if (bound) bound[r * L + s] = 0.0;
                continue;
            }
            double acc = 0.0, acc_abs = 0.0;
            for (int h = 0; h < H_I; ++h) {
                int64_t dot = 0, dot_abs = 0;
                for (int d = 0; d < 128; ++d) {
                    int64_t prod = qint[h * 128 + d] * kint[s * 128 + d];
                    dot += prod;
                    dot_abs += prod < 0 ? -prod : prod;
                }
                /* |dot| < 128 * 2^36 = 2^43, so the scaling to fp64 is exact */
                double D = ldexp((double)dot, -18);
                double relu = D > 0.0 ? D : 0.0;
                acc += wprime[h] * relu;
                acc_abs += fabs(wprime[h]) * ldexp((double)dot_abs, -18);
            }
            *out = (double)ks[s] * acc;
            if (bound) bound[r * L + s] = (double)ks[s] * acc_abs;
        }
    }
    free(kint);
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------- top-k */

typedef struct { double v; int64_t pos; } item_t;

/* (score descending, position ascending): a total order, so any sort is deterministic */
static int cmp_item(const void* a, const void* b)
{
    const item_t* x = (const item_t*)a;
    const item_t* y = (const item_t*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->pos > y->pos) - (x->pos < y->pos);
}

static int cmp_i32(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

static int fill_all_visible(int64_t n, int k, int32_t* out)
{
    for (int j = 0; j < k; ++j) out[j] = (j < n) ? (int32_t)j : -1;
    return 0;
}

int ora_topk_sort(const double* scores, int64_t ld, int64_t n_rows, const int64_t* n_vis,
                  int k, int32_t* idx)
{
    if (k <= 0 || n_rows < 0) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t n = n_vis[r];
        int32_t* out = idx + r * k;
        if (n < 0 || n > ld) { bad = 1; continue; }
        if (n <= k) { fill_all_visible(n, k, out); continue; }
        item_t* it = (item_t*)malloc(sizeof(item_t) * (size_t)n);
        if (!it) { bad = 1; continue; }
        for (int64_t s = 0; s < n; ++s) { it[s].v = scores[r * ld + s]; it[s].pos = s; }
        qsort(it, (size_t)n, sizeof(item_t), cmp_item);
        for (int j = 0; j < k; ++j) out[j] = (int32_t)it[j].pos;
        qsort(out, (size_t)k, sizeof(int32_t), cmp_i32);
        free(it);
    }
    return bad ? -1 : 0;
}

/* k-th largest (1-based) of v[0..n) by Hoare-style quickselect; reorders v. */
static double kth_largest(double* v, int64_t n, int64_t kth)
{
    int64_t lo = 0, hi = n - 1, want = kth - 1;   /* index in descending order */
    while (lo < hi) {
        double pivot = v[lo + (hi - lo) / 2];
        int64_t i = lo, j = hi;
        while (i <= j) {
            while (v[i] > pivot) ++i;
            while (v[j] < pivot) --j;
            if (i <= j) { double tmp = v[i]; v[i] = v[j]; v[j] = tmp; ++i; --j; }
        }
        if (want <= j) hi = j;
        else if (want >= i) lo = i;
        else return v[want];
    }
    return v[want];
}

int ora_topk_select(const double* scores, int64_t ld, int64_t n_rows, const int64_t* n_vis,
                    int k, int32_t* idx)
{
    if (k <= 0 || n_rows < 0) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t n = n_vis[r];
        int32_t* out = idx + r * k;
        if (n < 0 || n > ld) { bad = 1; continue; }
        if (n <= k) { fill_all_visible(n, k, out); continue; }
        const double* row = scores + r * ld;
        double* tmp = (double*)malloc(sizeof(double) * (size_t)n);
        if (!tmp) { bad = 1; continue; }
        memcpy(tmp, row, sizeof(double) * (size_t)n);
        const double tau = kth_largest(tmp, n, k);      /* the k-th best score */
        free(tmp);
        int64_t above = 0;
        for (int64_t s = 0; s < n; ++s) above += row[s] > tau;
        int64_t ties_left = k - above;                   /* >= 1 */
        int j = 0;
        for (int64_t s = 0; s < n && j < k; ++s) {
            if (row[s] > tau) out[j++] = (int32_t)s;
            else if (row[s] == tau && ties_left > 0) { out[j++] = (int32_t)s; --ties_left; }
        }
        if (j != k) bad = 1;
    }
    return bad ? -1 : 0;
}

/* --------------------------------------------------------------------- MLA */

/* softmax attention of one query head over a list of cache rows */
static void attend(const uint16_t* qrow, const uint16_t* kv, const int64_t* sel, int64_t m,
                   double sm_scale, double* logit, double* out, double* lse)
{
    double qv[576];
    for (int d = 0; d < 576; ++d) qv[d] = ora_bf16_value(qrow[d]);
    for (int d = 0; d < 512; ++d) out[d] = 0.0;
    if (m == 0) { *lse = -INFINITY; return; }
    double mx = -INFINITY;
    for (int64_t j = 0; j < m; ++j) {
        const uint16_t* row = kv + sel[j] * 576;
        double dot = 0.0;
        for (int d = 0; d < 576; ++d) dot += qv[d] * ora_bf16_value(row[d]);
        logit[j] = sm_scale * dot;
        if (logit[j] > mx) mx = logit[j];
    }
    double Z = 0.0;
    for (int64_t j = 0; j < m; ++j) Z += exp(logit[j] - mx);
    for (int64_t j = 0; j < m; ++j) {
        const double pj = exp(logit[j] - mx) / Z;
        const uint16_t* row = kv + sel[j] * 576;
        for (int d = 0; d < 512; ++d) out[d] += pj * ora_bf16_value(row[d]);
    }
    *lse = mx + log(Z);
}

int ora_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* idx, int64_t L,
                   int H, int k, double sm_scale, const int64_t* rows, int64_t n_rows,
                   double* out, double* lse)
{
    if (L <= 0 || H <= 0 || k <= 0 || n_rows < 0) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t t = rows[r];
        int64_t* sel = (int64_t*)malloc(sizeof(int64_t) * (size_t)k);
        double* logit = (double*)malloc(sizeof(double) * (size_t)k);
        int64_t m = 0;
        for (int j = 0; j < k; ++j) {
            int32_t s = idx[t * k + j];
            if (s < 0) continue;                  /* padding */
            if (s >= L) { bad = 1; continue; }
            sel[m++] = s;
        }
        for (int h = 0; h < H; ++h)
            attend(q + (t * H + h) * 576, kv, sel, m, sm_scale, logit,
                   out + (r * H + h) * 512, lse + r * H + h);
        free(sel);
        free(logit);
    }
    return bad ? -1 : 0;
}

int ora_dense_mla(const uint16_t* q, const uint16_t* kv, int64_t L, int H, int64_t q_pos0,
                  double sm_scale, const int64_t* rows, int64_t n_rows, double* out,
                  double* lse)
{
    /* Written independently of attend(): a streaming (running-max) softmax over every
     * visible position, no index list involved. */
    if (L <= 0 || H <= 0 || n_rows < 0 || q_pos0 < 0) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t t = rows[r];
        const int64_t p = q_pos0 + t;
        if (t < 0 || p >= L) { bad = 1; continue; }
        for (int h = 0; h < H; ++h) {
            const uint16_t* qrow = q + (t * H + h) * 576;
            double qv[576];
            for (int d = 0; d < 576; ++d) qv[d] = ora_bf16_value(qrow[d]);
            double* o = out + (r * H + h) * 512;
            double run_max = -INFINITY, run_sum = 0.0;
            for (int d = 0; d < 512; ++d) o[d] = 0.0;
            for (int64_t s = 0; s <= p; ++s) {
                const uint16_t* row = kv + s * 576;
                double dot = 0.0;
                for (int d = 0; d < 576; ++d)
                    dot += qv[d] * ora_bf16_value(row[d]);
                const double logit = sm_scale * dot;
                if (logit > run_max) {                 /* rescale what was summed so far */
                    const double f = exp(run_max - logit);
                    run_sum *= f;
                    for (int d = 0; d < 512; ++d) o[d] *= f;
                    run_max = logit;
                }
                const double e = exp(logit - run_max);
                run_sum += e;
                for (int d = 0; d < 512; ++d) o[d] += e * ora_bf16_value(row[d]);
            }
            for (int d = 0; d < 512; ++d) o[d] /= run_sum;
            lse[r * H + h] = run_max + log(run_sum);
        }
    }
    return bad ? -1 : 0;
}

/* ---- fp8 preparation of the indexer inputs, and the decode cache append ------------- */

/* Nearest e4m3fn code to y (|y| <= 448, the largest finite value), ties to the even code,
 * i.e. round to nearest even; the sign of y, zero included, goes to the sign bit. */
static uint8_t e4m3fn_nearest(float y)
{
    const int neg = signbit(y) != 0;
    const double a = fabs((double)y);
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        const double d = fabs(ora_e4m3fn_value((uint8_t)c) - a);
        if (d < bd || (d == bd && (c & 1) == 0)) {
            bd = d;
            best = c;
        }
    }
    return (uint8_t)(best | (neg << 7));
}

static float vec_elem(const void* x, int x_bf16, int64_t i)
{
    if (x_bf16) {
        const uint32_t u = (uint32_t)((const uint16_t*)x)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return f;
    }
    return ((const float*)x)[i];
}

int ora_quantize_e4m3(const void* x, int x_bf16, int64_t n, uint8_t* q8, float* scale)
{
    if (!x || !q8 || !scale || n < 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < n; ++v) {
        float amax = 0.f;
        for (int d = 0; d < 128; ++d) {
            const float a = fabsf(vec_elem(x, x_bf16, v * 128 + d));
            if (a > amax) amax = a;
        }
        const float s = amax > 0.f ? amax / 448.0f : 1.0f;   /* fp32 division */
        scale[v] = s;
        for (int d = 0; d < 128; ++d) {
            float y = vec_elem(x, x_bf16, v * 128 + d) / s;   /* rounded to fp32 */
            if (y > 448.f) y = 448.f;
            if (y < -448.f) y = -448.f;
            q8[v * 128 + d] = e4m3fn_nearest(y);
        }
    }
    return 0;
}

int ora_decode_append(int B, const int64_t* seq_start, const void* k_new, int k_bf16,
                      const uint16_t* kv_new, uint8_t* k8_cache, float* k_scale_cache,
                      uint16_t* kv_cache)
{
    if (B < 0 || !seq_start || !k_new || !kv_new || !k8_cache || !k_scale_cache || !kv_cache)
        return -1;
    for (int b = 0; b < B; ++b)
        if (seq_start[b + 1] <= seq_start[b]) return -1;
    const size_t esz = k_bf16 ? 2 : 4;
    for (int b = 0; b < B; ++b) {
        const int64_t r = seq_start[b + 1] - 1;
        ora_quantize_e4m3((const uint8_t*)k_new + (size_t)b * 128 * esz, k_bf16, 1,
                          k8_cache + r * 128, k_scale_cache + r);
        memcpy(kv_cache + r * 576, kv_new + (size_t)b * 576, 576 * sizeof(uint16_t));
    }
    return 0;
}

/* ---- alternative index rules ------------------------------------------------------- */

int ora_window_indices(int64_t T, int64_t q_pos0, int W, int32_t* idx)
{
    if (T < 0 || q_pos0 < 0 || W < 1 || !idx) return -1;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t p = q_pos0 + t;
        int j = 0;
        for (int64_t s = 0; s <= p; ++s)               /* the W positions ending at p */
            if (s > p - W) idx[t * W + j++] = (int32_t)s;
        for (; j < W; ++j) idx[t * W + j] = -1;
    }
    return 0;
}

int ora_local_selected(const int32_t* sel, int64_t T, int k, int64_t q_pos0, int W, int32_t* out)
{
    if (!sel || !out || T < 0 || k < 1 || W < 1 || q_pos0 < 0) return -1;
    const int M = W + k;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t p = q_pos0 + t;
        unsigned char* in = calloc((size_t)p + 1, 1);  /* membership over positions 0..p */
        if (!in) return -1;
        for (int64_t s = 0; s <= p; ++s) if (s > p - W) in[s] = 1;
        for (int j = 0; j < k; ++j) {
            const int32_t s = sel[t * k + j];
            if (s >= 0 && s <= p) in[s] = 1;
        }
        int j = 0;
        for (int64_t s = 0; s <= p && j < M; ++s) if (in[s]) out[t * M + j++] = (int32_t)s;
        for (; j < M; ++j) out[t * M + j] = -1;
        free(in);
    }
    return 0;
}

/* ---- indexer warm-up: KL to the head-averaged dense attention, and its gradient ------ */

static double dot_n(const double* a, const double* b, int n, double* abs_sum)
{
    double acc = 0.0, acc_abs = 0.0;
    for (int d = 0; d < n; ++d) {
        acc += a[d] * b[d];
        acc_abs += fabs(a[d] * b[d]);
    }
    if (abs_sum) *abs_sum = acc_abs;
    return acc;
}

/* whether a rounded evaluation of x = <a, b> might land on the other side of zero */
static int relu_ambiguous(double x, double abs_sum) { return fabs(x) <= ldexp(abs_sum, -16); }

int ora_warmup(const double* QI, const double* w, const double* q, const int64_t* pos,
               int64_t n_rows, const double* KI, const double* kv, int64_t L, int H_I, int H,
               double c, double sm_scale, double* kl, double* lse_t, double* lse_i, double* dq,
               double* dw, double* P, double* G, double* dk, double* kl_bnd, double* dw_bnd,
               double* dq_bnd, double* dq_amb, double* dk_bnd, double* dk_amb)
{
    if (L <= 0 || H_I <= 0 || H <= 0 || n_rows < 0) return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (pos[r] < 0 || pos[r] >= L) return -1;
    /* the gradient row G of every given row is kept when dk is wanted */
    double *Gall = NULL, *Aall = NULL;
    if (dk || dk_bnd || dk_amb) {
        Gall = (double*)calloc((size_t)n_rows * (size_t)L, sizeof(double));
        Aall = (double*)calloc((size_t)n_rows * (size_t)L, sizeof(double));
        if (!Gall || !Aall) {
            free(Gall);
            free(Aall);
            return -1;
        }
    }
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t n = pos[r] + 1;
        double* logit = (double*)malloc(sizeof(double) * (size_t)n);
        double* Pr = (double*)calloc((size_t)n, sizeof(double));
        double* I = (double*)malloc(sizeof(double) * (size_t)n);
        double* x = (double*)malloc(sizeof(double) * (size_t)n * (size_t)H_I);
        double* xa = (double*)malloc(sizeof(double) * (size_t)n * (size_t)H_I);
        double* Gr = (double*)malloc(sizeof(double) * (size_t)n);
        double* Ar = (double*)malloc(sizeof(double) * (size_t)n);
        if (!logit || !Pr || !I || !x || !xa || !Gr || !Ar) {
            bad = 1;
            free(logit); free(Pr); free(I); free(x); free(xa); free(Gr); free(Ar);
            continue;
        }
        /* teacher: each head's softmax over the visible keys, averaged over heads */
        for (int h = 0; h < H; ++h) {
            const double* qh = q + (r * H + h) * 576;
            double mx = -INFINITY;
            for (int64_t s = 0; s < n; ++s) {
                logit[s] = sm_scale * dot_n(qh, kv + s * 576, 576, NULL);
                if (logit[s] > mx) mx = logit[s];
            }
            double sum = 0.0;
            for (int64_t s = 0; s < n; ++s) sum += exp(logit[s] - mx);
            const double lse = mx + log(sum);
            lse_t[r * H + h] = lse;
            for (int64_t s = 0; s < n; ++s) Pr[s] += exp(logit[s] - lse) / H;
        }
        /* student: indexer scores and their softmax over the same keys */
        double mx = -INFINITY;
        for (int64_t s = 0; s < n; ++s) {
            double acc = 0.0;
            for (int h = 0; h < H_I; ++h) {
                const double xv = dot_n(QI + (r * H_I + h) * 128, KI + s * 128, 128,
                                        &xa[s * H_I + h]);
                x[s * H_I + h] = xv;
                acc += w[r * H_I + h] * (xv > 0.0 ? xv : 0.0);
            }
            I[s] = c * acc;
            if (I[s] > mx) mx = I[s];
        }
        double sum = 0.0;
        for (int64_t s = 0; s < n; ++s) sum += exp(I[s] - mx);
        const double lsei = mx + log(sum);
        lse_i[r] = lsei;
        /* KL(P || Q) and its gradient with respect to the scores */
        double klr = 0.0, klb = 0.0;
        for (int64_t s = 0; s < n; ++s) {
            const double logq = I[s] - lsei;
            if (Pr[s] > 0.0) {
                klr += Pr[s] * (log(Pr[s]) - logq);
                klb += Pr[s] * (fabs(log(Pr[s])) + fabs(logq));
            }
            Gr[s] = exp(logq) - Pr[s];
            Ar[s] = exp(logq) + Pr[s];
        }
        kl[r] = klr;
        if (kl_bnd) kl_bnd[r] = klb;
        /* back through the indexer into w and the query vectors */
        for (int h = 0; h < H_I; ++h) {
            const double wh = w[r * H_I + h];
            double dwh = 0.0, dwb = 0.0;
            double* dqh = dq + (r * H_I + h) * 128;
            for (int d = 0; d < 128; ++d) dqh[d] = 0.0;
            if (dq_bnd) for (int d = 0; d < 128; ++d) dq_bnd[(r * H_I + h) * 128 + d] = 0.0;
            if (dq_amb) for (int d = 0; d < 128; ++d) dq_amb[(r * H_I + h) * 128 + d] = 0.0;
            for (int64_t s = 0; s < n; ++s) {
                const double xv = x[s * H_I + h];
                dwh += Gr[s] * (xv > 0.0 ? xv : 0.0);
                dwb += Ar[s] * fabs(xv);
                const double* ks_ = KI + s * 128;
                if (xv > 0.0) {
                    for (int d = 0; d < 128; ++d) dqh[d] += Gr[s] * ks_[d];
                    if (dq_bnd)
                        for (int d = 0; d < 128; ++d)
                            dq_bnd[(r * H_I + h) * 128 + d] += fabs(c * wh * ks_[d]) * Ar[s];
                }
                if (dq_amb && relu_ambiguous(xv, xa[s * H_I + h]))
                    for (int d = 0; d < 128; ++d)
                        dq_amb[(r * H_I + h) * 128 + d] += fabs(c * wh * ks_[d]) * Ar[s];
            }
            for (int d = 0; d < 128; ++d) dqh[d] *= c * wh;
            dw[r * H_I + h] = c * dwh;
            if (dw_bnd) dw_bnd[r * H_I + h] = fabs(c) * dwb;
        }
        for (int64_t s = 0; s < L; ++s) {
            const double pv = s < n ? Pr[s] : 0.0, gv = s < n ? Gr[s] : 0.0;
            if (P) P[r * L + s] = pv;
            if (G) G[r * L + s] = gv;
            if (Gall) {
                Gall[r * L + s] = gv;
                Aall[r * L + s] = s < n ? Ar[s] : 0.0;
            }
        }
        free(logit); free(Pr); free(I); free(x); free(xa); free(Gr); free(Ar);
    }
    if (!bad && Gall) {
        /* dk: each key collects the rows that see it */
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t s = 0; s < L; ++s) {
            double acc[128], accb[128], acca[128];
            for (int d = 0; d < 128; ++d) acc[d] = accb[d] = acca[d] = 0.0;
            for (int64_t r = 0; r < n_rows; ++r) {
                if (pos[r] < s) continue;
                const double gv = Gall[r * L + s], av = Aall[r * L + s];
                for (int h = 0; h < H_I; ++h) {
                    const double* qh = QI + (r * H_I + h) * 128;
                    double xa_;
                    const double xv = dot_n(qh, KI + s * 128, 128, &xa_);
                    const double f = c * gv * w[r * H_I + h];
                    const double fb = fabs(c * w[r * H_I + h]) * av;
                    if (xv > 0.0)
                        for (int d = 0; d < 128; ++d) {
                            acc[d] += f * qh[d];
                            accb[d] += fb * fabs(qh[d]);
                        }
                    if (relu_ambiguous(xv, xa_))
                        for (int d = 0; d < 128; ++d) acca[d] += fb * fabs(qh[d]);
                }
            }
            for (int d = 0; d < 128; ++d) {
                if (dk) dk[s * 128 + d] = acc[d];
                if (dk_bnd) dk_bnd[s * 128 + d] = accb[d];
                if (dk_amb) dk_amb[s * 128 + d] = acca[d];
            }
        }
    }
    free(Gall);
    free(Aall);
    return bad ? -1 : 0;
}
