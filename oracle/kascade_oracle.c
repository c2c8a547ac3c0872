/*
 * kascade_oracle.c -- plain, slow CPU reference of Kascade's cross-layer
 * Top-k sparse attention (decode and prefill, anchor and reuse layers).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header or constant with the
 * HIP library.
 *
 * What it follows (pages: "microsoft/kascade" README, abstract; the
 * "I/O complexity of attention" abstract on thelatestinai.com/papers/2510.01718):
 *   - Dense attention is the textbook A = softmax(Q K^T / sqrt(d)) V
 *     (I/O-complexity abstract).
 *   - Anchor layers compute exact post-softmax scores, pool them per KV head
 *     over the query heads that share it (the abstract's "head-aware"
 *     selection; GQA grouping h -> h / G), and in prefill also over each
 *     32-query tile (abstract: "tile-level operations"; README notes: tile
 *     size 32), then take the exact Top-k key indices, k given as a percentage
 *     (README: "k=10", "--topk 10").
 *   - Reuse layers attend only over an anchor's index set, read through a
 *     per-KV-head map to an anchor KV head (abstract: indices reused in
 *     intermediate layers, head-aware; README "Running Evaluations": head
 *     mappings stored per model).
 * Readings taken where the pages are silent (each one is a documented
 * choice, not something the pages state):
 *   - pooling is the SUM of each head's own softmax probabilities (each head
 *     normalised over its full causal row first);
 *   - k = round-half-up(pct * n / 100), clamped to [0, n]; decode uses at
 *     least 1 key;
 *   - exact ties are broken toward the lower key index; the decision is
 *     taken on the pooled score rounded to fp32 (the precision in which the
 *     GPU path takes it); index sets are stored in ascending order;
 *   - prefill tile t (rows [32t, 32t+32)) selects from the keys before the
 *     tile, [0, 32t), and always adds its own causal diagonal block;
 *     tile 0 selects nothing;
 *   - the output of a selected set is attention renormalised over that set
 *     (prefill: the set plus the causal diagonal keys of the row);
 *   - query head h uses KV head h / G.
 * Selection variants (the README's "Reproducibility" commands name
 * strategies that pool per KV-head group or over all heads; max-pooling is a
 * further variant of the pooling operator): the _v entry points take a
 * pooling scope (0: the G heads sharing a KV head, one set per KV head;
 * 1: all query heads, one set shared by every KV head) and operator (0: sum,
 * 1: maximum); the plain entry points are scope 0 with the sum.
 *
 * Arithmetic is IEEE double throughout (inputs arrive as float, which holds
 * bf16 values exactly). Work units are independent and each is computed by
 * one thread in a fixed order, so results do not depend on the thread count.
 *
 * Status codes: 0 ok, 1 bad argument, 2 allocation failure, 3 index out of
 * range in a supplied index set.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD_ARG 1
#define ORC_NOMEM 2
#define ORC_BAD_INDEX 3

/* ------------------------------------------------------------------ */
/* k rule                                                              */
/* ------------------------------------------------------------------ */

/* round-half-up(pct * n / 100), clamped to [0, n]. */
int64_t orc_topk_count(int64_t n, int32_t pct)
{
    if (n <= 0 || pct <= 0) return 0;
    int64_t k = ((int64_t)pct * n + 50) / 100;
    if (k > n) k = n;
    if (k < 0) k = 0;
    return k;
}

static int64_t decode_k(int64_t n, int32_t pct)
{
    int64_t k = orc_topk_count(n, pct);
    if (k < 1 && n >= 1) k = 1;
    return k;
}

/* Number of tiles and per-tile index-set offsets (CSR) for prefill.
 * offsets has n_tiles + 1 entries; returns the total index count. */
int64_t orc_prefill_offsets(int64_t n, int32_t tile, int32_t pct, int64_t *offsets)
{
    int64_t T = (n + tile - 1) / tile;
    int64_t acc = 0;
    for (int64_t t = 0; t < T; ++t) {
        if (offsets) offsets[t] = acc;
        acc += orc_topk_count(t * (int64_t)tile, pct);
    }
    if (offsets) offsets[T] = acc;
    return acc;
}

/* ------------------------------------------------------------------ */
/* small helpers                                                       */
/* ------------------------------------------------------------------ */

static double dot_scaled(const float *a, const float *b, int D, double scale)
{
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += (double)a[d] * (double)b[d];
    return acc * scale;
}

typedef struct { float val; int64_t idx; } orc_pair;

/* Order: larger value first; equal values -> lower index first. */
static int cmp_pair(const void *pa, const void *pb)
{
    const orc_pair *a = (const orc_pair *)pa, *b = (const orc_pair *)pb;
    if (a->val > b->val) return -1;
    if (a->val < b->val) return 1;
    if (a->idx < b->idx) return -1;
    if (a->idx > b->idx) return 1;
    return 0;
}

static int cmp_i32(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/* Exact Top-k of `score` (n entries) under (value desc, index asc), values
 * compared after rounding to float. Writes k indices in ascending order. */
static int select_topk(const double *score, int64_t n, int64_t k, int32_t *out)
{
    if (k <= 0) return ORC_OK;
    orc_pair *p = (orc_pair *)malloc((size_t)n * sizeof(orc_pair));
    if (!p) return ORC_NOMEM;
    for (int64_t j = 0; j < n; ++j) { p[j].val = (float)score[j]; p[j].idx = j; }
    qsort(p, (size_t)n, sizeof(orc_pair), cmp_pair);
    for (int64_t i = 0; i < k; ++i) out[i] = (int32_t)p[i].idx;
    free(p);
    qsort(out, (size_t)k, sizeof(int32_t), cmp_i32);
    return ORC_OK;
}

/* Softmax-weighted sum of V rows over the key list `keys` (n_keys entries)
 * given their logits: o = sum_j exp(s_j - m) v_j / sum_j exp(s_j - m). */
static void weighted_rows(const double *logit, const int64_t *keys, int64_t n_keys,
                          const float *vbase, int D, double *o)
{
    double m = -INFINITY;
    for (int64_t a = 0; a < n_keys; ++a) if (logit[a] > m) m = logit[a];
    double l = 0.0;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t a = 0; a < n_keys; ++a) {
        double e = exp(logit[a] - m);
        l += e;
        const float *vr = vbase + keys[a] * (int64_t)D;
        for (int d = 0; d < D; ++d) o[d] += e * (double)vr[d];
    }
    for (int d = 0; d < D; ++d) o[d] /= l;
}

static int check_shape(int B, int Hq, int Hkv, int64_t N, int D)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || D <= 0) return ORC_BAD_ARG;
    if (Hq % Hkv) return ORC_BAD_ARG;
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* dense attention (the textbook definition)                          */
/* ------------------------------------------------------------------ */

/* q [B,Hq,Nq,D], k/v [B,Hkv,Nk,D], o [B,Hq,Nq,D]. With causal != 0, query
 * row i sees keys j <= i + (Nk - Nq) (its position at the end of the key
 * sequence). scale <= 0 means 1/sqrt(D). */
int orc_dense_attention(const float *q, const float *k, const float *v, double *o,
                        int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int D,
                        int causal, double scale)
{
    if (check_shape(B, Hq, Hkv, Nk, D) || Nq <= 0 || Nq > Nk) return ORC_BAD_ARG;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    const int G = Hq / Hkv;
    int status = ORC_OK;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)Nk * sizeof(double));
        int64_t *keys = (int64_t *)malloc((size_t)Nk * sizeof(int64_t));
        if (!s || !keys) {
#pragma omp atomic write
            status = ORC_NOMEM;
        } else {
            for (int64_t j = 0; j < Nk; ++j) keys[j] = j;
#pragma omp for collapse(2) schedule(dynamic)
            for (int64_t bh = 0; bh < (int64_t)B * Hq; ++bh) {
                for (int64_t i = 0; i < Nq; ++i) {
                    int64_t b = bh / Hq, h = bh % Hq, g = h / G;
                    const float *qi = q + ((b * Hq + h) * Nq + i) * D;
                    const float *kb = k + (b * Hkv + g) * Nk * D;
                    const float *vb = v + (b * Hkv + g) * Nk * D;
                    int64_t nvis = causal ? (i + (Nk - Nq) + 1) : Nk;
                    for (int64_t j = 0; j < nvis; ++j) s[j] = dot_scaled(qi, kb + j * D, D, scale);
                    weighted_rows(s, keys, nvis, vb, D, o + ((b * Hq + h) * Nq + i) * D);
                }
            }
        }
        free(s);
        free(keys);
    }
    return status;
}

/* ------------------------------------------------------------------ */
/* decode                                                              */
/* ------------------------------------------------------------------ */

/* Anchor layer, one new token per sequence, with the pooling variants the
 * README names among its strategies ("Reproducibility": post-softmax pooling
 * per KV-head group, pooling over all heads) plus max-pooling:
 *   scope 0: one set per (b, KV head g), pooled over the G query heads that
 *            share g (the method's head-aware selection);
 *   scope 1: one set per b, pooled over all Hq query heads and shared by
 *            every KV head;
 *   op 0:    pooled score = sum of the heads' probabilities;
 *   op 1:    pooled score = their maximum.
 * q [B,Hq,D]; k/v [B,Hkv,N,D]; with Hs = (scope ? 1 : Hkv):
 * idx_out [B,Hs,kk] (kk = decode k); o_out [B,Hq,D]; pooled_out [B,Hs,N] or
 * NULL. Each query head's output is attention over its set. */
int orc_decode_anchor_v(const float *q, const float *k, const float *v,
                        int B, int Hq, int Hkv, int64_t N, int D, int32_t pct, double scale,
                        int scope, int op, int32_t *idx_out, double *o_out, double *pooled_out)
{
    if (check_shape(B, Hq, Hkv, N, D) || pct < 1 || pct > 100) return ORC_BAD_ARG;
    if ((scope != 0 && scope != 1) || (op != 0 && op != 1)) return ORC_BAD_ARG;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    const int G = Hq / Hkv;
    const int Hs = scope ? 1 : Hkv;       /* sets per batch row */
    const int ng = scope ? Hkv : 1;       /* KV heads pooled into one set */
    const int nh = ng * G;                /* query heads pooled into one set */
    const int64_t kk = decode_k(N, pct);
    int status = ORC_OK;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)nh * N * sizeof(double));
        double *P = (double *)malloc((size_t)N * sizeof(double));
        double *mrow = (double *)malloc((size_t)nh * sizeof(double));
        double *lrow = (double *)malloc((size_t)nh * sizeof(double));
        double *sel = (double *)malloc((size_t)kk * sizeof(double));
        int64_t *keys = (int64_t *)malloc((size_t)kk * sizeof(int64_t));
        if (!s || !P || !mrow || !lrow || !sel || !keys) {
#pragma omp atomic write
            status = ORC_NOMEM;
        } else {
#pragma omp for schedule(dynamic)
            for (int64_t u = 0; u < (int64_t)B * Hs; ++u) {
                int64_t b = u / Hs, g0 = scope ? 0 : u % Hs;
                /* 1. per-head logits and softmax statistics over all keys;
                 *    head x of the unit is query head (g0 + x / G) * G + x % G */
                for (int x = 0; x < nh; ++x) {
                    const int64_t g = g0 + x / G;
                    const float *kb = k + (b * Hkv + g) * N * D;
                    const float *qh = q + (b * Hq + g * G + x % G) * D;
                    double m = -INFINITY;
                    for (int64_t j = 0; j < N; ++j) {
                        s[x * N + j] = dot_scaled(qh, kb + j * D, D, scale);
                        if (s[x * N + j] > m) m = s[x * N + j];
                    }
                    double l = 0.0;
                    for (int64_t j = 0; j < N; ++j) l += exp(s[x * N + j] - m);
                    mrow[x] = m;
                    lrow[x] = l;
                }
                /* 2. pool the post-softmax probabilities over the unit's heads */
                for (int64_t j = 0; j < N; ++j) {
                    double acc = 0.0;
                    for (int x = 0; x < nh; ++x) {
                        const double p = exp(s[x * N + j] - mrow[x]) / lrow[x];
                        acc = op ? (p > acc ? p : acc) : acc + p;
                    }
                    P[j] = acc;
                }
                if (pooled_out) memcpy(pooled_out + u * N, P, (size_t)N * sizeof(double));
                /* 3. exact Top-k */
                int32_t *S = idx_out + u * kk;
                if (select_topk(P, N, kk, S) != ORC_OK) {
#pragma omp atomic write
                    status = ORC_NOMEM;
                    continue;
                }
                /* 4. attention over the selected keys, per head */
                for (int64_t a = 0; a < kk; ++a) keys[a] = S[a];
                for (int x = 0; x < nh; ++x) {
                    const int64_t g = g0 + x / G;
                    const float *vb = v + (b * Hkv + g) * N * D;
                    for (int64_t a = 0; a < kk; ++a) sel[a] = s[x * N + S[a]];
                    weighted_rows(sel, keys, kk, vb, D, o_out + (b * Hq + g * G + x % G) * D);
                }
            }
        }
        free(s); free(P); free(mrow); free(lrow); free(sel); free(keys);
    }
    return status;
}

/* The method's own anchor layer: scope 0 (per KV-head group), sum pooling. */
int orc_decode_anchor(const float *q, const float *k, const float *v,
                      int B, int Hq, int Hkv, int64_t N, int D, int32_t pct, double scale,
                      int32_t *idx_out, double *o_out, double *pooled_out)
{
    return orc_decode_anchor_v(q, k, v, B, Hq, Hkv, N, D, pct, scale, 0, 0, idx_out, o_out, pooled_out);
}

/* Reuse layer with one anchor set per query head: query head h attends over
 * anchor_idx[b, qmap[h], :] (qmap [Hq], values in [0, Hkv_a)) with its own
 * KV head's K and V. The README stores head mappings per model ("Running
 * Evaluations"); mapping per query head is the finer of the two
 * granularities a GQA model allows. */
int orc_decode_reuse_q(const float *q, const float *k, const float *v,
                       int B, int Hq, int Hkv, int64_t N, int D, double scale,
                       const int32_t *anchor_idx, int Hkv_a, int64_t kk,
                       const int32_t *qmap, double *o_out)
{
    if (check_shape(B, Hq, Hkv, N, D) || Hkv_a <= 0 || kk <= 0) return ORC_BAD_ARG;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    for (int h = 0; h < Hq; ++h)
        if (qmap[h] < 0 || qmap[h] >= Hkv_a) return ORC_BAD_ARG;
    for (int64_t i = 0; i < (int64_t)B * Hkv_a * kk; ++i)
        if (anchor_idx[i] < 0 || anchor_idx[i] >= N) return ORC_BAD_INDEX;
    const int G = Hq / Hkv;
    int status = ORC_OK;
#pragma omp parallel
    {
        double *sel = (double *)malloc((size_t)kk * sizeof(double));
        int64_t *keys = (int64_t *)malloc((size_t)kk * sizeof(int64_t));
        if (!sel || !keys) {
#pragma omp atomic write
            status = ORC_NOMEM;
        } else {
#pragma omp for schedule(dynamic)
            for (int64_t u = 0; u < (int64_t)B * Hq; ++u) {
                int64_t b = u / Hq, h = u % Hq, g = h / G;
                const int32_t *S = anchor_idx + (b * Hkv_a + qmap[h]) * kk;
                const float *kb = k + (b * Hkv + g) * N * D;
                const float *vb = v + (b * Hkv + g) * N * D;
                const float *qh = q + (b * Hq + h) * D;
                for (int64_t a = 0; a < kk; ++a) keys[a] = S[a];
                for (int64_t a = 0; a < kk; ++a) sel[a] = dot_scaled(qh, kb + keys[a] * D, D, scale);
                weighted_rows(sel, keys, kk, vb, D, o_out + (b * Hq + h) * D);
            }
        }
        free(sel); free(keys);
    }
    return status;
}

/* Reuse layer: attention over the anchor's index set of the mapped KV head.
 * anchor_idx [B, Hkv_a, kk]; head_map [Hkv] with values in [0, Hkv_a): every
 * query head of KV head g reads set head_map[g]. */
int orc_decode_reuse(const float *q, const float *k, const float *v,
                     int B, int Hq, int Hkv, int64_t N, int D, double scale,
                     const int32_t *anchor_idx, int Hkv_a, int64_t kk,
                     const int32_t *head_map, double *o_out)
{
    if (check_shape(B, Hq, Hkv, N, D)) return ORC_BAD_ARG;
    const int G = Hq / Hkv;
    int32_t *qmap = (int32_t *)malloc((size_t)Hq * sizeof(int32_t));
    if (!qmap) return ORC_NOMEM;
    for (int h = 0; h < Hq; ++h) qmap[h] = head_map[h / G];
    int st = orc_decode_reuse_q(q, k, v, B, Hq, Hkv, N, D, scale, anchor_idx, Hkv_a, kk, qmap, o_out);
    free(qmap);
    return st;
}

/* ------------------------------------------------------------------ */
/* prefill                                                             */
/* ------------------------------------------------------------------ */
/*
 * Layouts. The oracle works on a tile range [t0, t1) so that single tiles of
 * long prompts can be checked:
 *   q      [B, Hq, R, D]  holding query rows [tile*t0, tile*t0 + R)
 *   k, v   [B, Hkv, N, D] the whole prompt
 *   o_out  [B, Hq, R, D]
 *   idx    [B, Hkv, off[t1] - off[t0]]  index sets of tiles t0..t1-1 (CSR,
 *          offsets from orc_prefill_offsets, rebased to off[t0])
 * where R = min(N, tile*t1) - tile*t0.
 */

static int64_t range_rows(int64_t N, int32_t tile, int64_t t0, int64_t t1)
{
    int64_t end = t1 * tile < N ? t1 * tile : N;
    return end - t0 * tile;
}

/* Pooled score of one unit over keys [0, min(N, tile*(t+1))): over the query
 * heads of KV heads [g0, g0 + ng) and the tile's rows i >= j, the sum (op 0)
 * or the maximum (op 1) of the row's softmax probability of key j (softmax
 * over the causal row j' <= i). `rowbuf` holds at least N doubles. */
static void prefill_pool_unit(const float *q, const float *k, int B, int Hq, int Hkv,
                              int64_t N, int D, int32_t tile, double scale,
                              int64_t t0, int64_t R, int64_t b, int64_t t, int64_t g0, int ng,
                              int op, double *P, double *rowbuf)
{
    (void)B;
    const int G = Hq / Hkv;
    const int64_t i0 = t * tile;
    const int64_t i1 = (i0 + tile < N) ? i0 + tile : N;
    for (int64_t j = 0; j < i1; ++j) P[j] = 0.0;
    for (int64_t g = g0; g < g0 + ng; ++g) {
        const float *kb = k + (b * Hkv + g) * N * D;
        for (int r = 0; r < G; ++r) {
            const int64_t h = g * G + r;
            for (int64_t i = i0; i < i1; ++i) {
                const float *qi = q + ((b * Hq + h) * R + (i - t0 * tile)) * D;
                double m = -INFINITY;
                for (int64_t j = 0; j <= i; ++j) {
                    rowbuf[j] = dot_scaled(qi, kb + j * D, D, scale);
                    if (rowbuf[j] > m) m = rowbuf[j];
                }
                double l = 0.0;
                for (int64_t j = 0; j <= i; ++j) l += exp(rowbuf[j] - m);
                for (int64_t j = 0; j <= i; ++j) {
                    const double p = exp(rowbuf[j] - m) / l;
                    P[j] = op ? (p > P[j] ? p : P[j]) : P[j] + p;
                }
            }
        }
    }
}

/* Output rows of query head h of tile t: each row attends over the index set
 * S (n_sel keys, all before the tile) plus its causal diagonal keys [i0, i],
 * with the K and V of h's KV head. */
static void prefill_output_head(const float *q, const float *k, const float *v,
                                int Hq, int Hkv, int64_t N, int D, int32_t tile, double scale,
                                int64_t t0, int64_t R, int64_t b, int64_t t, int64_t h,
                                const int32_t *S, int64_t n_sel,
                                double *o_out, double *logit, int64_t *keys)
{
    const int G = Hq / Hkv;
    const int64_t g = h / G;
    const int64_t i0 = t * tile;
    const int64_t i1 = (i0 + tile < N) ? i0 + tile : N;
    const float *kb = k + (b * Hkv + g) * N * D;
    const float *vb = v + (b * Hkv + g) * N * D;
    {
        for (int64_t i = i0; i < i1; ++i) {
            const float *qi = q + ((b * Hq + h) * R + (i - t0 * tile)) * D;
            int64_t n = 0;
            for (int64_t a = 0; a < n_sel; ++a) keys[n++] = S[a];
            for (int64_t j = i0; j <= i; ++j) keys[n++] = j;
            for (int64_t a = 0; a < n; ++a) logit[a] = dot_scaled(qi, kb + keys[a] * D, D, scale);
            weighted_rows(logit, keys, n, vb, D, o_out + ((b * Hq + h) * R + (i - t0 * tile)) * D);
        }
    }
}

/* Output rows of one (b, t, g) unit: every query head of KV head g over S. */
static void prefill_output_unit(const float *q, const float *k, const float *v,
                                int Hq, int Hkv, int64_t N, int D, int32_t tile, double scale,
                                int64_t t0, int64_t R, int64_t b, int64_t t, int64_t g,
                                const int32_t *S, int64_t n_sel,
                                double *o_out, double *logit, int64_t *keys)
{
    const int G = Hq / Hkv;
    for (int r = 0; r < G; ++r)
        prefill_output_head(q, k, v, Hq, Hkv, N, D, tile, scale, t0, R, b, t, g * G + r, S, n_sel,
                            o_out, logit, keys);
}

/* Pooled scores of a single unit, for checking: P_out has
 * min(N, tile*(t+1)) entries (selection candidates are the first tile*t).
 * Unit (b, t, gs): scope 0 pools KV head gs's group, scope 1 all heads
 * (gs = 0); op as in prefill_pool_unit. */
int orc_prefill_pooled_v(const float *q, const float *k, int B, int Hq, int Hkv, int64_t N,
                         int D, int32_t tile, double scale, int64_t t0, int64_t t1,
                         int scope, int op, int64_t b, int64_t t, int64_t gs, double *P_out)
{
    if (check_shape(B, Hq, Hkv, N, D) || tile <= 0) return ORC_BAD_ARG;
    if ((scope != 0 && scope != 1) || (op != 0 && op != 1)) return ORC_BAD_ARG;
    const int Hs = scope ? 1 : Hkv;
    int64_t T = (N + tile - 1) / tile;
    if (t0 < 0 || t1 > T || t0 >= t1 || t < t0 || t >= t1 || b < 0 || b >= B || gs < 0 || gs >= Hs)
        return ORC_BAD_ARG;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    double *rowbuf = (double *)malloc((size_t)N * sizeof(double));
    if (!rowbuf) return ORC_NOMEM;
    prefill_pool_unit(q, k, B, Hq, Hkv, N, D, tile, scale, t0, range_rows(N, tile, t0, t1),
                      b, t, scope ? 0 : gs, scope ? Hkv : 1, op, P_out, rowbuf);
    free(rowbuf);
    return ORC_OK;
}

int orc_prefill_pooled(const float *q, const float *k, int B, int Hq, int Hkv, int64_t N,
                       int D, int32_t tile, double scale, int64_t t0, int64_t t1,
                       int64_t b, int64_t t, int64_t g, double *P_out)
{
    return orc_prefill_pooled_v(q, k, B, Hq, Hkv, N, D, tile, scale, t0, t1, 0, 0, b, t, g, P_out);
}

/* Prefill anchor layer over tiles [t0, t1): pooled tile scores, exact Top-k_t
 * per (b, t, set), and the output rows. Pooling variants as in
 * orc_decode_anchor_v: scope 0 gives one set per (b, t, KV head), scope 1 one
 * set per (b, t) pooled over all query heads and shared by every KV head
 * (idx_out [B, Hs, off[t1] - off[t0]], Hs = scope ? 1 : Hkv); op 0 sums,
 * op 1 takes the maximum over the pooled heads and rows. */
int orc_prefill_anchor_v(const float *q, const float *k, const float *v,
                         int B, int Hq, int Hkv, int64_t N, int D, int32_t tile, int32_t pct,
                         double scale, int64_t t0, int64_t t1, int scope, int op,
                         int32_t *idx_out, double *o_out)
{
    if (check_shape(B, Hq, Hkv, N, D) || tile <= 0 || pct < 1 || pct > 100) return ORC_BAD_ARG;
    if ((scope != 0 && scope != 1) || (op != 0 && op != 1)) return ORC_BAD_ARG;
    const int Hs = scope ? 1 : Hkv;
    const int ng = scope ? Hkv : 1;
    const int64_t T = (N + tile - 1) / tile;
    if (t0 < 0 || t1 > T || t0 >= t1) return ORC_BAD_ARG;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    int64_t *off = (int64_t *)malloc((size_t)(T + 1) * sizeof(int64_t));
    if (!off) return ORC_NOMEM;
    orc_prefill_offsets(N, tile, pct, off);
    const int64_t R = range_rows(N, tile, t0, t1);
    const int64_t tot = off[t1] - off[t0];
    const int64_t n_units = (int64_t)B * (t1 - t0) * Hs;
    int status = ORC_OK;
#pragma omp parallel
    {
        double *P = (double *)malloc((size_t)N * sizeof(double));
        double *rowbuf = (double *)malloc((size_t)(N + tile) * sizeof(double));
        int64_t *keys = (int64_t *)malloc((size_t)(N + tile) * sizeof(int64_t));
        if (!P || !rowbuf || !keys) {
#pragma omp atomic write
            status = ORC_NOMEM;
        } else {
            /* big tiles first: better balance */
#pragma omp for schedule(dynamic)
            for (int64_t u = 0; u < n_units; ++u) {
                int64_t tt = (t1 - 1) - (u / ((int64_t)B * Hs));
                int64_t rem = u % ((int64_t)B * Hs);
                int64_t b = rem / Hs, gs = rem % Hs;
                int64_t kt = off[tt + 1] - off[tt];
                int32_t *S = idx_out + (b * Hs + gs) * tot + (off[tt] - off[t0]);
                prefill_pool_unit(q, k, B, Hq, Hkv, N, D, tile, scale, t0, R, b, tt, gs * ng, ng, op,
                                  P, rowbuf);
                if (select_topk(P, tt * (int64_t)tile, kt, S) != ORC_OK) {
#pragma omp atomic write
                    status = ORC_NOMEM;
                    continue;
                }
                for (int64_t g = gs * ng; g < gs * ng + ng; ++g)
                    prefill_output_unit(q, k, v, Hq, Hkv, N, D, tile, scale, t0, R, b, tt, g,
                                        S, kt, o_out, rowbuf, keys);
            }
        }
        free(P); free(rowbuf); free(keys);
    }
    free(off);
    return status;
}

/* The method's own prefill anchor layer: per KV-head group, sum pooling. */
int orc_prefill_anchor(const float *q, const float *k, const float *v,
                       int B, int Hq, int Hkv, int64_t N, int D, int32_t tile, int32_t pct,
                       double scale, int64_t t0, int64_t t1,
                       int32_t *idx_out, double *o_out)
{
    return orc_prefill_anchor_v(q, k, v, B, Hq, Hkv, N, D, tile, pct, scale, t0, t1, 0, 0,
                                idx_out, o_out);
}

/* Prefill reuse layer over tiles [t0, t1) with one anchor set per query head:
 * tile t of query head h attends over the anchor's set of tile t for anchor
 * KV head qmap[h] (qmap [Hq]) plus the causal diagonal. anchor_idx is the
 * anchor's full CSR array [B, Hkv_a, total]. */
int orc_prefill_reuse_q(const float *q, const float *k, const float *v,
                        int B, int Hq, int Hkv, int64_t N, int D, int32_t tile, int32_t pct,
                        double scale, int64_t t0, int64_t t1,
                        const int32_t *anchor_idx, int Hkv_a, const int32_t *qmap,
                        double *o_out)
{
    if (check_shape(B, Hq, Hkv, N, D) || tile <= 0 || pct < 1 || pct > 100 || Hkv_a <= 0)
        return ORC_BAD_ARG;
    const int64_t T = (N + tile - 1) / tile;
    if (t0 < 0 || t1 > T || t0 >= t1) return ORC_BAD_ARG;
    for (int h = 0; h < Hq; ++h)
        if (qmap[h] < 0 || qmap[h] >= Hkv_a) return ORC_BAD_ARG;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    int64_t *off = (int64_t *)malloc((size_t)(T + 1) * sizeof(int64_t));
    if (!off) return ORC_NOMEM;
    const int64_t total = orc_prefill_offsets(N, tile, pct, off);
    /* every index of tile t must lie before the tile */
    for (int64_t b = 0; b < B; ++b)
        for (int64_t ga = 0; ga < Hkv_a; ++ga)
            for (int64_t t = t0; t < t1; ++t)
                for (int64_t a = off[t]; a < off[t + 1]; ++a) {
                    int32_t j = anchor_idx[(b * Hkv_a + ga) * total + a];
                    if (j < 0 || j >= t * tile) { free(off); return ORC_BAD_INDEX; }
                }
    const int64_t R = range_rows(N, tile, t0, t1);
    const int64_t n_units = (int64_t)B * (t1 - t0) * Hq;
    int status = ORC_OK;
#pragma omp parallel
    {
        double *rowbuf = (double *)malloc((size_t)(N + tile) * sizeof(double));
        int64_t *keys = (int64_t *)malloc((size_t)(N + tile) * sizeof(int64_t));
        if (!rowbuf || !keys) {
#pragma omp atomic write
            status = ORC_NOMEM;
        } else {
#pragma omp for schedule(dynamic)
            for (int64_t u = 0; u < n_units; ++u) {
                int64_t tt = (t1 - 1) - (u / ((int64_t)B * Hq));
                int64_t rem = u % ((int64_t)B * Hq);
                int64_t b = rem / Hq, h = rem % Hq;
                const int32_t *S = anchor_idx + (b * Hkv_a + qmap[h]) * total + off[tt];
                prefill_output_head(q, k, v, Hq, Hkv, N, D, tile, scale, t0, R, b, tt, h,
                                    S, off[tt + 1] - off[tt], o_out, rowbuf, keys);
            }
        }
        free(rowbuf); free(keys);
    }
    free(off);
    return status;
}

/* Prefill reuse layer over tiles [t0, t1): tile t of KV head g attends over
 * the anchor's set of tile t for anchor KV head head_map[g] plus the causal
 * diagonal. anchor_idx is the anchor's full CSR array [B, Hkv_a, total]. */
int orc_prefill_reuse(const float *q, const float *k, const float *v,
                      int B, int Hq, int Hkv, int64_t N, int D, int32_t tile, int32_t pct,
                      double scale, int64_t t0, int64_t t1,
                      const int32_t *anchor_idx, int Hkv_a, const int32_t *head_map,
                      double *o_out)
{
    if (check_shape(B, Hq, Hkv, N, D)) return ORC_BAD_ARG;
    const int G = Hq / Hkv;
    int32_t *qmap = (int32_t *)malloc((size_t)Hq * sizeof(int32_t));
    if (!qmap) return ORC_NOMEM;
    for (int h = 0; h < Hq; ++h) qmap[h] = head_map[h / G];
    int st = orc_prefill_reuse_q(q, k, v, B, Hq, Hkv, N, D, tile, pct, scale, t0, t1,
                                 anchor_idx, Hkv_a, qmap, o_out);
    free(qmap);
    return st;
}

/* ------------------------------------------------------------------ */
/* proposal-refined reuse (decode)                                     */
/* ------------------------------------------------------------------ */

/* Refined layer of proposal-refined reuse (the Prism Attention page,
 * thelatestinai.com/papers/2610.22985: a proposal layer exports a pool of
 * rho * kappa candidate keys; each refined layer selects its own kappa keys
 * within the pool). Reading taken here: KV head g's pool is
 * pool_idx[b, head_map[g], :] (n_pool keys, ascending); each query head of
 * the group gets its softmax over the pool's keys with this layer's q and K;
 * the probabilities are summed over the group; the exact Top-kappa within the
 * pool (ties to the lower key) is the refined set, written to idx_out[b, g, :]
 * ascending; each head attends over it. pool_idx [B, Hkv_p, n_pool];
 * idx_out [B, Hkv, kappa]; o_out [B, Hq, D]. */
int orc_decode_refine(const float *q, const float *k, const float *v,
                      int B, int Hq, int Hkv, int64_t N, int D, double scale,
                      const int32_t *pool_idx, int Hkv_p, int64_t n_pool,
                      const int32_t *head_map, int64_t kappa, int32_t *idx_out, double *o_out)
{
    if (check_shape(B, Hq, Hkv, N, D) || Hkv_p <= 0 || n_pool <= 0 || kappa <= 0 || kappa > n_pool)
        return ORC_BAD_ARG;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    for (int g = 0; g < Hkv; ++g)
        if (head_map[g] < 0 || head_map[g] >= Hkv_p) return ORC_BAD_ARG;
    for (int64_t i = 0; i < (int64_t)B * Hkv_p * n_pool; ++i)
        if (pool_idx[i] < 0 || pool_idx[i] >= N) return ORC_BAD_INDEX;
    const int G = Hq / Hkv;
    int status = ORC_OK;
#pragma omp parallel
    {
        double *s = (double *)malloc((size_t)G * n_pool * sizeof(double));
        double *P = (double *)malloc((size_t)n_pool * sizeof(double));
        int32_t *pos = (int32_t *)malloc((size_t)kappa * sizeof(int32_t));
        double *sel = (double *)malloc((size_t)kappa * sizeof(double));
        int64_t *keys = (int64_t *)malloc((size_t)kappa * sizeof(int64_t));
        if (!s || !P || !pos || !sel || !keys) {
#pragma omp atomic write
            status = ORC_NOMEM;
        } else {
#pragma omp for schedule(dynamic)
            for (int64_t u = 0; u < (int64_t)B * Hkv; ++u) {
                int64_t b = u / Hkv, g = u % Hkv;
                const int32_t *pool = pool_idx + (b * Hkv_p + head_map[g]) * n_pool;
                const float *kb = k + (b * Hkv + g) * N * D;
                const float *vb = v + (b * Hkv + g) * N * D;
                /* 1. each head's softmax over the pool's keys */
                for (int64_t a = 0; a < n_pool; ++a) P[a] = 0.0;
                for (int r = 0; r < G; ++r) {
                    const float *qh = q + (b * Hq + g * G + r) * D;
                    double m = -INFINITY;
                    for (int64_t a = 0; a < n_pool; ++a) {
                        s[r * n_pool + a] = dot_scaled(qh, kb + (int64_t)pool[a] * D, D, scale);
                        if (s[r * n_pool + a] > m) m = s[r * n_pool + a];
                    }
                    double l = 0.0;
                    for (int64_t a = 0; a < n_pool; ++a) l += exp(s[r * n_pool + a] - m);
                    /* 2. summed over the group's heads */
                    for (int64_t a = 0; a < n_pool; ++a) P[a] += exp(s[r * n_pool + a] - m) / l;
                }
                /* 3. exact Top-kappa within the pool: positions in the pool are
                 *    in key order, so the lower position is the lower key */
                if (select_topk(P, n_pool, kappa, pos) != ORC_OK) {
#pragma omp atomic write
                    status = ORC_NOMEM;
                    continue;
                }
                int32_t *S = idx_out + u * kappa;
                for (int64_t a = 0; a < kappa; ++a) { S[a] = pool[pos[a]]; keys[a] = S[a]; }
                /* 4. attention over the refined set, per head */
                for (int r = 0; r < G; ++r) {
                    for (int64_t a = 0; a < kappa; ++a) sel[a] = s[r * n_pool + pos[a]];
                    weighted_rows(sel, keys, kappa, vb, D, o_out + (b * Hq + g * G + r) * D);
                }
            }
        }
        free(s); free(P); free(pos); free(sel); free(keys);
    }
    return status;
}
