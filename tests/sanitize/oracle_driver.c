/* Runs every entry point of the CPU oracle on small seeded inputs (ragged
 * tiles, N = 1, k = N, every pooling variant, sub-ranges of tiles, bad
 * arguments), built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py. Checks the invariants that hold at any size: the
 * pooled mass, sets inside their candidate ranges and ascending, identical
 * results for a tile range and the full run. Exit status 0 = all passed. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t orc_topk_count(int64_t n, int32_t pct);
int64_t orc_prefill_offsets(int64_t n, int32_t tile, int32_t pct, int64_t *offsets);
int orc_dense_attention(const float *q, const float *k, const float *v, double *o, int B, int Hq, int Hkv,
                        int64_t Nq, int64_t Nk, int D, int causal, double scale);
int orc_decode_anchor_v(const float *q, const float *k, const float *v, int B, int Hq, int Hkv, int64_t N, int D,
                        int32_t pct, double scale, int scope, int op, int32_t *idx_out, double *o_out,
                        double *pooled_out);
int orc_decode_reuse(const float *q, const float *k, const float *v, int B, int Hq, int Hkv, int64_t N, int D,
                     double scale, const int32_t *anchor_idx, int Hkv_a, int64_t kk, const int32_t *head_map,
                     double *o_out);
int orc_decode_reuse_q(const float *q, const float *k, const float *v, int B, int Hq, int Hkv, int64_t N, int D,
                       double scale, const int32_t *anchor_idx, int Hkv_a, int64_t kk, const int32_t *qmap,
                       double *o_out);
int orc_decode_refine(const float *q, const float *k, const float *v, int B, int Hq, int Hkv, int64_t N, int D,
                      double scale, const int32_t *pool_idx, int Hkv_p, int64_t n_pool, const int32_t *head_map,
                      int64_t kappa, int32_t *idx_out, double *o_out);
int orc_prefill_pooled_v(const float *q, const float *k, int B, int Hq, int Hkv, int64_t N, int D, int32_t tile,
                         double scale, int64_t t0, int64_t t1, int scope, int op, int64_t b, int64_t t, int64_t gs,
                         double *P_out);
int orc_prefill_anchor_v(const float *q, const float *k, const float *v, int B, int Hq, int Hkv, int64_t N, int D,
                         int32_t tile, int32_t pct, double scale, int64_t t0, int64_t t1, int scope, int op,
                         int32_t *idx_out, double *o_out);
int orc_prefill_reuse(const float *q, const float *k, const float *v, int B, int Hq, int Hkv, int64_t N, int D,
                      int32_t tile, int32_t pct, double scale, int64_t t0, int64_t t1, const int32_t *anchor_idx,
                      int Hkv_a, const int32_t *head_map, double *o_out);
int orc_prefill_reuse_q(const float *q, const float *k, const float *v, int B, int Hq, int Hkv, int64_t N, int D,
                        int32_t tile, int32_t pct, double scale, int64_t t0, int64_t t1, const int32_t *anchor_idx,
                        int Hkv_a, const int32_t *qmap, double *o_out);

static int failures = 0;
#define CHECK(c)                                                         \
  do {                                                                   \
    if (!(c)) {                                                          \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static float urand(void) {
  rng = rng * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((rng >> 40) * (1.0 / 16777216.0)) * 2.f - 1.f;
}
static float *rand_buf(size_t n) {
  float *p = (float *)malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = urand();
  return p;
}
static void check_sets(const int32_t *s, int64_t n, int64_t lim) {
  for (int64_t i = 0; i < n; ++i) {
    CHECK(s[i] >= 0 && s[i] < lim);
    if (i) CHECK(s[i] > s[i - 1]);
  }
}

static void decode_cases(int B, int Hq, int Hkv, int64_t N, int D) {
  const int G = Hq / Hkv;
  float *q = rand_buf((size_t)B * Hq * D), *k = rand_buf((size_t)B * Hkv * N * D), *v = rand_buf((size_t)B * Hkv * N * D);
  for (int pct = 1; pct <= 100; pct += 33) {
    int64_t kk = orc_topk_count(N, pct);
    if (kk < 1) kk = 1;
    for (int scope = 0; scope <= 1; ++scope)
      for (int op = 0; op <= 1; ++op) {
        const int Hs = scope ? 1 : Hkv;
        int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * B * Hs * kk);
        double *o = (double *)malloc(sizeof(double) * B * Hq * D);
        double *P = (double *)malloc(sizeof(double) * B * Hs * N);
        CHECK(orc_decode_anchor_v(q, k, v, B, Hq, Hkv, N, D, pct, 0.0, scope, op, idx, o, P) == 0);
        for (int u = 0; u < B * Hs; ++u) {
          check_sets(idx + (int64_t)u * kk, kk, N);
          if (op == 0) {
            double m = 0;
            for (int64_t j = 0; j < N; ++j) m += P[(int64_t)u * N + j];
            CHECK(fabs(m - (scope ? Hq : G)) < 1e-9 * (scope ? Hq : G));
          }
        }
        for (int i = 0; i < B * Hq * D; ++i) CHECK(isfinite(o[i]));
        if (scope == 0 && op == 0) {
          int32_t *hm = (int32_t *)malloc(sizeof(int32_t) * Hkv);
          int32_t *qm = (int32_t *)malloc(sizeof(int32_t) * Hq);
          for (int g = 0; g < Hkv; ++g) hm[g] = Hkv - 1 - g;
          for (int h = 0; h < Hq; ++h) qm[h] = hm[h / G];
          double *o1 = (double *)malloc(sizeof(double) * B * Hq * D), *o2 = (double *)malloc(sizeof(double) * B * Hq * D);
          CHECK(orc_decode_reuse(q, k, v, B, Hq, Hkv, N, D, 0.0, idx, Hkv, kk, hm, o1) == 0);
          CHECK(orc_decode_reuse_q(q, k, v, B, Hq, Hkv, N, D, 0.0, idx, Hkv, kk, qm, o2) == 0);
          CHECK(memcmp(o1, o2, sizeof(double) * B * Hq * D) == 0);
          hm[0] = Hkv;   /* out of range: rejected */
          CHECK(orc_decode_reuse(q, k, v, B, Hq, Hkv, N, D, 0.0, idx, Hkv, kk, hm, o1) != 0);
          /* refined layer over the set as a pool, kappa = half of it */
          int64_t kappa = kk > 1 ? kk / 2 : 1;
          int32_t *ridx = (int32_t *)malloc(sizeof(int32_t) * B * Hkv * kappa);
          hm[0] = 0;
          CHECK(orc_decode_refine(q, k, v, B, Hq, Hkv, N, D, 0.0, idx, Hkv, kk, hm, kappa, ridx, o1) == 0);
          check_sets(ridx, kappa, N);
          free(ridx); free(hm); free(qm); free(o1); free(o2);
        }
        free(idx); free(o); free(P);
      }
  }
  CHECK(orc_decode_anchor_v(q, k, v, B, Hq, Hkv, N, D, 0, 0.0, 0, 0, NULL, NULL, NULL) != 0);
  free(q); free(k); free(v);
}

static void prefill_cases(int B, int Hq, int Hkv, int64_t N, int D) {
  const int tile = 32, pct = 25;
  const int64_t T = (N + tile - 1) / tile;
  int64_t *off = (int64_t *)malloc(sizeof(int64_t) * (T + 1));
  const int64_t total = orc_prefill_offsets(N, tile, pct, off);
  CHECK(off[0] == 0 && off[T] == total);
  float *q = rand_buf((size_t)B * Hq * N * D), *k = rand_buf((size_t)B * Hkv * N * D), *v = rand_buf((size_t)B * Hkv * N * D);
  double *o = (double *)malloc(sizeof(double) * B * Hq * N * D);
  double *od = (double *)malloc(sizeof(double) * B * Hq * N * D);
  CHECK(orc_dense_attention(q, k, v, od, B, Hq, Hkv, N, N, D, 1, 0.0) == 0);
  for (int scope = 0; scope <= 1; ++scope)
    for (int op = 0; op <= 1; ++op) {
      const int Hs = scope ? 1 : Hkv;
      int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (B * Hs * total + 1));
      CHECK(orc_prefill_anchor_v(q, k, v, B, Hq, Hkv, N, D, tile, pct, 0.0, 0, T, scope, op, idx, o) == 0);
      for (int u = 0; u < B * Hs; ++u)
        for (int64_t t = 0; t < T; ++t) check_sets(idx + u * total + off[t], off[t + 1] - off[t], tile * t);
      /* the last tile alone gives the same set and rows */
      if (T > 1) {
        const int64_t R = N - tile * (T - 1), nt = off[T] - off[T - 1];
        float *qr = (float *)malloc(sizeof(float) * B * Hq * R * D);
        for (int bh = 0; bh < B * Hq; ++bh)
          memcpy(qr + (int64_t)bh * R * D, q + ((int64_t)bh * N + tile * (T - 1)) * D, sizeof(float) * R * D);
        int32_t *idx1 = (int32_t *)malloc(sizeof(int32_t) * (B * Hs * nt + 1));
        double *o1 = (double *)malloc(sizeof(double) * B * Hq * R * D);
        CHECK(orc_prefill_anchor_v(qr, k, v, B, Hq, Hkv, N, D, tile, pct, 0.0, T - 1, T, scope, op, idx1, o1) == 0);
        for (int u = 0; u < B * Hs; ++u)
          CHECK(memcmp(idx1 + u * nt, idx + u * total + off[T - 1], sizeof(int32_t) * nt) == 0);
        double *P = (double *)malloc(sizeof(double) * N);
        CHECK(orc_prefill_pooled_v(qr, k, B, Hq, Hkv, N, D, tile, 0.0, T - 1, T, scope, op, B - 1, T - 1, Hs - 1, P) == 0);
        if (op == 0) {
          double m = 0;
          for (int64_t j = 0; j < N; ++j) m += P[j];
          CHECK(fabs(m - (double)R * (scope ? Hq : Hq / Hkv)) < 1e-9 * m);
        }
        free(P); free(qr); free(idx1); free(o1);
      }
      if (scope == 0 && op == 0) {
        int32_t *hm = (int32_t *)malloc(sizeof(int32_t) * Hkv), *qm = (int32_t *)malloc(sizeof(int32_t) * Hq);
        for (int g = 0; g < Hkv; ++g) hm[g] = g;
        for (int h = 0; h < Hq; ++h) qm[h] = h / (Hq / Hkv);
        double *o2 = (double *)malloc(sizeof(double) * B * Hq * N * D), *o3 = (double *)malloc(sizeof(double) * B * Hq * N * D);
        CHECK(orc_prefill_reuse(q, k, v, B, Hq, Hkv, N, D, tile, pct, 0.0, 0, T, idx, Hkv, hm, o2) == 0);
        CHECK(orc_prefill_reuse_q(q, k, v, B, Hq, Hkv, N, D, tile, pct, 0.0, 0, T, idx, Hkv, qm, o3) == 0);
        /* identity reuse of the anchor's own sets reproduces its output */
        for (int64_t i = 0; i < (int64_t)B * Hq * N * D; ++i) CHECK(fabs(o2[i] - o[i]) < 1e-9 && o2[i] == o3[i]);
        free(hm); free(qm); free(o2); free(o3);
      }
      free(idx);
    }
  /* pct 100: the output is dense causal attention */
  int32_t *all = (int32_t *)malloc(sizeof(int32_t) * (B * Hkv * orc_prefill_offsets(N, tile, 100, NULL) + 1));
  CHECK(orc_prefill_anchor_v(q, k, v, B, Hq, Hkv, N, D, tile, 100, 0.0, 0, T, 0, 0, all, o) == 0);
  for (int64_t i = 0; i < (int64_t)B * Hq * N * D; ++i) CHECK(fabs(o[i] - od[i]) < 1e-9);
  CHECK(orc_prefill_anchor_v(q, k, v, B, Hq, Hkv, N, D, 16, 0, 0.0, 0, T, 0, 0, all, o) != 0);
  free(all); free(q); free(k); free(v); free(o); free(od); free(off);
}

int main(void) {
  for (int64_t n = 0; n < 300; ++n)
    for (int pct = 0; pct <= 101; ++pct) {
      const int64_t kk = orc_topk_count(n, pct);
      CHECK(kk >= 0 && kk <= (n > 0 ? n : 0));
    }
  decode_cases(2, 8, 2, 1, 16);
  decode_cases(2, 8, 2, 37, 16);
  decode_cases(1, 6, 3, 130, 8);
  prefill_cases(2, 8, 2, 100, 16);
  prefill_cases(1, 4, 4, 32, 8);
  prefill_cases(1, 2, 1, 70, 8);
  printf("oracle driver: %d failure(s)\n", failures);
  return failures ? 1 : 0;
}
