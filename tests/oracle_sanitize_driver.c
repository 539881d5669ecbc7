/*
 * oracle_sanitize_driver.c -- runs every entry point of the fp64 oracle on a
 * tiny paged cache so the oracle can be built and exercised under the host
 * address and undefined-behaviour sanitizers (tests/test_oracle_sanitize.py).
 *
 * Test infrastructure: links the oracle only.  Inputs come from a small
 * linear congruential generator; a partial last page, a permuted page table
 * and a pool with unused pages are included.  Besides running clean under the
 * sanitizers, it checks a few identities the oracle must satisfy on any input:
 * a budget covering every page reproduces dense attention, a page's
 * from-scratch bounds equal that page's row of the whole-request bounds, and
 * the selected pages are the k best under (score desc, page asc).
 * Exit status 0 on success.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "quest_oracle.h"

static uint64_t rng = 0x9e3779b97f4a7c15ull;

static double uniform(void) {            /* in [-1, 1) */
  rng = rng * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(rng >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

static uint16_t to_bf16(float f) {       /* round to nearest even */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static int fail(const char *what) {
  fprintf(stderr, "oracle driver: %s\n", what);
  return 1;
}

static int run(int elem) {
  const int Hq = 4, Hkv = 2, D = 16, P = 4, ctx = 13, pool = 6;
  const int n = (ctx + P - 1) / P;     /* 4 logical pages, the last one partial */
  const int es = elem == QO_BF16 ? 2 : 4;
  qo_shape s = {elem, Hq, Hkv, D, P, pool};
  const int32_t pt[4] = {5, 0, 3, 1}; /* physical pages 2 and 4 unused */
  void *kc = calloc((size_t)pool * Hkv * P * D, es);
  void *vc = calloc((size_t)pool * Hkv * D * P, es);
  void *kn = malloc((size_t)ctx * Hkv * D * es);
  void *vn = malloc((size_t)ctx * Hkv * D * es);
  void *q = malloc((size_t)Hq * D * es);
  double *bounds = malloc(sizeof(double) * n * Hkv * 2 * D);
  double *bj = malloc(sizeof(double) * Hkv * 2 * D);
  double *scores = malloc(sizeof(double) * Hkv * n);
  double *hscores = malloc(sizeof(double) * Hq * n);
  double *out = malloc(sizeof(double) * Hq * D), *dense = malloc(sizeof(double) * Hq * D);
  int32_t sel[8 * 4], nsel[8];
  int bad = 0;
  for (int i = 0; i < ctx * Hkv * D; ++i) {
    const float kf = (float)uniform(), vf = (float)uniform();
    if (elem == QO_BF16) {
      ((uint16_t *)kn)[i] = to_bf16(kf);
      ((uint16_t *)vn)[i] = to_bf16(vf);
    } else {
      ((float *)kn)[i] = kf;
      ((float *)vn)[i] = vf;
    }
  }
  for (int i = 0; i < Hq * D; ++i) {
    const float qf = (float)uniform();
    if (elem == QO_BF16) ((uint16_t *)q)[i] = to_bf16(qf);
    else ((float *)q)[i] = qf;
  }
  /* store the prompt in two calls (the second starts mid-page) */
  qo_store_tokens(&s, 6, kn, vn, 0, pt, kc, vc);
  qo_store_tokens(&s, ctx - 6, (const char *)kn + (size_t)6 * Hkv * D * es,
                  (const char *)vn + (size_t)6 * Hkv * D * es, 6, pt, kc, vc);
  qo_request_bounds(&s, kc, pt, ctx, bounds);
  for (int j = 0; j < n; ++j) {
    qo_page_bounds(&s, kc, pt, ctx, j, bj);
    if (memcmp(bj, bounds + (size_t)j * Hkv * 2 * D, sizeof(double) * Hkv * 2 * D) != 0)
      bad |= fail("page bounds differ from the request's row");
  }
  for (int reduce = QO_REDUCE_MAX; reduce <= QO_REDUCE_SUM; ++reduce)
    qo_request_scores(&s, q, bounds, n, reduce, scores);
  qo_request_scores(&s, q, bounds, n, QO_REDUCE_MAX, scores);
  qo_request_head_scores(&s, q, bounds, n, hscores);
  const int k = qo_pages_for_budget(8, ctx, P);
  if (k != 2) bad |= fail("budget of 8 tokens at page 4 is not 2 pages");
  for (int g = 0; g < Hkv; ++g) {
    qo_select(scores + (size_t)g * n, n, k, sel + g * 4);
    nsel[g] = k;
    /* every unselected page is below (or tied above) every selected one */
    for (int a = 0; a < n; ++a) {
      int picked = 0;
      for (int x = 0; x < k; ++x) picked |= sel[g * 4 + x] == a;
      if (picked) continue;
      for (int x = 0; x < k; ++x) {
        const int b = sel[g * 4 + x];
        const double sa = scores[(size_t)g * n + a], sb = scores[(size_t)g * n + b];
        if (sa > sb || (sa == sb && a < b)) bad |= fail("selection is not the top k");
      }
    }
    for (int x = 1; x < k; ++x)
      if (sel[g * 4 + x] <= sel[g * 4 + x - 1]) bad |= fail("selection not ascending");
    qo_select_forced(scores + (size_t)g * n, n, 3, 1, 1, sel + g * 4);
  }
  for (int g = 0; g < Hkv; ++g) {
    qo_select(scores + (size_t)g * n, n, k, sel + g * 4);
    nsel[g] = k;
  }
  const double scale = 1.0 / sqrt((double)D);
  qo_request_attend(&s, q, kc, vc, pt, ctx, sel, nsel, 4, scale, out);
  int32_t hsel[4 * 4], hn[4];
  for (int h = 0; h < Hq; ++h) {
    qo_select(hscores + (size_t)h * n, n, k, hsel + h * 4);
    hn[h] = k;
  }
  qo_request_attend_heads(&s, q, kc, vc, pt, ctx, hsel, hn, 4, scale, out);
  /* every page selected: equals dense attention */
  for (int g = 0; g < Hkv; ++g) {
    for (int j = 0; j < n; ++j) sel[g * 4 + j] = j;
    nsel[g] = n;
  }
  qo_request_attend(&s, q, kc, vc, pt, ctx, sel, nsel, 4, scale, out);
  qo_request_dense(&s, q, kc, vc, pt, ctx, scale, dense);
  for (int i = 0; i < Hq * D; ++i)
    if (fabs(out[i] - dense[i]) > 1e-12) bad |= fail("all pages selected differs from dense");
  free(kc); free(vc); free(kn); free(vn); free(q); free(bounds); free(bj);
  free(scores); free(hscores); free(out); free(dense);
  return bad;
}

int main(void) {
  const int bad = run(QO_F32) | run(QO_BF16);
  if (!bad) printf("oracle driver ok\n");
  return bad;
}
