/*
 * quest_oracle.c -- plain, slow fp64 CPU oracle for Quest query-aware sparse
 * decode attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, helper or constant with the HIP
 * library.
 *
 * What it follows:
 *  - Sparse-vLLM skill page "add-sparse-method", Placement Rules items 2-4: the
 *    method keeps persistent per-page metadata, refreshes it after KV is
 *    written (on_kv_stored) and builds its decode view from the current layer's
 *    q (build_decode_view).
 *  - SparseEngine digest ("SparseEngine: Sparse-First Inference Engine"),
 *    Method key points: Quest registers query-relevant page selection; the
 *    cache manager owns KV representation, physical layout, position mapping
 *    and metadata; the attention view hands explicit KV to the backend.
 *  - The reading of Quest's arithmetic that this oracle and the library both
 *    follow (the pages name the method, its page metadata and its hooks, but
 *    never write its formulas): per page the elementwise min and max of its
 *    keys; per page the upper bound sum_d max(q_d*min_d, q_d*max_d) of q.k
 *    over any key inside that box; the top-k pages by that bound within a
 *    token budget; attention over them.
 *
 * Every step is written as its definition, in fp64, with loops in the order a
 * reader checks by eye.  Inputs are upcast exactly (bf16 and fp32 values are
 * exactly representable in fp64; the product of two of them is exact in fp64).
 * Readings taken where the pages are silent are marked READING.
 */
#include "quest_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- element access ---------------------------------------------------- */

/* Value of element i of an array of the given element type, exactly in fp64.
 * A bfloat16 pattern is the upper half of the binary32 with the same value. */
static double elem_value(const void *base, int64_t i, int32_t elem) {
  if (elem == QO_F32) return (double)((const float *)base)[i];
  uint32_t bits = ((uint32_t)((const uint16_t *)base)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static size_t elem_bytes(int32_t elem) { return elem == QO_F32 ? 4u : 2u; }

/* Offset of K[phys][g][slot][d] in the K pool (token-major page). */
static int64_t k_offset(const qo_shape *s, int64_t phys, int32_t g,
                        int32_t slot, int32_t d) {
  return ((phys * s->num_kv_heads + g) * s->page_size + slot) *
             (int64_t)s->head_dim + d;
}

/* Offset of V[phys][g][d][slot] in the V pool (dim-major page). */
static int64_t v_offset(const qo_shape *s, int64_t phys, int32_t g,
                        int32_t slot, int32_t d) {
  return ((phys * s->num_kv_heads + g) * s->head_dim + d) *
             (int64_t)s->page_size + slot;
}

static int32_t pages_of(int32_t ctx, int32_t page_size) {
  return ctx <= 0 ? 0 : (ctx + page_size - 1) / page_size;
}

/* ---- on_kv_stored: writing KV into the paged pool ----------------------- */

/* Position p of a request lives in logical page p / P at slot p mod P; the
 * page table maps the logical page to its physical page (the cache manager's
 * position mapping, SparseEngine digest, Method key points). */
void qo_store_tokens(const qo_shape *s, int32_t n_new, const void *k_new,
                     const void *v_new, int32_t pos0, const int32_t *pt_row,
                     void *k_cache, void *v_cache) {
  const size_t eb = elem_bytes(s->elem);
  const int32_t H = s->num_kv_heads, D = s->head_dim, P = s->page_size;
  for (int32_t i = 0; i < n_new; ++i) {
    const int32_t pos = pos0 + i;
    const int64_t phys = pt_row[pos / P];
    const int32_t slot = pos % P;
    for (int32_t g = 0; g < H; ++g) {
      for (int32_t d = 0; d < D; ++d) {
        const int64_t src = ((int64_t)i * H + g) * D + d;
        memcpy((char *)k_cache + k_offset(s, phys, g, slot, d) * eb,
               (const char *)k_new + src * eb, eb);
        memcpy((char *)v_cache + v_offset(s, phys, g, slot, d) * eb,
               (const char *)v_new + src * eb, eb);
      }
    }
  }
}

/* ---- page metadata ------------------------------------------------------ */

/* Quest page metadata: for logical page j, KV head g and channel d, the
 * smallest and the largest key value over the page's valid tokens, i.e. the
 * positions jP .. min((j+1)P, ctx)-1.  Slots at or past ctx never take part
 * (READING: a partial last page covers only its written tokens). */
void qo_page_bounds(const qo_shape *s, const void *k_cache,
                    const int32_t *pt_row, int32_t ctx, int32_t j,
                    double *bounds_j) {
  const int32_t H = s->num_kv_heads, D = s->head_dim, P = s->page_size;
  const int64_t phys = pt_row[j];
  const int32_t first = j * P;
  const int32_t last = (first + P < ctx ? first + P : ctx); /* exclusive */
  for (int32_t g = 0; g < H; ++g) {
    for (int32_t d = 0; d < D; ++d) {
      double lo = INFINITY, hi = -INFINITY;
      for (int32_t pos = first; pos < last; ++pos) {
        const double x =
            elem_value(k_cache, k_offset(s, phys, g, pos - first, d), s->elem);
        if (x < lo) lo = x;
        if (x > hi) hi = x;
      }
      bounds_j[((int64_t)g * 2 + 0) * D + d] = lo;
      bounds_j[((int64_t)g * 2 + 1) * D + d] = hi;
    }
  }
}

void qo_request_bounds(const qo_shape *s, const void *k_cache,
                       const int32_t *pt_row, int32_t ctx, double *bounds) {
  const int32_t n = pages_of(ctx, s->page_size);
  const int64_t per_page = (int64_t)s->num_kv_heads * 2 * s->head_dim;
  for (int32_t j = 0; j < n; ++j)
    qo_page_bounds(s, k_cache, pt_row, ctx, j, bounds + j * per_page);
}

/* ---- build_decode_view: page scores ------------------------------------- */

/* Quest's criticality bound for q head h and page j:
 *     U[h][j] = sum_d max(q[h][d] * min[j][d], q[h][d] * max[j][d]),
 * the largest q.k any key inside the page's min/max box can reach.
 * READING (GQA): q head h reads KV head g = h / G with G = Hq / Hkv, and a KV
 * head's page score combines its G q heads by MAX (so the score bounds q.k of
 * every q head in the group) or, as a variant, by SUM.
 * READING: q enters unscaled (the softmax scale is positive and does not
 * change the order). */
void qo_request_scores(const qo_shape *s, const void *q_r,
                       const double *bounds, int32_t n_pages, int32_t reduce,
                       double *scores) {
  const int32_t Hq = s->num_q_heads, H = s->num_kv_heads, D = s->head_dim;
  const int32_t G = Hq / H;
  for (int32_t g = 0; g < H; ++g) {
    for (int32_t j = 0; j < n_pages; ++j) {
      const double *lo = bounds + (((int64_t)j * H + g) * 2 + 0) * D;
      const double *hi = bounds + (((int64_t)j * H + g) * 2 + 1) * D;
      double score = (reduce == QO_REDUCE_MAX) ? -INFINITY : 0.0;
      for (int32_t h = g * G; h < (g + 1) * G; ++h) {
        double u = 0.0;
        for (int32_t d = 0; d < D; ++d) {
          const double qd = elem_value(q_r, (int64_t)h * D + d, s->elem);
          const double a = qd * lo[d], b = qd * hi[d];
          u += (a > b ? a : b);
        }
        if (reduce == QO_REDUCE_MAX)
          score = (u > score ? u : score);
        else
          score += u;
      }
      scores[(int64_t)g * n_pages + j] = score;
    }
  }
}

/* Per-q-head scores (READING, a variant the pages leave open: the selection
 * is not shared across a GQA group): U[h][j] of every q head h, which reads
 * the bounds of its KV head h / G.  By definition this is the group score of
 * a group of one head, so it is computed as exactly that. */
void qo_request_head_scores(const qo_shape *s, const void *q_r,
                            const double *bounds, int32_t n_pages, double *scores) {
  const int32_t Hq = s->num_q_heads, H = s->num_kv_heads, D = s->head_dim;
  const int32_t G = Hq / H;
  const size_t esz = elem_bytes(s->elem);
  qo_shape one = *s;
  one.num_q_heads = 1;
  one.num_kv_heads = 1;
  double *b1 = (double *)malloc(sizeof(double) * ((size_t)n_pages * 2 * D + 1));
  for (int32_t h = 0; h < Hq; ++h) {
    const int32_t kvh = h / G;
    for (int32_t j = 0; j < n_pages; ++j)
      memcpy(b1 + (int64_t)j * 2 * D, bounds + ((int64_t)j * H + kvh) * 2 * D,
             sizeof(double) * 2 * (size_t)D);
    qo_request_scores(&one, (const char *)q_r + (size_t)h * D * esz, b1, n_pages,
                      QO_REDUCE_MAX, scores + (int64_t)h * n_pages);
  }
  free(b1);
}

/* ---- build_decode_view: top-k within the token budget ------------------- */

/* READING: a budget of B tokens buys floor(B / P) whole pages, at least one
 * and at most the request's page count; an empty request selects nothing. */
int32_t qo_pages_for_budget(int32_t budget_tokens, int32_t ctx,
                            int32_t page_size) {
  const int32_t n = pages_of(ctx, page_size);
  if (n == 0) return 0;
  int32_t k = budget_tokens / page_size;
  if (k < 1) k = 1;
  if (k > n) k = n;
  return k;
}

typedef struct {
  double score;
  int32_t page;
} scored_page;

/* Larger score first; equal scores: lower logical page first (READING). */
static int by_score_then_page(const void *pa, const void *pb) {
  const scored_page *a = (const scored_page *)pa, *b = (const scored_page *)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  return (a->page > b->page) - (a->page < b->page);
}

static int ascending_int(const void *pa, const void *pb) {
  const int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  return (a > b) - (a < b);
}

/* The k pages with the largest scores, ties to the lower logical index,
 * reported in ascending page order (READING: ascending, so the selected view
 * keeps the request's position order). */
void qo_select(const double *scores, int32_t n, int32_t k, int32_t *sel) {
  if (k <= 0 || n <= 0) return;
  scored_page *all = (scored_page *)malloc(sizeof(scored_page) * (size_t)n);
  for (int32_t j = 0; j < n; ++j) {
    all[j].score = scores[j];
    all[j].page = j;
  }
  qsort(all, (size_t)n, sizeof(scored_page), by_score_then_page);
  for (int32_t i = 0; i < k; ++i) sel[i] = all[i].page;
  qsort(sel, (size_t)k, sizeof(int32_t), ascending_int);
  free(all);
}

/* Forced pages (READING, a variant the pages leave open): the first n_sink
 * and the last n_recent pages of a request are kept ahead of every scored
 * page, the lower page first among themselves; the budget still fixes k, and
 * the remaining slots follow qo_select's order.  The result is ascending. */
static int forced_page(int32_t j, int32_t n, int32_t n_sink, int32_t n_recent) {
  return j < n_sink || j >= n - n_recent;
}

typedef struct {
  int forced;
  scored_page sp;
} ranked_page;

static int forced_then_score(const void *pa, const void *pb) {
  const ranked_page *a = (const ranked_page *)pa, *b = (const ranked_page *)pb;
  if (a->forced != b->forced) return a->forced ? -1 : 1;
  if (a->forced) return (a->sp.page > b->sp.page) - (a->sp.page < b->sp.page);
  return by_score_then_page(&a->sp, &b->sp);
}

void qo_select_forced(const double *scores, int32_t n, int32_t k, int32_t n_sink,
                      int32_t n_recent, int32_t *sel) {
  if (k <= 0 || n <= 0) return;
  ranked_page *all = (ranked_page *)malloc(sizeof(ranked_page) * (size_t)n);
  for (int32_t j = 0; j < n; ++j) {
    all[j].forced = forced_page(j, n, n_sink, n_recent);
    all[j].sp.score = scores[j];
    all[j].sp.page = j;
  }
  qsort(all, (size_t)n, sizeof(ranked_page), forced_then_score);
  for (int32_t i = 0; i < k; ++i) sel[i] = all[i].sp.page;
  qsort(sel, (size_t)k, sizeof sel[0], ascending_int);
  free(all);
}

/* ---- attention over the selected view ----------------------------------- */

/* For q head h (KV head g = h / G): logits l_t = sm_scale * q_h . k_t over the
 * valid tokens t of the pages g selected, weights softmax(l), output
 * sum_t w_t v_t.  READING: sm_scale = 1/sqrt(D) is the caller's choice; a head
 * whose view holds no token outputs zeros. */
static void attend_one_head(const qo_shape *s, const void *q_r,
                            const void *k_cache, const void *v_cache,
                            const int32_t *pt_row, int32_t ctx,
                            const int32_t *pages, int32_t npages, int32_t h,
                            double sm_scale, double *out_h) {
  const int32_t H = s->num_kv_heads, D = s->head_dim, P = s->page_size;
  const int32_t g = h / (s->num_q_heads / H);
  double *logit = (double *)malloc(sizeof(double) * ((size_t)npages * P + 1));
  int64_t *tok_phys = (int64_t *)malloc(sizeof(int64_t) * ((size_t)npages * P + 1));
  int32_t *tok_slot = (int32_t *)malloc(sizeof(int32_t) * ((size_t)npages * P + 1));
  int32_t ntok = 0;
  for (int32_t i = 0; i < npages; ++i) {
    const int32_t j = pages[i];
    const int64_t phys = pt_row[j];
    for (int32_t slot = 0; slot < P; ++slot) {
      if (j * P + slot >= ctx) break;
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d)
        dot += elem_value(q_r, (int64_t)h * D + d, s->elem) *
               elem_value(k_cache, k_offset(s, phys, g, slot, d), s->elem);
      logit[ntok] = sm_scale * dot;
      tok_phys[ntok] = phys;
      tok_slot[ntok] = slot;
      ++ntok;
    }
  }
  for (int32_t d = 0; d < D; ++d) out_h[d] = 0.0;
  if (ntok > 0) {
    double m = -INFINITY;
    for (int32_t t = 0; t < ntok; ++t) m = (logit[t] > m ? logit[t] : m);
    double denom = 0.0;
    for (int32_t t = 0; t < ntok; ++t) denom += exp(logit[t] - m);
    for (int32_t t = 0; t < ntok; ++t) {
      const double w = exp(logit[t] - m) / denom;
      for (int32_t d = 0; d < D; ++d)
        out_h[d] += w * elem_value(v_cache,
                                   v_offset(s, tok_phys[t], g, tok_slot[t], d),
                                   s->elem);
    }
  }
  free(logit);
  free(tok_phys);
  free(tok_slot);
}

void qo_request_attend(const qo_shape *s, const void *q_r, const void *k_cache,
                       const void *v_cache, const int32_t *pt_row, int32_t ctx,
                       const int32_t *sel, const int32_t *nsel,
                       int32_t sel_stride, double sm_scale, double *out) {
  const int32_t Hq = s->num_q_heads, G = Hq / s->num_kv_heads;
  for (int32_t h = 0; h < Hq; ++h) {
    const int32_t g = h / G;
    attend_one_head(s, q_r, k_cache, v_cache, pt_row, ctx,
                    sel + (int64_t)g * sel_stride, nsel[g], h, sm_scale,
                    out + (int64_t)h * s->head_dim);
  }
}

/* Attention with one selection per q head: head h attends the pages in
 * sel[h][0 .. nsel[h]-1] of its KV head. */
void qo_request_attend_heads(const qo_shape *s, const void *q_r, const void *k_cache,
                             const void *v_cache, const int32_t *pt_row, int32_t ctx,
                             const int32_t *sel, const int32_t *nsel,
                             int32_t sel_stride, double sm_scale, double *out) {
  for (int32_t h = 0; h < s->num_q_heads; ++h)
    attend_one_head(s, q_r, k_cache, v_cache, pt_row, ctx, sel + (int64_t)h * sel_stride,
                    nsel[h], h, sm_scale, out + (int64_t)h * s->head_dim);
}

/* Dense attention is the view that holds every page (the vanilla method). */
void qo_request_dense(const qo_shape *s, const void *q_r, const void *k_cache,
                      const void *v_cache, const int32_t *pt_row, int32_t ctx,
                      double sm_scale, double *out) {
  const int32_t n = pages_of(ctx, s->page_size);
  int32_t *all = (int32_t *)malloc(sizeof(int32_t) * ((size_t)n + 1));
  for (int32_t j = 0; j < n; ++j) all[j] = j;
  for (int32_t h = 0; h < s->num_q_heads; ++h)
    attend_one_head(s, q_r, k_cache, v_cache, pt_row, ctx, all, n, h, sm_scale,
                    out + (int64_t)h * s->head_dim);
  free(all);
}
