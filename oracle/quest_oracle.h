/*
 * quest_oracle.h -- declarations of the fp64 CPU oracle for Quest query-aware
 * sparse decode over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This header belongs to the oracle alone: the HIP
 * library does not include it and the oracle includes nothing of the HIP
 * library.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline leg may load the oracle.
 *
 * Storage conventions the oracle reads (restated here independently of the
 * library's own header; both describe the same byte layout):
 *   element type  QO_F32 = IEEE binary32, QO_BF16 = raw bfloat16 bit patterns
 *   K pool        [num_pool_pages][Hkv][P][D]   (token-major inside a page)
 *   V pool        [num_pool_pages][Hkv][D][P]   (dim-major inside a page)
 *   page table    one int32 row per request: logical page j -> physical page
 *   q, out        [Hq][D] per request
 *   bounds        fp64 [n_pages][Hkv][2][D], index 0 = elementwise min,
 *                 index 1 = elementwise max
 *   scores        fp64 [Hkv][n_pages]
 */
#ifndef QUEST_ORACLE_H
#define QUEST_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { QO_F32 = 0, QO_BF16 = 1 };
enum { QO_REDUCE_MAX = 0, QO_REDUCE_SUM = 1 };

typedef struct {
  int32_t elem;            /* QO_F32 or QO_BF16 */
  int32_t num_q_heads;     /* Hq */
  int32_t num_kv_heads;    /* Hkv, divides Hq */
  int32_t head_dim;        /* D */
  int32_t page_size;       /* P */
  int64_t num_pool_pages;  /* physical pages in the pool */
} qo_shape;

/* Writes n_new tokens (k_new/v_new laid out [n_new][Hkv][D]) at logical
 * positions pos0 .. pos0+n_new-1 of one request. */
void qo_store_tokens(const qo_shape *s, int32_t n_new, const void *k_new,
                     const void *v_new, int32_t pos0, const int32_t *pt_row,
                     void *k_cache, void *v_cache);

/* Elementwise key min/max of every logical page of one request, from scratch
 * over the request's valid tokens (positions < ctx). */
void qo_request_bounds(const qo_shape *s, const void *k_cache,
                       const int32_t *pt_row, int32_t ctx, double *bounds);

/* Same, for the single logical page j only (bounds_j is [Hkv][2][D]). */
void qo_page_bounds(const qo_shape *s, const void *k_cache,
                    const int32_t *pt_row, int32_t ctx, int32_t j,
                    double *bounds_j);

/* Per-page upper-bound score of every KV head's group for one request. */
void qo_request_scores(const qo_shape *s, const void *q_r,
                       const double *bounds, int32_t n_pages, int32_t reduce,
                       double *scores);

/* Per-q-head page scores [Hq][n_pages]: each head's own bound, no group
 * reduction. */
void qo_request_head_scores(const qo_shape *s, const void *q_r,
                            const double *bounds, int32_t n_pages, double *scores);

/* Number of pages a token budget buys for a request of ctx tokens. */
int32_t qo_pages_for_budget(int32_t budget_tokens, int32_t ctx,
                            int32_t page_size);

/* Top-k pages of one score row; writes k logical ids in ascending order. */
void qo_select(const double *scores, int32_t n, int32_t k, int32_t *sel);

/* The same with the first n_sink and last n_recent pages kept first. */
void qo_select_forced(const double *scores, int32_t n, int32_t k, int32_t n_sink,
                      int32_t n_recent, int32_t *sel);

/* Softmax attention of every q head over the valid tokens of the pages its KV
 * head selected.  sel is [Hkv][sel_stride], nsel is [Hkv]. */
void qo_request_attend(const qo_shape *s, const void *q_r, const void *k_cache,
                       const void *v_cache, const int32_t *pt_row, int32_t ctx,
                       const int32_t *sel, const int32_t *nsel,
                       int32_t sel_stride, double sm_scale, double *out);

/* Attention with one selection per q head: sel is [Hq][sel_stride], nsel [Hq]. */
void qo_request_attend_heads(const qo_shape *s, const void *q_r, const void *k_cache,
                             const void *v_cache, const int32_t *pt_row, int32_t ctx,
                             const int32_t *sel, const int32_t *nsel,
                             int32_t sel_stride, double sm_scale, double *out);

/* Dense attention: every valid token of the request. */
void qo_request_dense(const qo_shape *s, const void *q_r, const void *k_cache,
                      const void *v_cache, const int32_t *pt_row, int32_t ctx,
                      double sm_scale, double *out);

#ifdef __cplusplus
}
#endif

#endif /* QUEST_ORACLE_H */
