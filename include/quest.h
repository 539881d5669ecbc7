/*
 * quest.h -- C ABI of libquest.so: Quest query-aware sparse decode attention
 * over a paged KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The method.  The pages name Quest, its persistent page metadata and the
 * two hooks it uses, but never write its arithmetic; this library computes
 * the reading stated here and in each entry point below: per KV page, the
 * elementwise minimum and maximum of the page's keys; at each decode step
 * the current query gives every page an upper bound on q.k over that min/max
 * box, the best pages within a token budget are selected per KV head, and
 * attention runs over those pages only.
 *
 * Where the pages put it.  The Sparse-vLLM skill page "add-sparse-method"
 * (Placement Rules 2-4, Decision Rules) places persistent per-page metadata in
 * the method's cache manager, refreshes it through on_kv_stored after KV is
 * written, and builds the decode-time view from the current layer's q through
 * build_decode_view.  The SparseEngine digest ("SparseEngine: Sparse-First
 * Inference Engine", Method key points) registers Quest's query-relevant page
 * selection as a lifecycle hook, lets each method's cache manager own KV
 * representation, physical layout, position mapping and metadata, and hands
 * the backend an explicit-KV attention view.  The entry points map onto
 * those steps:
 *     quest_append_kv      on_kv_stored: KV store + fused min/max refresh
 *     quest_page_scores    build_decode_view, part 1: per-page bounds from q
 *     quest_append_score   the two above fused into one pass
 *     quest_topk_pages     build_decode_view, part 2: top-k within the budget
 *                          (quest_topk_pages_forced: with sink / recent pages
 *                          always kept)
 *     quest_sparse_decode  attention over the selected explicit-KV view
 *
 * Conventions shared by every entry point
 *  - All buffers are device memory owned by the caller (the cache manager
 *    role).  The library allocates nothing, keeps no pointer after a call
 *    returns and holds no state between calls (the one exception is the
 *    library-owned scratch array of quest_decode_step_noalloc, described
 *    there).  The layout struct is read during the call only.
 *  - Every call is asynchronous: it validates its arguments on the host,
 *    enqueues kernels on `stream` (a hipStream_t passed as void*, NULL for the
 *    null stream) and returns.  It never synchronises, allocates or copies
 *    device memory to the host, so a sequence of calls may be captured into a
 *    hipGraph.
 *  - Return value: QUEST_OK (0) or a negative quest_status.  Validation runs
 *    before any HIP call; on a validation error nothing is launched.  A launch
 *    failure reported by HIP returns QUEST_ERR_HIP.  Nothing is printed, no
 *    exception crosses the ABI, the library never aborts.
 *  - batch == 0 is valid and launches nothing.  Size limits (QUEST_ERR_SHAPE
 *    beyond them): 0 <= batch <= 65535, batch * num_q_heads <= 2^19,
 *    max_pages_per_seq * page_size <= INT32_MAX and max_pages_per_seq *
 *    num_kv_heads < 2^30 (every launch grid stays within 2^32 work-items).
 *  - Device-side preconditions, not checked on the host (the data lives on the
 *    device): page-table entries of live pages lie in [0, num_pool_pages);
 *    ctx_lens[r] <= max_pages_per_seq * page_size; budgets >= 0.  No kernel
 *    touches memory outside the pool for a live page whose id lies outside
 *    [0, num_pool_pages): such a page scores -inf, is never stored to and
 *    contributes no token to the attention.  Kernels clamp every other index
 *    into its row; results for inputs that break the other preconditions are
 *    unspecified.
 *  - Numbers: q, K, V, the page metadata and the output share one element type
 *    (fp32, or bf16 with round-to-nearest-even on every bf16 write).  Scores,
 *    softmax statistics and accumulators are fp32.
 */
#ifndef QUEST_H
#define QUEST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QUEST_ABI_VERSION 1

typedef enum {
  QUEST_OK = 0,
  QUEST_ERR_NULL = -1,        /* a required pointer is NULL */
  QUEST_ERR_SHAPE = -2,       /* inconsistent or out-of-range sizes */
  QUEST_ERR_UNSUPPORTED = -3, /* valid but not built: dtype, D, P, G */
  QUEST_ERR_WORKSPACE = -4,   /* workspace missing or too small */
  QUEST_ERR_ABI = -5,         /* layout.abi_version != QUEST_ABI_VERSION */
  QUEST_ERR_HIP = -6,         /* the HIP runtime rejected a launch */
  QUEST_ERR_SCRATCH = -7      /* beyond the static scratch of quest_decode_step_noalloc */
} quest_status;

/* Bytes of the library-owned device scratch of quest_decode_step_noalloc
 * (one copy per GPU, held until the process ends). */
#define QUEST_STATIC_SCRATCH_BYTES (16u << 20)

typedef enum { QUEST_F32 = 0, QUEST_BF16 = 1 } quest_dtype;

/* How a KV head's page score combines the scores of the q heads that share
 * it (grouped-query attention).  MAX keeps the score an upper bound of q.k for
 * every q head of the group; SUM bounds the group-summed logit. */
typedef enum { QUEST_REDUCE_MAX = 0, QUEST_REDUCE_SUM = 1 } quest_group_reduce;

/* Whose pages are selected (a variant the pages leave open).  PER_KV_HEAD:
 * the q heads of a KV head share one selection from the group score (the
 * layout's R = Hkv selection rows per request).  PER_Q_HEAD: every q head
 * scores and selects its own pages from its own bound, with no group
 * reduction (R = Hq rows per request); each q head then attends its own
 * pages, so the selected K/V bytes grow with the group size. */
typedef enum { QUEST_SELECT_PER_KV_HEAD = 0, QUEST_SELECT_PER_Q_HEAD = 1 } quest_selection;

/* Shape of one attention layer's paged cache.
 *   num_q_heads (Hq) and num_kv_heads (Hkv): Hq % Hkv == 0, G = Hq/Hkv <= 16;
 *     q head h reads KV head h / G.
 *   head_dim (D): 64 or 128.   page_size (P): 8, 16, 32 or 64 tokens (64
 *   with fp32 only at D = 64).
 *   dtype: quest_dtype of q, K, V, metadata and output.
 *   num_pool_pages: physical pages in the pool shared by all requests.
 *   max_pages_per_seq: row stride of the page table and of the score array.
 *   selection: quest_selection; it fixes R, the selection rows per request
 *     (R = Hkv per KV head, R = Hq per q head).  Other values return
 *     QUEST_ERR_UNSUPPORTED. */
typedef struct {
  int32_t abi_version;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t dtype;
  int64_t num_pool_pages;
  int32_t max_pages_per_seq;
  int32_t selection;          /* quest_selection (0: per KV head) */
} quest_layout;

/* Device layouts (row-major, contiguous):
 *   k_cache    [num_pool_pages][Hkv][P][D]   token-major pages
 *   v_cache    [num_pool_pages][Hkv][D][P]   dim-major pages (each channel's
 *                                            P values are contiguous)
 *   kmeta      [num_pool_pages][Hkv][2][D]   [..][0][d] = min, [..][1][d] = max
 *   page_table int32 [batch][max_pages_per_seq]: logical page j of request r
 *              -> physical page; position p lives in logical page p / P at slot
 *              p % P.  Only entries j < ceil(ctx/P) are read.
 *   ctx_lens   int32 [batch]: valid tokens of each request.
 *   q, out     [batch][Hq][D]
 *   scores     fp32 [batch][R][max_pages_per_seq]
 *   budget_tokens int32 [batch]
 *   sel_pages  int32 [batch][R][max_k]; num_sel int32 [batch][R]
 * (R = Hkv with the default per-KV-head selection; below, "row g" is KV head
 * g then, or q head g with per-q-head selection.) */

/* Returns QUEST_ABI_VERSION of the loaded library. */
int quest_abi_version(void);

/* Static, human-readable name of a quest_status value. */
const char *quest_status_string(int status);

/* on_kv_stored (Sparse-vLLM "add-sparse-method", Placement Rules 3): stores
 * new tokens and refreshes the page metadata in one pass.
 *   k_new, v_new  [T][Hkv][D]; request r owns rows cu_new[r] .. cu_new[r+1]-1
 *                 (cu_new int32 [batch+1], device, non-decreasing, cu_new[0]=0)
 *   ctx_before    int32 [batch], device: tokens request r held before; its new
 *                 tokens take positions ctx_before[r], ctx_before[r]+1, ...
 *   max_new_per_seq  host hint, >= 0: the largest per-request token count; it
 *                 sizes the grid only (every token is stored whatever it is).
 * K and V go to their slots.  For every touched page and KV head, the metadata
 * becomes the elementwise min/max of the new tokens when the first new token
 * sits at the page's slot 0 (a fresh page: nothing stale from a previous owner
 * survives), and otherwise of the stored metadata and the new tokens.  Min and
 * max are exact (no rounding).  A request's pages must not be shared with
 * another request's new tokens in the same call. */
int quest_append_kv(const quest_layout *layout, int32_t batch,
                    const void *k_new, const void *v_new,
                    const int32_t *cu_new, const int32_t *ctx_before,
                    int32_t max_new_per_seq, const int32_t *page_table,
                    void *k_cache, void *v_cache, void *kmeta, void *stream);

/* build_decode_view, part 1 (Placement Rules 4; SparseEngine digest, Method
 * key points, query-relevant page selection): for every request r, KV head g
 * and logical page j < ceil(ctx_lens[r]/P),
 *   U[h][j] = sum_d max(q[r][h][d]*min[j][g][d], q[r][h][d]*max[j][g][d])
 * for each q head h of group g (q unscaled), and
 *   scores[r][g][j] = max_h U[h][j]   (group_reduce MAX) or sum_h (SUM).
 * With per-q-head selection there is no reduction: scores[r][h][j] = U[h][j]
 * for every q head h (group_reduce is still validated but has no effect).
 * Products of bf16 values are exact in fp32 (fp32 inputs: each product is
 * fused into its fp32 add); sums are fp32 in an unspecified order.  A page
 * whose page-table entry lies outside [0, num_pool_pages) scores -inf.
 * Entries j >= ceil(ctx/P) are not written. */
int quest_page_scores(const quest_layout *layout, int32_t batch,
                      const void *q, const void *kmeta,
                      const int32_t *page_table, const int32_t *ctx_lens,
                      int32_t group_reduce, float *scores, void *stream);

/* on_kv_stored followed by build_decode_view part 1, in one pass: exactly
 * quest_append_kv(layout, batch, k_new, v_new, cu_new, ctx_before,
 * max_new_per_seq, page_table, k_cache, v_cache, kmeta) then
 * quest_page_scores(layout, batch, q, kmeta, page_table, ctx_lens,
 * group_reduce, scores) with ctx_lens[r] = ctx_before[r] + (cu_new[r+1] -
 * cu_new[r]).  It is one kernel (bf16 and fp32): the scoring work-group that
 * owns a touched page stores the new tokens and refreshes the page's min/max
 * first, so the metadata is read once; max_new_per_seq is validated but the
 * grid does not depend on it.  Arguments and layouts as in those two calls. */
int quest_append_score(const quest_layout *layout, int32_t batch, const void *q,
                       const void *k_new, const void *v_new, const int32_t *cu_new,
                       const int32_t *ctx_before, int32_t max_new_per_seq,
                       const int32_t *page_table, void *k_cache, void *v_cache,
                       void *kmeta, int32_t group_reduce, float *scores, void *stream);

/* build_decode_view, part 2 (Sparse-vLLM "add-sparse-method", Placement
 * Rules 4: the decode view is built from the current layer's q; SparseEngine
 * digest, Method key points: Quest's query-relevant page selection):
 * k_r = min(max_k, clamp(floor(budget_tokens[r] /
 * P), 1, n_r)) pages per (request, selection row), n_r = ceil(ctx_lens[r]/P);
 * k_r = 0 when ctx_lens[r] == 0.  The k_r pages with the largest scores are
 * selected; equal scores go to the lower logical page (-0.0 equals +0.0).
 * sel_pages[r][g][0..k_r-1] receives their logical ids in ascending order,
 * the rest of the row -1; num_sel[r][g] = k_r.  Selection is exact: any
 * correct top-k of the given scores returns the same ids. */
int quest_topk_pages(const quest_layout *layout, int32_t batch,
                     const float *scores, const int32_t *ctx_lens,
                     const int32_t *budget_tokens, int32_t max_k,
                     int32_t *sel_pages, int32_t *num_sel, void *stream);

/* quest_topk_pages with forced pages, a variant the pages leave open (a
 * selection that always keeps attention-sink and most-recent pages): for
 * request r with n_r pages, the pages j < n_sink and j >= n_r - n_recent are
 * ranked above every scored page, the lower page first among them; k_r is
 * computed as in quest_topk_pages (the budget still decides how many pages
 * are kept, forced ones included), so when k_r is smaller than the forced
 * set the k_r lowest forced pages are kept.  Output as in quest_topk_pages;
 * n_sink = n_recent = 0 is exactly quest_topk_pages.  n_sink or n_recent < 0
 * returns QUEST_ERR_SHAPE. */
int quest_topk_pages_forced(const quest_layout *layout, int32_t batch,
                            const float *scores, const int32_t *ctx_lens,
                            const int32_t *budget_tokens, int32_t max_k,
                            int32_t n_sink, int32_t n_recent,
                            int32_t *sel_pages, int32_t *num_sel, void *stream);

/* Workspace bytes quest_sparse_decode needs for this batch and max_k (0 for
 * batch 0).  A pure function of its arguments; never calls HIP. */
size_t quest_sparse_decode_workspace_bytes(const quest_layout *layout,
                                           int32_t batch, int32_t max_k);

/* Attention over the explicit-KV view (SparseEngine digest, Method key
 * points, AttentionView): for q head h of request r, with g = h / G,
 *   out[r][h] = sum_t softmax_t(sm_scale * q[r][h].k_t) v_t
 * over the valid tokens t (< ctx_lens[r]) of KV head g in the pages
 * sel_pages[r][x][0 .. num_sel[r][x]-1] of its selection row x (x = g per KV
 * head, x = h per q head).  A head with no token in its view outputs zeros.
 * Split-K: pages are spread over work-groups, each keeps a running max, sum
 * and fp32 accumulator, and a second kernel merges the partials.  The bf16
 * path feeds each fp32 softmax weight to the matrix-core P*V product as the
 * sum of two bf16 values (about 16 significant bits).
 * workspace: device memory of at least quest_sparse_decode_workspace_bytes;
 * contents on entry do not matter. */
int quest_sparse_decode(const quest_layout *layout, int32_t batch,
                        const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *page_table, const int32_t *ctx_lens,
                        const int32_t *sel_pages, const int32_t *num_sel,
                        int32_t max_k, float sm_scale, void *out,
                        void *workspace, size_t workspace_bytes, void *stream);

/* quest_topk_pages_forced followed by quest_sparse_decode on its selection,
 * in fewer launches where the shape allows (one kernel for the selection and
 * the attention, then the merge, or no merge when each selection row is
 * attended by one work-group).  Arguments as in those two calls; the
 * workspace of quest_sparse_decode_workspace_bytes suffices.  The selection
 * and counts written are exactly those of quest_topk_pages_forced.  The
 * outputs equal the two calls' up to the order of the fp32 sums inside a
 * work-group (the fused kernel merges 16 waves of half the pages each, and
 * may split a row differently): the same tolerance against exact attention
 * holds.  In the fused kernel every split of a row repeats the row's
 * selection, which pays while the grid fits one resident work-group per CU:
 * bf16, rows of at most 8192 pages, D = 64 or D = 128 with 16-token pages,
 * and a split of each row into at most 256 / (batch x rows) parts of at most
 * 256 pages; other shapes take the two kernels in sequence.  Errors: those
 * of both calls. */
int quest_topk_sparse_decode(const quest_layout *layout, int32_t batch,
                             const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *page_table, const int32_t *ctx_lens,
                             const float *scores, const int32_t *budget_tokens,
                             int32_t max_k, int32_t n_sink, int32_t n_recent,
                             float sm_scale, int32_t *sel_pages, int32_t *num_sel,
                             void *out, void *workspace, size_t workspace_bytes,
                             void *stream);

/* 1 if quest_topk_sparse_decode runs the fused kernel for this batch and
 * max_k, 0 if it runs the two kernels (or batch is 0), a negative
 * quest_status for invalid arguments.  Never calls HIP. */
int quest_topk_sparse_decode_fused(const quest_layout *layout, int32_t batch,
                                   int32_t max_k);

/* The launch plan quest_topk_sparse_decode uses (for reports and tests):
 * *fused = 1 for the fused kernel (then *num_splits and *pages_per_split are
 * its plan), 0 for the two kernels (then they are quest_sparse_decode_plan's).
 * The fused plan never has more splits than quest_sparse_decode_plan's, so
 * the workspace of quest_sparse_decode_workspace_bytes always suffices.
 * Never calls HIP; QUEST_ERR_NULL for a NULL output pointer. */
int quest_topk_sparse_decode_plan(const quest_layout *layout, int32_t batch,
                                  int32_t max_k, int32_t *fused, int32_t *num_splits,
                                  int32_t *pages_per_split);

/* The whole decode step of one layer in one call: quest_append_score (the
 * new tokens' store and page bounds, then the page scores; "add-sparse-method",
 * Placement Rules 2-4: on_kv_stored, then build_decode_view from the current
 * q) followed by quest_topk_sparse_decode on those scores (the selection
 * within the budget and attention over the explicit-KV view, SparseEngine
 * digest, Method key points).  Arguments as in those two calls; ctx_lens must
 * equal ctx_before plus each request's new tokens.  Results equal the two
 * calls' bit for bit.  Errors: those of both calls. */
int quest_decode_step(const quest_layout *layout, int32_t batch, const void *q,
                      const void *k_new, const void *v_new, const int32_t *cu_new,
                      const int32_t *ctx_before, int32_t max_new_per_seq,
                      const int32_t *page_table, void *k_cache, void *v_cache, void *kmeta,
                      int32_t group_reduce, const int32_t *ctx_lens,
                      const int32_t *budget_tokens, int32_t max_k, int32_t n_sink,
                      int32_t n_recent, float sm_scale, float *scores, int32_t *sel_pages,
                      int32_t *num_sel, void *out, void *workspace, size_t workspace_bytes,
                      void *stream);

/* quest_decode_step for callers that cannot allocate device memory (code
 * under hipGraph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step, the same kernels and the same results bit for
 * bit, but the decode's split partials live in a library-owned device array
 * of QUEST_STATIC_SCRATCH_BYTES (16 MiB) per GPU instead of a caller
 * workspace.  The caller still passes every input and output.  The call
 * allocates and frees nothing; on its first use on a device (the calling
 * thread's current device, which must be the stream's) it looks up that
 * device's copy of the array, a host call that allocates nothing.
 * Limits: the call needs quest_sparse_decode_workspace_bytes(layout, batch,
 * max_k) <= QUEST_STATIC_SCRATCH_BYTES, else QUEST_ERR_SCRATCH with nothing
 * launched (at 4 KV heads, G 8, D 128: any max_k up to batch 126, whose
 * rows take at most 8 splits each).
 * Concurrency: every call on one GPU shares that GPU's array, and the array
 * keeps the last call's partials (their contents on entry do not matter;
 * nothing needs clearing).  Calls that may overlap on one GPU (several
 * streams, several host threads) race on it and must be serialised by the
 * caller.  Arguments and other errors as in quest_decode_step. */
int quest_decode_step_noalloc(const quest_layout *layout, int32_t batch, const void *q,
                              const void *k_new, const void *v_new, const int32_t *cu_new,
                              const int32_t *ctx_before, int32_t max_new_per_seq,
                              const int32_t *page_table, void *k_cache, void *v_cache,
                              void *kmeta, int32_t group_reduce, const int32_t *ctx_lens,
                              const int32_t *budget_tokens, int32_t max_k, int32_t n_sink,
                              int32_t n_recent, float sm_scale, float *scores,
                              int32_t *sel_pages, int32_t *num_sel, void *out, void *stream);

/* Launch plan quest_sparse_decode uses (for reports): number of KV splits per
 * (request, selection row) and pages per split.  Never calls HIP. */
int quest_sparse_decode_plan(const quest_layout *layout, int32_t batch,
                             int32_t max_k, int32_t *num_splits,
                             int32_t *pages_per_split);

#ifdef __cplusplus
}
#endif

#endif /* QUEST_H */
