// quest_abi.cpp -- the C ABI declared in include/quest.h: host-side argument
// validation, then dispatch to the gfx950 kernels on the caller's stream.
//
// Conventions taken from the 1Cat-vLLM page "Developing 1Cat runtime
// extensions" (Change a native binding): a versioned interface that rejects
// what it cannot express before doing any work, and native hot paths that
// consume prebound values rather than environment strings.  No function here
// reads the environment, allocates, synchronises or prints.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "quest.h"
#include "quest_launch.h"

namespace {

using quest::Dims;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Validates the layout; fills dm.  Never calls HIP.
int check_layout(const quest_layout *L, Dims &dm) {
  if (L == nullptr) return QUEST_ERR_NULL;
  if (L->abi_version != QUEST_ABI_VERSION) return QUEST_ERR_ABI;
  if (L->num_q_heads <= 0 || L->num_kv_heads <= 0 || L->head_dim <= 0 ||
      L->page_size <= 0 || L->num_pool_pages <= 0 || L->max_pages_per_seq <= 0)
    return QUEST_ERR_SHAPE;
  if (L->num_q_heads % L->num_kv_heads != 0) return QUEST_ERR_SHAPE;
  if (L->dtype != QUEST_F32 && L->dtype != QUEST_BF16) return QUEST_ERR_UNSUPPORTED;
  if (L->head_dim != 64 && L->head_dim != 128) return QUEST_ERR_UNSUPPORTED;
  if (L->page_size != 8 && L->page_size != 16 && L->page_size != 32 && L->page_size != 64)
    return QUEST_ERR_UNSUPPORTED;
  // fp32 pages of 64 tokens at D = 128 would need more than 64 KB of LDS in
  // the fp32 decode kernel's staging
  if (L->dtype == QUEST_F32 && L->page_size == 64 && L->head_dim == 128)
    return QUEST_ERR_UNSUPPORTED;
  const int G = L->num_q_heads / L->num_kv_heads;
  if (G > 16) return QUEST_ERR_UNSUPPORTED;
  // keep per-request token counts inside int32 arithmetic
  if ((int64_t)L->max_pages_per_seq * L->page_size > INT32_MAX) return QUEST_ERR_SHAPE;
  // the scoring grid (64 pages x one KV head per 256-thread work-group) stays
  // under 2^32 work-items per dimension
  if ((int64_t)L->max_pages_per_seq * L->num_kv_heads >= ((int64_t)1 << 30))
    return QUEST_ERR_SHAPE;
  if (L->selection != QUEST_SELECT_PER_KV_HEAD && L->selection != QUEST_SELECT_PER_Q_HEAD)
    return QUEST_ERR_UNSUPPORTED;
  dm.Hq = L->num_q_heads;
  dm.Hkv = L->num_kv_heads;
  dm.G = G;
  if (L->selection == QUEST_SELECT_PER_Q_HEAD) {
    dm.R = dm.Hq;
    dm.Gcols = 1;
    dm.gdiv = G;
  } else {
    dm.R = dm.Hkv;
    dm.Gcols = G;
    dm.gdiv = 1;
  }
  dm.D = L->head_dim;
  dm.P = L->page_size;
  dm.dtype = L->dtype;
  dm.pool = L->num_pool_pages;
  dm.max_pages = L->max_pages_per_seq;
  return QUEST_OK;
}

// batch <= 65535 (grid y of the scoring, top-k and append kernels) and
// batch * Hq <= 2^19, which keeps every other grid under 2^32 work-items:
// the bf16 decode launches at most 8 splits per row once a batch has more
// than 1024 selection rows (at most 256 work-groups below that), so at most
// 2^19 x 8 work-groups of 512 threads; the fp32 decode at most rows + 2048
// work-groups of 256; the merge batch * Hq work-groups of 128.
int check_batch(int32_t batch, const Dims &dm) {
  if (batch < 0 || batch > 65535) return QUEST_ERR_SHAPE;
  if ((int64_t)batch * dm.Hq > ((int64_t)1 << 19)) return QUEST_ERR_SHAPE;
  return QUEST_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? QUEST_OK : QUEST_ERR_HIP; }

// Validation shared by quest_decode_step and quest_decode_step_noalloc
// (everything but the workspace).
int check_decode_step(const quest_layout *layout, int32_t batch, const void *q,
                      const void *k_new, const void *v_new, const int32_t *cu_new,
                      const int32_t *ctx_before, int32_t max_new_per_seq,
                      const int32_t *page_table, const void *k_cache, const void *v_cache,
                      const void *kmeta, int32_t group_reduce, const int32_t *ctx_lens,
                      const int32_t *budget_tokens, int32_t max_k, int32_t n_sink,
                      int32_t n_recent, float sm_scale, const float *scores,
                      const int32_t *sel_pages, const int32_t *num_sel, const void *out,
                      Dims &dm) {
  int st = check_layout(layout, dm);
  if (st != QUEST_OK) return st;
  if ((st = check_batch(batch, dm)) != QUEST_OK) return st;
  if (max_new_per_seq < 0 || max_k <= 0 || n_sink < 0 || n_recent < 0) return QUEST_ERR_SHAPE;
  if (!std::isfinite(sm_scale)) return QUEST_ERR_SHAPE;
  if (group_reduce != QUEST_REDUCE_MAX && group_reduce != QUEST_REDUCE_SUM)
    return QUEST_ERR_UNSUPPORTED;
  if (batch == 0) return QUEST_OK;
  if (!q || !k_new || !v_new || !cu_new || !ctx_before || !page_table || !k_cache ||
      !v_cache || !kmeta || !ctx_lens || !budget_tokens || !scores || !sel_pages || !num_sel ||
      !out)
    return QUEST_ERR_NULL;
  if (dm.dtype == QUEST_BF16 && (!aligned16(q) || !aligned16(kmeta) || !aligned16(k_cache) ||
                                 !aligned16(v_cache)))
    return QUEST_ERR_SHAPE;
  return QUEST_OK;
}

}  // namespace

extern "C" {

int quest_abi_version(void) { return QUEST_ABI_VERSION; }

const char *quest_status_string(int status) {
  switch (status) {
    case QUEST_OK: return "ok";
    case QUEST_ERR_NULL: return "a required pointer is NULL";
    case QUEST_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case QUEST_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, page_size or group size";
    case QUEST_ERR_WORKSPACE: return "workspace missing or too small";
    case QUEST_ERR_ABI: return "layout abi_version does not match the library";
    case QUEST_ERR_HIP: return "the HIP runtime rejected a launch";
    case QUEST_ERR_SCRATCH:
      return "the step needs more than the library's static scratch (QUEST_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int quest_append_kv(const quest_layout *layout, int32_t batch, const void *k_new,
                    const void *v_new, const int32_t *cu_new, const int32_t *ctx_before,
                    int32_t max_new_per_seq, const int32_t *page_table, void *k_cache,
                    void *v_cache, void *kmeta, void *stream) {
  Dims dm;
  int st = check_layout(layout, dm);
  if (st != QUEST_OK) return st;
  if ((st = check_batch(batch, dm)) != QUEST_OK) return st;
  if (max_new_per_seq < 0) return QUEST_ERR_SHAPE;
  if (batch == 0) return QUEST_OK;
  if (!k_new || !v_new || !cu_new || !ctx_before || !page_table || !k_cache || !v_cache ||
      !kmeta)
    return QUEST_ERR_NULL;
  return launched(quest::launch_append(dm, batch, k_new, v_new, cu_new, ctx_before,
                                       max_new_per_seq, page_table, k_cache, v_cache, kmeta,
                                       (hipStream_t)stream));
}

int quest_page_scores(const quest_layout *layout, int32_t batch, const void *q,
                      const void *kmeta, const int32_t *page_table, const int32_t *ctx_lens,
                      int32_t group_reduce, float *scores, void *stream) {
  Dims dm;
  int st = check_layout(layout, dm);
  if (st != QUEST_OK) return st;
  if ((st = check_batch(batch, dm)) != QUEST_OK) return st;
  if (group_reduce != QUEST_REDUCE_MAX && group_reduce != QUEST_REDUCE_SUM)
    return QUEST_ERR_UNSUPPORTED;
  if (batch == 0) return QUEST_OK;
  if (!q || !kmeta || !page_table || !ctx_lens || !scores) return QUEST_ERR_NULL;
  if (dm.dtype == QUEST_BF16 && (!aligned16(q) || !aligned16(kmeta))) return QUEST_ERR_SHAPE;
  return launched(quest::launch_page_scores(dm, batch, q, kmeta, page_table, ctx_lens,
                                            group_reduce, scores, (hipStream_t)stream));
}

int quest_append_score(const quest_layout *layout, int32_t batch, const void *q,
                       const void *k_new, const void *v_new, const int32_t *cu_new,
                       const int32_t *ctx_before, int32_t max_new_per_seq,
                       const int32_t *page_table, void *k_cache, void *v_cache, void *kmeta,
                       int32_t group_reduce, float *scores, void *stream) {
  Dims dm;
  int st = check_layout(layout, dm);
  if (st != QUEST_OK) return st;
  if ((st = check_batch(batch, dm)) != QUEST_OK) return st;
  if (max_new_per_seq < 0) return QUEST_ERR_SHAPE;
  if (group_reduce != QUEST_REDUCE_MAX && group_reduce != QUEST_REDUCE_SUM)
    return QUEST_ERR_UNSUPPORTED;
  if (batch == 0) return QUEST_OK;
  if (!q || !k_new || !v_new || !cu_new || !ctx_before || !page_table || !k_cache ||
      !v_cache || !kmeta || !scores)
    return QUEST_ERR_NULL;
  if (dm.dtype == QUEST_BF16 && (!aligned16(q) || !aligned16(kmeta))) return QUEST_ERR_SHAPE;
  return launched(quest::launch_append_scores(dm, batch, q, k_new, v_new, cu_new, ctx_before,
                                              max_new_per_seq, page_table, k_cache, v_cache,
                                              kmeta, group_reduce, scores,
                                              (hipStream_t)stream));
}

int quest_topk_pages_forced(const quest_layout *layout, int32_t batch, const float *scores,
                            const int32_t *ctx_lens, const int32_t *budget_tokens,
                            int32_t max_k, int32_t n_sink, int32_t n_recent,
                            int32_t *sel_pages, int32_t *num_sel, void *stream) {
  Dims dm;
  int st = check_layout(layout, dm);
  if (st != QUEST_OK) return st;
  if ((st = check_batch(batch, dm)) != QUEST_OK) return st;
  if (max_k <= 0 || n_sink < 0 || n_recent < 0) return QUEST_ERR_SHAPE;
  if (batch == 0) return QUEST_OK;
  if (!scores || !ctx_lens || !budget_tokens || !sel_pages || !num_sel) return QUEST_ERR_NULL;
  return launched(quest::launch_topk(dm, batch, scores, ctx_lens, budget_tokens, max_k,
                                     n_sink, n_recent, sel_pages, num_sel,
                                     (hipStream_t)stream));
}

int quest_topk_pages(const quest_layout *layout, int32_t batch, const float *scores,
                     const int32_t *ctx_lens, const int32_t *budget_tokens, int32_t max_k,
                     int32_t *sel_pages, int32_t *num_sel, void *stream) {
  return quest_topk_pages_forced(layout, batch, scores, ctx_lens, budget_tokens, max_k, 0, 0,
                                 sel_pages, num_sel, stream);
}

size_t quest_sparse_decode_workspace_bytes(const quest_layout *layout, int32_t batch,
                                           int32_t max_k) {
  Dims dm;
  if (check_layout(layout, dm) != QUEST_OK || check_batch(batch, dm) != QUEST_OK ||
      max_k <= 0)
    return 0;
  return quest::decode_workspace_bytes(dm, batch, max_k);
}

int quest_sparse_decode_plan(const quest_layout *layout, int32_t batch, int32_t max_k,
                             int32_t *num_splits, int32_t *pages_per_split) {
  Dims dm;
  int st = check_layout(layout, dm);
  if (st != QUEST_OK) return st;
  if ((st = check_batch(batch, dm)) != QUEST_OK) return st;
  if (max_k <= 0) return QUEST_ERR_SHAPE;
  if (!num_splits || !pages_per_split) return QUEST_ERR_NULL;
  const quest::DecodePlan p = quest::decode_plan(dm, batch, max_k);
  *num_splits = p.n_split;
  *pages_per_split = p.pages_per_split;
  return QUEST_OK;
}

int quest_sparse_decode(const quest_layout *layout, int32_t batch, const void *q,
                        const void *k_cache, const void *v_cache, const int32_t *page_table,
                        const int32_t *ctx_lens, const int32_t *sel_pages,
                        const int32_t *num_sel, int32_t max_k, float sm_scale, void *out,
                        void *workspace, size_t workspace_bytes, void *stream) {
  Dims dm;
  int st = check_layout(layout, dm);
  if (st != QUEST_OK) return st;
  if ((st = check_batch(batch, dm)) != QUEST_OK) return st;
  if (max_k <= 0) return QUEST_ERR_SHAPE;
  if (!std::isfinite(sm_scale)) return QUEST_ERR_SHAPE;
  if (batch == 0) return QUEST_OK;
  if (!q || !k_cache || !v_cache || !page_table || !ctx_lens || !sel_pages || !num_sel || !out)
    return QUEST_ERR_NULL;
  if (dm.dtype == QUEST_BF16 &&
      (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)))
    return QUEST_ERR_SHAPE;
  const size_t need = quest::decode_workspace_bytes(dm, batch, max_k);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
    return QUEST_ERR_WORKSPACE;
  return launched(quest::launch_decode(dm, batch, q, k_cache, v_cache, page_table, ctx_lens,
                                       sel_pages, num_sel, max_k, sm_scale, out,
                                       (float *)workspace, (hipStream_t)stream));
}

int quest_topk_sparse_decode(const quest_layout *layout, int32_t batch, const void *q,
                             const void *k_cache, const void *v_cache,
                             const int32_t *page_table, const int32_t *ctx_lens,
                             const float *scores, const int32_t *budget_tokens, int32_t max_k,
                             int32_t n_sink, int32_t n_recent, float sm_scale,
                             int32_t *sel_pages, int32_t *num_sel, void *out, void *workspace,
                             size_t workspace_bytes, void *stream) {
  Dims dm;
  int st = check_layout(layout, dm);
  if (st != QUEST_OK) return st;
  if ((st = check_batch(batch, dm)) != QUEST_OK) return st;
  if (max_k <= 0 || n_sink < 0 || n_recent < 0) return QUEST_ERR_SHAPE;
  if (!std::isfinite(sm_scale)) return QUEST_ERR_SHAPE;
  if (batch == 0) return QUEST_OK;
  if (!q || !k_cache || !v_cache || !page_table || !ctx_lens || !scores || !budget_tokens ||
      !sel_pages || !num_sel || !out)
    return QUEST_ERR_NULL;
  if (dm.dtype == QUEST_BF16 &&
      (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)))
    return QUEST_ERR_SHAPE;
  const size_t need = quest::decode_workspace_bytes(dm, batch, max_k);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
    return QUEST_ERR_WORKSPACE;
  return launched(quest::launch_topk_decode(dm, batch, q, k_cache, v_cache, page_table,
                                            ctx_lens, scores, budget_tokens, max_k, n_sink,
                                            n_recent, sm_scale, sel_pages, num_sel, out,
                                            (float *)workspace, (hipStream_t)stream));
}

int quest_decode_step_noalloc(const quest_layout *layout, int32_t batch, const void *q,
                              const void *k_new, const void *v_new, const int32_t *cu_new,
                              const int32_t *ctx_before, int32_t max_new_per_seq,
                              const int32_t *page_table, void *k_cache, void *v_cache,
                              void *kmeta, int32_t group_reduce, const int32_t *ctx_lens,
                              const int32_t *budget_tokens, int32_t max_k, int32_t n_sink,
                              int32_t n_recent, float sm_scale, float *scores,
                              int32_t *sel_pages, int32_t *num_sel, void *out, void *stream) {
  Dims dm;
  const int st = check_decode_step(layout, batch, q, k_new, v_new, cu_new, ctx_before,
                                   max_new_per_seq, page_table, k_cache, v_cache, kmeta,
                                   group_reduce, ctx_lens, budget_tokens, max_k, n_sink,
                                   n_recent, sm_scale, scores, sel_pages, num_sel, out, dm);
  if (st != QUEST_OK || batch == 0) return st;
  if (quest::decode_workspace_bytes(dm, batch, max_k) > (size_t)QUEST_STATIC_SCRATCH_BYTES)
    return QUEST_ERR_SCRATCH;
  void *scratch = nullptr;
  if (quest::static_scratch(&scratch) != hipSuccess) return QUEST_ERR_HIP;
  return launched(quest::launch_decode_step(
      dm, batch, q, k_new, v_new, cu_new, ctx_before, max_new_per_seq, page_table, k_cache,
      v_cache, kmeta, group_reduce, ctx_lens, budget_tokens, max_k, n_sink, n_recent, sm_scale,
      scores, sel_pages, num_sel, out, (float *)scratch, (hipStream_t)stream));
}

int quest_decode_step(const quest_layout *layout, int32_t batch, const void *q,
                      const void *k_new, const void *v_new, const int32_t *cu_new,
                      const int32_t *ctx_before, int32_t max_new_per_seq,
                      const int32_t *page_table, void *k_cache, void *v_cache, void *kmeta,
                      int32_t group_reduce, const int32_t *ctx_lens,
                      const int32_t *budget_tokens, int32_t max_k, int32_t n_sink,
                      int32_t n_recent, float sm_scale, float *scores, int32_t *sel_pages,
                      int32_t *num_sel, void *out, void *workspace, size_t workspace_bytes,
                      void *stream) {
  Dims dm;
  const int st = check_decode_step(layout, batch, q, k_new, v_new, cu_new, ctx_before,
                                   max_new_per_seq, page_table, k_cache, v_cache, kmeta,
                                   group_reduce, ctx_lens, budget_tokens, max_k, n_sink,
                                   n_recent, sm_scale, scores, sel_pages, num_sel, out, dm);
  if (st != QUEST_OK || batch == 0) return st;
  const size_t need = quest::decode_workspace_bytes(dm, batch, max_k);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
    return QUEST_ERR_WORKSPACE;
  return launched(quest::launch_decode_step(
      dm, batch, q, k_new, v_new, cu_new, ctx_before, max_new_per_seq, page_table, k_cache,
      v_cache, kmeta, group_reduce, ctx_lens, budget_tokens, max_k, n_sink, n_recent, sm_scale,
      scores, sel_pages, num_sel, out, (float *)workspace, (hipStream_t)stream));
}

int quest_topk_sparse_decode_fused(const quest_layout *layout, int32_t batch, int32_t max_k) {
  Dims dm;
  int st = check_layout(layout, dm);
  if (st != QUEST_OK) return st;
  if ((st = check_batch(batch, dm)) != QUEST_OK) return st;
  if (max_k <= 0) return QUEST_ERR_SHAPE;
  return batch > 0 && quest::topk_decode_fused(dm, batch, max_k) ? 1 : 0;
}

int quest_topk_sparse_decode_plan(const quest_layout *layout, int32_t batch, int32_t max_k,
                                  int32_t *fused, int32_t *num_splits,
                                  int32_t *pages_per_split) {
  Dims dm;
  int st = check_layout(layout, dm);
  if (st != QUEST_OK) return st;
  if ((st = check_batch(batch, dm)) != QUEST_OK) return st;
  if (max_k <= 0) return QUEST_ERR_SHAPE;
  if (!fused || !num_splits || !pages_per_split) return QUEST_ERR_NULL;
  const bool one = batch > 0 && quest::topk_decode_fused(dm, batch, max_k);
  const quest::DecodePlan p =
      one ? quest::fused_plan(dm, batch, max_k) : quest::decode_plan(dm, batch, max_k);
  *fused = one ? 1 : 0;
  *num_splits = p.n_split;
  *pages_per_split = p.pages_per_split;
  return QUEST_OK;
}

}  // extern "C"
