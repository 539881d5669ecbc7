// quest_launch.h -- internal interface between the C ABI (quest_abi.cpp) and
// the kernel files.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "quest_plan.h"

namespace quest {

hipError_t launch_append(const Dims &dm, int batch, const void *k_new,
                         const void *v_new, const int32_t *cu_new,
                         const int32_t *ctx_before, int max_new,
                         const int32_t *page_table, void *k_cache,
                         void *v_cache, void *kmeta, hipStream_t stream);

hipError_t launch_page_scores(const Dims &dm, int batch, const void *q,
                              const void *kmeta, const int32_t *page_table,
                              const int32_t *ctx_lens, int reduce,
                              float *scores, hipStream_t stream);

// on_kv_stored and the page scores in one pass over the metadata (bf16: one
// kernel; fp32: two launches).  Request lengths are ctx_before + new tokens.
hipError_t launch_append_scores(const Dims &dm, int batch, const void *q, const void *k_new,
                                const void *v_new, const int32_t *cu_new,
                                const int32_t *ctx_before, int max_new,
                                const int32_t *page_table, void *k_cache, void *v_cache,
                                void *kmeta, int reduce, float *scores, hipStream_t stream);

// n_sink / n_recent >= 0: the first / last pages of each request kept first.
hipError_t launch_topk(const Dims &dm, int batch, const float *scores,
                       const int32_t *ctx_lens, const int32_t *budget_tokens,
                       int max_k, int n_sink, int n_recent, int32_t *sel_pages,
                       int32_t *num_sel, hipStream_t stream);

hipError_t launch_decode(const Dims &dm, int batch, const void *q,
                         const void *k_cache, const void *v_cache,
                         const int32_t *page_table, const int32_t *ctx_lens,
                         const int32_t *sel_pages, const int32_t *num_sel,
                         int max_k, float sm_scale, void *out,
                         float *workspace, hipStream_t stream);

// Top-k (forced pages as in launch_topk) then the decode of the selection;
// one kernel where topk_decode_fused() says so, else launch_topk +
// launch_decode.
hipError_t launch_topk_decode(const Dims &dm, int batch, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *page_table,
                              const int32_t *ctx_lens, const float *scores,
                              const int32_t *budget_tokens, int max_k, int n_sink,
                              int n_recent, float sm_scale, int32_t *sel_pages,
                              int32_t *num_sel, void *out, float *workspace,
                              hipStream_t stream);

// The whole decode step: launch_append_scores, then launch_topk_decode on
// its scores.
hipError_t launch_decode_step(const Dims &dm, int batch, const void *q, const void *k_new,
                              const void *v_new, const int32_t *cu_new,
                              const int32_t *ctx_before, int max_new,
                              const int32_t *page_table, void *k_cache, void *v_cache,
                              void *kmeta, int reduce, const int32_t *ctx_lens,
                              const int32_t *budget_tokens, int max_k, int n_sink,
                              int n_recent, float sm_scale, float *scores,
                              int32_t *sel_pages, int32_t *num_sel, void *out,
                              float *workspace, hipStream_t stream);

// This device's copy of the library-owned scratch array of
// QUEST_STATIC_SCRATCH_BYTES (the current device's; looked up on first use).
hipError_t static_scratch(void **ptr);

}  // namespace quest
