// topk_pages.hip -- the top-k kernel: one 1024-thread work-group per
// (request, selection row) runs the row selection of topk_select.h and
// writes the kept pages in ascending order.
#include "quest_launch.h"
#include "topk_select.h"

namespace quest {

template <bool kRegs>
__global__ __launch_bounds__(kTopkThreads) void topk_pages_kernel(
    int R, int P, int max_pages, int max_k, int n_sink, int n_recent,
    const float *__restrict__ scores, const int32_t *__restrict__ ctx_lens,
    const int32_t *__restrict__ budget_tokens, int32_t *__restrict__ sel_pages,
    int32_t *__restrict__ num_sel) {
  __shared__ TopkShared sh;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  // grid (selection row, request): no division by runtime values
  const int r = blockIdx.y;
  const int row = r * R + (int)blockIdx.x;
  const int log2p = __builtin_ctz(P);                 // the page size is a power of two
  const float *s = scores + (int64_t)row * max_pages;
  const int span = reg_span(max_pages);               // pages per wave of a register row
  // Register rows: the whole score row is loaded in the same round trip as
  // the request's length and budget (entries past the length are ignored).
  float sv[kRegs ? kPerThread : 1];
  if constexpr (kRegs) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int j = wave * span + i * kWave + lane;
      sv[i] = s[min(j, max_pages - 1)];
    }
  }
  const int ctx = ctx_lens[r];
  int n, k;
  row_size(ctx, budget_tokens[r], log2p, max_pages, max_k, n, k);
  int32_t *out = sel_pages + (int64_t)row * max_k;
  if (tid == 0) num_sel[row] = k;
  for (int i = k + tid; i < max_k; i += kTopkThreads) out[i] = -1;
  auto emit = [&](int pos, int j) { out[pos] = j; };
  if (n_sink > 0 || n_recent > 0) select_row<kRegs, true>(sh, s, sv, span, n, k, n_sink, n_recent, emit);
  else select_row<kRegs, false>(sh, s, sv, span, n, k, 0, 0, emit);
}

hipError_t launch_topk(const Dims &dm, int batch, const float *scores,
                       const int32_t *ctx_lens, const int32_t *budget_tokens,
                       int max_k, int n_sink, int n_recent, int32_t *sel_pages,
                       int32_t *num_sel, hipStream_t stream) {
  dim3 grid((unsigned)dm.R, (unsigned)batch);        // one work-group per selection row
  if (dm.max_pages <= kRegKeys)
    hipLaunchKernelGGL(topk_pages_kernel<true>, grid, dim3(kTopkThreads), 0, stream, dm.R,
                       dm.P, dm.max_pages, max_k, n_sink, n_recent, scores, ctx_lens,
                       budget_tokens, sel_pages, num_sel);
  else
    hipLaunchKernelGGL(topk_pages_kernel<false>, grid, dim3(kTopkThreads), 0, stream, dm.R,
                       dm.P, dm.max_pages, max_k, n_sink, n_recent, scores, ctx_lens,
                       budget_tokens, sel_pages, num_sel);
  return hipGetLastError();
}

}  // namespace quest
