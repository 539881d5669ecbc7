// append_kv.hip -- on_kv_stored: store new K/V tokens into their page slots
// and refresh the pages' elementwise key min/max in the same pass.
//
// Sparse-vLLM skill "add-sparse-method", Placement Rules 2-3: the method's
// persistent page metadata lives with the cache and is updated after KV is
// written.  The metadata is Quest's per-page elementwise key min and max.
//
// One work-group owns one touched page of one request, so every metadata row
// has exactly one writer; its threads walk the page's (KV head, channel)
// pairs (append_inline.h holds the per-channel body).
#include "append_inline.h"
#include "quest_launch.h"

namespace quest {

template <typename T>
__global__ __launch_bounds__(256) void append_kv_kernel(
    int Hkv, int D, int P, int64_t pool, int max_pages,
    const T *__restrict__ k_new, const T *__restrict__ v_new,
    const int32_t *__restrict__ cu_new, const int32_t *__restrict__ ctx_before,
    const int32_t *__restrict__ page_table, T *__restrict__ k_cache,
    T *__restrict__ v_cache, T *__restrict__ kmeta) {
  const int r = blockIdx.y;
  const int row0 = cu_new[r];
  const int n_new = cu_new[r + 1] - row0;
  if (n_new <= 0) return;
  const int p0 = ctx_before[r];
  if (p0 < 0) return;
  const int p1 = p0 + n_new;                 // exclusive
  const int first_page = p0 / P;
  const int last_page = (p1 - 1) / P;
  const int32_t *pt = page_table + (int64_t)r * max_pages;

  for (int page = first_page + (int)blockIdx.x; page <= last_page; page += gridDim.x) {
    if (page >= max_pages) break;
    const int64_t phys = pt[page];
    if (phys < 0 || phys >= pool) continue;
    for (int e = threadIdx.x; e < Hkv * D; e += blockDim.x) {
      const int g = e / D, d = e - g * D;
      const AppendSpan a = append_span(phys, Hkv, g, P, page, p0, p1, row0);
      append_channel<T>(a, d, Hkv, D, P, k_new, v_new, k_cache, v_cache, kmeta);
    }
  }
}

hipError_t launch_append(const Dims &dm, int batch, const void *k_new,
                         const void *v_new, const int32_t *cu_new,
                         const int32_t *ctx_before, int max_new,
                         const int32_t *page_table, void *k_cache,
                         void *v_cache, void *kmeta, hipStream_t stream) {
  // A request's new tokens touch at most ceil(max_new / P) + 1 pages.
  long pages = (long)(max_new + dm.P - 1) / dm.P + 1;
  if (pages > 65535) pages = 65535;      // blocks loop over the rest
  if (pages < 1) pages = 1;
  dim3 grid((unsigned)pages, (unsigned)batch);
  dim3 block(256);
  if (dm.dtype == 0) {
    hipLaunchKernelGGL(append_kv_kernel<float>, grid, block, 0, stream, dm.Hkv, dm.D,
                       dm.P, dm.pool, dm.max_pages, (const float *)k_new,
                       (const float *)v_new, cu_new, ctx_before, page_table,
                       (float *)k_cache, (float *)v_cache, (float *)kmeta);
  } else {
    hipLaunchKernelGGL(append_kv_kernel<uint16_t>, grid, block, 0, stream, dm.Hkv, dm.D,
                       dm.P, dm.pool, dm.max_pages, (const uint16_t *)k_new,
                       (const uint16_t *)v_new, cu_new, ctx_before, page_table,
                       (uint16_t *)k_cache, (uint16_t *)v_cache, (uint16_t *)kmeta);
  }
  return hipGetLastError();
}

}  // namespace quest
