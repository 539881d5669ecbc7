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

// One (page, KV head, 8 channels) unit of append_pages_kernel.
template <int P>
__device__ __forceinline__ void append_page_group(
    int Hkv, int D, int page, int64_t head, int g, int d0, int p0, int p1, int row0,
    const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
    uint16_t *__restrict__ k_cache, uint16_t *__restrict__ v_cache,
    uint16_t *__restrict__ kmeta) {
  const int lo_pos = max(p0, page * P), hi_pos = min(p1, (page + 1) * P);
  const bool fresh = lo_pos == page * P;

  float lo[8], hi[8];
  if (fresh) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      lo[c] = __builtin_huge_valf();
      hi[c] = -__builtin_huge_valf();
    }
  } else {
    const uint4 a = *(const uint4 *)(kmeta + (head * 2 + 0) * D + d0);
    const uint4 b = *(const uint4 *)(kmeta + (head * 2 + 1) * D + d0);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      lo[c] = bf16_bits_to_f32((aw[c / 2] >> (16 * (c & 1))) & 0xffffu);
      hi[c] = bf16_bits_to_f32((bw[c / 2] >> (16 * (c & 1))) & 0xffffu);
    }
  }
  // The page in blocks of SB slots (bounded registers for large pages); in
  // each block all loads first, clamped rows for slots outside the new range.
  constexpr int SB = P < 16 ? P : 16;
  for (int s0 = 0; s0 < P; s0 += SB) {
    const int b_lo = page * P + s0;
    if (b_lo + SB <= lo_pos || b_lo >= hi_pos) continue;  // no new slot here
    const bool full = lo_pos <= b_lo && b_lo + SB <= hi_pos;
    uint4 kv[SB], vv[SB];
#pragma unroll
    for (int s = 0; s < SB; ++s) {
      const int pos = min(max(b_lo + s, lo_pos), hi_pos - 1);
      const int64_t src = ((int64_t)(row0 + pos - p0) * Hkv + g) * D + d0;
      kv[s] = *(const uint4 *)(k_new + src);
      vv[s] = *(const uint4 *)(v_new + src);
    }
#pragma unroll
    for (int s = 0; s < SB; ++s) {
      const int pos = b_lo + s;
      if (pos < lo_pos || pos >= hi_pos) continue;
      *(uint4 *)(k_cache + (head * P + s0 + s) * D + d0) = kv[s];
      const uint32_t w[4] = {kv[s].x, kv[s].y, kv[s].z, kv[s].w};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float x = bf16_bits_to_f32((w[c / 2] >> (16 * (c & 1))) & 0xffffu);
        if (x < lo[c]) lo[c] = x;
        if (x > hi[c]) hi[c] = x;
      }
    }
    // V: channel d0 + c of the page is the row (head * D + d0 + c) of P slots;
    // this block is its slots s0 .. s0 + SB - 1
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint16_t *vrow = v_cache + (head * D + d0 + c) * P + s0;
      const int sh = 16 * (c & 1);
      if (full) {
        uint32_t out[SB / 2];
#pragma unroll
        for (int t = 0; t < SB / 2; ++t) {
          const uint32_t *x0 = (const uint32_t *)&vv[2 * t];
          const uint32_t *x1 = (const uint32_t *)&vv[2 * t + 1];
          out[t] = ((x0[c / 2] >> sh) & 0xffffu) | (((x1[c / 2] >> sh) & 0xffffu) << 16);
        }
#pragma unroll
        for (int t = 0; t < SB / 8; ++t)
          *(uint4 *)(vrow + 8 * t) =
              make_uint4(out[4 * t], out[4 * t + 1], out[4 * t + 2], out[4 * t + 3]);
      } else {
#pragma unroll
        for (int s = 0; s < SB; ++s) {
          const int pos = b_lo + s;
          if (pos < lo_pos || pos >= hi_pos) continue;
          const uint32_t *x0 = (const uint32_t *)&vv[s];
          vrow[s] = (uint16_t)((x0[c / 2] >> sh) & 0xffffu);
        }
      }
    }
  }
  // lo and hi are stored values (or the unchanged metadata): exact in bf16
  uint32_t lw[4], hw[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    lw[t] = (__float_as_uint(lo[2 * t]) >> 16) | (__float_as_uint(lo[2 * t + 1]) & 0xffff0000u);
    hw[t] = (__float_as_uint(hi[2 * t]) >> 16) | (__float_as_uint(hi[2 * t + 1]) & 0xffff0000u);
  }
  *(uint4 *)(kmeta + (head * 2 + 0) * D + d0) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  *(uint4 *)(kmeta + (head * 2 + 1) * D + d0) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
}

// bf16 with 16-byte aligned tensors: one thread per (page, KV head, group of
// 8 channels), so at Hkv = 4, D = 128 a wave covers one page.  Every new
// token's 8 channels of K and V arrive as one 16-byte load each; K is stored
// 16 bytes at a time (token-major); V is held for the whole page and
// transposed in registers, so a page whose slots are all new writes each
// channel's P slots as P*2 contiguous bytes (dim-major).  Positions are
// visited in order with the same strict comparisons as append_channel, so the
// metadata matches it bit for bit.
template <int P>
__global__ __launch_bounds__(256) void append_pages_kernel(
    int Hkv, int D, int64_t pool, int max_pages, const uint16_t *__restrict__ k_new,
    const uint16_t *__restrict__ v_new, const int32_t *__restrict__ cu_new,
    const int32_t *__restrict__ ctx_before, const int32_t *__restrict__ page_table,
    uint16_t *__restrict__ k_cache, uint16_t *__restrict__ v_cache,
    uint16_t *__restrict__ kmeta) {
  const int r = blockIdx.y;
  const int row0 = cu_new[r];
  const int n_new = cu_new[r + 1] - row0;
  if (n_new <= 0) return;
  const int p0 = ctx_before[r];
  if (p0 < 0) return;
  const int p1 = p0 + n_new;                 // exclusive
  const int groups = D / 8;                  // channel groups per KV head
  const int per_page = Hkv * groups;
  const int64_t units = (int64_t)((p1 - 1) / P - p0 / P + 1) * per_page;
  for (int64_t unit = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; unit < units;
       unit += (int64_t)gridDim.x * blockDim.x) {
    const int64_t page64 = p0 / P + unit / per_page;
    if (page64 >= max_pages) break;
    const int rem = (int)(unit % per_page);
    const int g = rem / groups, d0 = (rem - g * groups) * 8;
    const int64_t phys = page_table[(int64_t)r * max_pages + page64];
    if (phys < 0 || phys >= pool) continue;
    append_page_group<P>(Hkv, D, (int)page64, phys * Hkv + g, g, d0, p0, p1, row0, k_new, v_new,
                         k_cache, v_cache, kmeta);
  }
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

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
  } else if (aligned16(k_new) && aligned16(v_new) && aligned16(k_cache) &&
             aligned16(v_cache) && aligned16(kmeta) && dm.D % 8 == 0) {
    const long units = pages * dm.Hkv * (dm.D / 8);
    dim3 vgrid((unsigned)((units + 255) / 256), (unsigned)batch);
#define QUEST_APPEND_PAGES(PP)                                                            \
  hipLaunchKernelGGL(append_pages_kernel<PP>, vgrid, block, 0, stream, dm.Hkv, dm.D, dm.pool,   \
                     dm.max_pages, (const uint16_t *)k_new, (const uint16_t *)v_new, cu_new,   \
                     ctx_before, page_table, (uint16_t *)k_cache, (uint16_t *)v_cache,        \
                     (uint16_t *)kmeta)
    if (dm.P == 8) QUEST_APPEND_PAGES(8);
    else if (dm.P == 16) QUEST_APPEND_PAGES(16);
    else if (dm.P == 32) QUEST_APPEND_PAGES(32);
    else QUEST_APPEND_PAGES(64);
#undef QUEST_APPEND_PAGES
  } else {
    hipLaunchKernelGGL(append_kv_kernel<uint16_t>, grid, block, 0, stream, dm.Hkv, dm.D,
                       dm.P, dm.pool, dm.max_pages, (const uint16_t *)k_new,
                       (const uint16_t *)v_new, cu_new, ctx_before, page_table,
                       (uint16_t *)k_cache, (uint16_t *)v_cache, (uint16_t *)kmeta);
  }
  return hipGetLastError();
}

}  // namespace quest
