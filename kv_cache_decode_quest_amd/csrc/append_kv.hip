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

// Position-ordered min / max of two partial results, the earlier positions'
// on the left: the left value is kept on ties, as a scan in position order
// with strict comparisons keeps the first-seen one.
__device__ __forceinline__ float first_min(float left, float right) {
  return right < left ? right : left;
}
__device__ __forceinline__ float first_max(float left, float right) {
  return right > left ? right : left;
}

// bf16, 16-byte aligned tensors, D 64 or 128: one wave per (page, KV head)
// of a request's new tokens.  Lane l holds the 8 channels of group
// cg = l % (D / 8) for the page slots tq * kSlots .. tq * kSlots + kSlots - 1,
// tq = l / (D / 8): every new token's 8 channels of K and of V arrive as one
// 16-byte load each, K is stored 16 bytes per token (token-major), V as
// kSlots slots per channel (dim-major).  Each lane scans its slots in
// position order; the token groups are then combined in position order
// (earlier slots on the left), so the page's min / max are the first-seen
// values a single scan in position order would keep, bit for bit.
template <int P, int D>
__global__ __launch_bounds__(256) void append_pages_kernel(
    int Hkv, int64_t pool, int max_pages, const uint16_t *__restrict__ k_new,
    const uint16_t *__restrict__ v_new, const int32_t *__restrict__ cu_new,
    const int32_t *__restrict__ ctx_before, const int32_t *__restrict__ page_table,
    uint16_t *__restrict__ k_cache, uint16_t *__restrict__ v_cache,
    uint16_t *__restrict__ kmeta) {
  constexpr int kGroups = D / 8;                 // channel groups per KV head
  constexpr int kTokenGroups = kWave / kGroups;  // 4 at D 128, 8 at D 64
  constexpr int kSlots = P / kTokenGroups;       // page slots per lane
  constexpr int SB = kSlots < 8 ? kSlots : 8;    // slots loaded at once
  static_assert(kSlots >= 1 && kSlots % SB == 0, "page size vs head size");
  const int lane = lane_id();
  const int cg = lane % kGroups, tq = lane / kGroups;
  const int r = blockIdx.y;
  const int row0 = cu_new[r];
  const int n_new = cu_new[r + 1] - row0;
  if (n_new <= 0) return;
  const int p0 = ctx_before[r];
  if (p0 < 0) return;
  const int p1 = p0 + n_new;                 // exclusive
  const int first = p0 / P;
  const int64_t units = (int64_t)((p1 - 1) / P - first + 1) * Hkv;
  const int waves = blockDim.x / kWave;
  for (int64_t u = (int64_t)blockIdx.x * waves + (threadIdx.x >> 6); u < units;
       u += (int64_t)gridDim.x * waves) {
    const int64_t page64 = first + u / Hkv;
    if (page64 >= max_pages) break;
    const int page = (int)page64, g = (int)(u % Hkv);
    const int64_t phys = page_table[(int64_t)r * max_pages + page];
    if (phys < 0 || phys >= pool) continue;
    const int64_t head = phys * Hkv + g;
    const int lo_pos = max(p0, page * P), hi_pos = min(p1, (page + 1) * P);

    float lo[8], hi[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      lo[c] = __builtin_huge_valf();
      hi[c] = -__builtin_huge_valf();
    }
#pragma unroll
    for (int s0 = 0; s0 < kSlots; s0 += SB) {
      const int slot0 = tq * kSlots + s0;
      const int b_lo = page * P + slot0;
      // all loads first, from clamped rows for slots outside the new range
      uint4 kv[SB], vv[SB];
#pragma unroll
      for (int s = 0; s < SB; ++s) {
        const int pos = min(max(b_lo + s, lo_pos), hi_pos - 1);
        const int64_t src = ((int64_t)(row0 + pos - p0) * Hkv + g) * D + cg * 8;
        kv[s] = *(const uint4 *)(k_new + src);
        vv[s] = *(const uint4 *)(v_new + src);
      }
#pragma unroll
      for (int s = 0; s < SB; ++s) {
        const int pos = b_lo + s;
        if (pos < lo_pos || pos >= hi_pos) continue;
        *(uint4 *)(k_cache + (head * P + slot0 + s) * D + cg * 8) = kv[s];
        const uint32_t w[4] = {kv[s].x, kv[s].y, kv[s].z, kv[s].w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float x = bf16_bits_to_f32((w[c / 2] >> (16 * (c & 1))) & 0xffffu);
          if (x < lo[c]) lo[c] = x;
          if (x > hi[c]) hi[c] = x;
        }
      }
      // V: channel cg * 8 + c of the page is the row (head * D + cg * 8 + c)
      // of P slots; this lane's part of it is slots slot0 .. slot0 + SB - 1
      const bool full = lo_pos <= b_lo && b_lo + SB <= hi_pos;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint16_t *vrow = v_cache + (head * D + cg * 8 + c) * P + slot0;
        const int sh = 16 * (c & 1);
        uint32_t h[SB];
#pragma unroll
        for (int s = 0; s < SB; ++s) {
          const uint32_t *x = (const uint32_t *)&vv[s];
          h[s] = (x[c / 2] >> sh) & 0xffffu;
        }
        if (full) {
          if constexpr (SB == 1) {
            vrow[0] = (uint16_t)h[0];
          } else if constexpr (SB == 2) {
            *(uint32_t *)vrow = h[0] | (h[1] << 16);
          } else if constexpr (SB == 4) {
            *(uint2 *)vrow = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
          } else {
            *(uint4 *)vrow = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                        h[4] | (h[5] << 16), h[6] | (h[7] << 16));
          }
        } else {
#pragma unroll
          for (int s = 0; s < SB; ++s) {
            const int pos = b_lo + s;
            if (pos >= lo_pos && pos < hi_pos) vrow[s] = (uint16_t)h[s];
          }
        }
      }
    }
    // token groups in position order: pairs of lane rows (xor 16), then
    // halves (xor 32); at D 64 first the two token groups of a row (xor 8)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if constexpr (kTokenGroups == 8) {
        const float olo = __shfl_xor(lo[c], 8, kWave), ohi = __shfl_xor(hi[c], 8, kWave);
        const bool left = (tq & 1) == 0;
        lo[c] = left ? first_min(lo[c], olo) : first_min(olo, lo[c]);
        hi[c] = left ? first_max(hi[c], ohi) : first_max(ohi, hi[c]);
      }
      float a, b;
      pair_xor16(lo[c], a, b);
      lo[c] = first_min(a, b);
      pair_xor32(lo[c], a, b);
      lo[c] = first_min(a, b);
      pair_xor16(hi[c], a, b);
      hi[c] = first_max(a, b);
      pair_xor32(hi[c], a, b);
      hi[c] = first_max(a, b);
    }
    if (tq == 0) {
      uint16_t *mlo = kmeta + (head * 2 + 0) * D + cg * 8;
      uint16_t *mhi = kmeta + (head * 2 + 1) * D + cg * 8;
      if (lo_pos != page * P) {                // the page's earlier slots come first
        const uint4 a = *(const uint4 *)mlo, b = *(const uint4 *)mhi;
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          lo[c] = first_min(bf16_bits_to_f32((aw[c / 2] >> (16 * (c & 1))) & 0xffffu), lo[c]);
          hi[c] = first_max(bf16_bits_to_f32((bw[c / 2] >> (16 * (c & 1))) & 0xffffu), hi[c]);
        }
      }
      // lo and hi are stored values (or the unchanged metadata): exact in bf16
      uint32_t lw[4], hw[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        lw[t] = (__float_as_uint(lo[2 * t]) >> 16) | (__float_as_uint(lo[2 * t + 1]) & 0xffff0000u);
        hw[t] = (__float_as_uint(hi[2 * t]) >> 16) | (__float_as_uint(hi[2 * t + 1]) & 0xffff0000u);
      }
      *(uint4 *)mlo = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      *(uint4 *)mhi = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    }
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
             aligned16(v_cache) && aligned16(kmeta) && (dm.D == 64 || dm.D == 128)) {
    // one wave per (page, KV head), 4 waves per work-group; blocks loop over
    // the rest past the grid limit
    long wgs = (pages * dm.Hkv + 3) / 4;
    if (wgs > 65535) wgs = 65535;
    dim3 vgrid((unsigned)wgs, (unsigned)batch);
#define QUEST_APPEND_PAGES(PP, DD)                                                        \
  hipLaunchKernelGGL((append_pages_kernel<PP, DD>), vgrid, block, 0, stream, dm.Hkv, dm.pool, \
                     dm.max_pages, (const uint16_t *)k_new, (const uint16_t *)v_new, cu_new,   \
                     ctx_before, page_table, (uint16_t *)k_cache, (uint16_t *)v_cache,        \
                     (uint16_t *)kmeta)
#define QUEST_APPEND_PAGES_D(PP) \
  if (dm.D == 128) QUEST_APPEND_PAGES(PP, 128); else QUEST_APPEND_PAGES(PP, 64)
    if (dm.P == 8) { QUEST_APPEND_PAGES_D(8); }
    else if (dm.P == 16) { QUEST_APPEND_PAGES_D(16); }
    else if (dm.P == 32) { QUEST_APPEND_PAGES_D(32); }
    else { QUEST_APPEND_PAGES_D(64); }
#undef QUEST_APPEND_PAGES_D
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
