// append_inline.h -- the per-channel body of on_kv_stored, shared by the
// standalone append kernel and the fused append + score kernel.
//
// For one (page, KV head, channel d): stores channel d of the page's new
// tokens into their slots (K token-major, V dim-major) and refreshes the
// page's min/max of that channel.  The comparisons are strict (x < lo,
// x > hi), which keeps the first-seen value among equal ones, so an
// incremental update equals a from-scratch scan of the page in position order
// bit for bit (signed zeros included).
#pragma once

#include "quest_device.h"

namespace quest {

struct AppendSpan {
  int64_t head;     // phys * Hkv + g
  int g;
  int page;         // logical page
  int lo_pos;       // first new position in the page
  int hi_pos;       // one past the last new position in the page
  int p0;           // first new position of the request
  int row0;         // row of the request's first new token in k_new / v_new
  bool fresh;       // the first new token sits at slot 0: restart the min/max
};

// The new positions [p0, p1) that fall in logical page `page`.
__device__ __forceinline__ AppendSpan append_span(int64_t phys, int Hkv, int g, int P, int page,
                                                  int p0, int p1, int row0) {
  AppendSpan a;
  a.head = phys * Hkv + g;
  a.g = g;
  a.page = page;
  a.lo_pos = max(p0, page * P);
  a.hi_pos = min(p1, (page + 1) * P);
  a.p0 = p0;
  a.row0 = row0;
  a.fresh = (a.lo_pos == page * P);
  return a;
}

template <typename T>
__device__ __forceinline__ void append_channel(const AppendSpan &a, int d, int Hkv, int D, int P,
                                               const T *__restrict__ k_new,
                                               const T *__restrict__ v_new,
                                               T *__restrict__ k_cache, T *__restrict__ v_cache,
                                               T *__restrict__ kmeta) {
  float lo, hi;
  if (a.fresh) {
    lo = __builtin_huge_valf();
    hi = -__builtin_huge_valf();
  } else {
    lo = Elem<T>::load(kmeta, (a.head * 2 + 0) * D + d);
    hi = Elem<T>::load(kmeta, (a.head * 2 + 1) * D + d);
  }
  for (int pos = a.lo_pos; pos < a.hi_pos; ++pos) {
    const int64_t src = ((int64_t)(a.row0 + pos - a.p0) * Hkv + a.g) * D + d;
    const int slot = pos - a.page * P;
    const T kx = k_new[src];
    k_cache[(a.head * P + slot) * D + d] = kx;
    v_cache[(a.head * D + d) * P + slot] = v_new[src];
    const float x = Elem<T>::load(&kx, 0);
    if (x < lo) lo = x;
    if (x > hi) hi = x;
  }
  // lo and hi are stored values (or the unchanged metadata), so writing them
  // back in the storage type is exact.
  Elem<T>::store(kmeta, (a.head * 2 + 0) * D + d, lo);
  Elem<T>::store(kmeta, (a.head * 2 + 1) * D + d, hi);
}

}  // namespace quest
