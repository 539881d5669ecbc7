// hbm_probe.hip -- measurement kernels (libquest_probe.so, include/quest_probe.h):
// what plain reads of HBM achieve on this chip, for the two access patterns
// of the Quest decode step, so the step's kernels can be reported against
// the practical read rate as well as the nameplate peak.
//   stream read: a contiguous buffer read once with 16-byte loads (the
//                pattern of the page-metadata scan);
//   chunk gather: whole chunks (one K page and one V page of one KV head)
//                at scattered offsets (the pattern of the selected-page
//                reads).
// Each kernel folds what it loads into an XOR that is stored only when it
// equals a value the caller passes and no data can produce in practice, so
// no load is dead code and nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "quest_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__device__ __forceinline__ uint32_t fold(uint4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4 *__restrict__ p,
                                                               size_t n16, uint32_t never,
                                                               uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= fold(v[u]);
  }
  for (; i < n16; i += stride) acc ^= fold(p[i]);
  if (acc == never) sink[0] = acc;
}

// One wave per chunk pair (K chunk and V chunk at the same element offset),
// all of a lane's loads of the pair issued before the first use.
template <int kPer>
__global__ __launch_bounds__(kThreads) void gather_read_kernel(
    const uint4 *__restrict__ a, const uint4 *__restrict__ b, const int64_t *__restrict__ offs,
    int n_chunks, uint32_t never, uint32_t *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int waves = gridDim.x * (kThreads / 64);
  uint32_t acc = 0;
  for (int c = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); c < n_chunks; c += waves) {
    const int64_t o = offs[c];
    uint4 va[kPer], vb[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) va[u] = a[o + u * 64 + lane];
#pragma unroll
    for (int u = 0; u < kPer; ++u) vb[u] = b[o + u * 64 + lane];
#pragma unroll
    for (int u = 0; u < kPer; ++u) acc ^= fold(va[u]) ^ fold(vb[u]);
  }
  if (acc == never) sink[0] = acc;
}

}  // namespace

extern "C" {

int quest_probe_stream_read(const void *buf, size_t bytes, int work_groups, uint32_t never,
                            uint32_t *sink, void *stream) {
  if (buf == nullptr || sink == nullptr) return -1;
  if (bytes % 16 != 0 || ((uintptr_t)buf & 15u) != 0 || work_groups <= 0) return -2;
  if (bytes == 0) return 0;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)work_groups), dim3(kThreads), 0,
                     (hipStream_t)stream, (const uint4 *)buf, bytes / 16, never, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int quest_probe_gather_read(const void *a, const void *b, const int64_t *chunk_offsets16,
                            int n_chunks, int chunk_bytes, int work_groups, uint32_t never,
                            uint32_t *sink, void *stream) {
  if (a == nullptr || b == nullptr || chunk_offsets16 == nullptr || sink == nullptr) return -1;
  if (((uintptr_t)a & 15u) != 0 || ((uintptr_t)b & 15u) != 0 || n_chunks < 0 ||
      work_groups <= 0)
    return -2;
  if (n_chunks == 0) return 0;
  const hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)work_groups), block(kThreads);
  switch (chunk_bytes) {
    case 2048:
      hipLaunchKernelGGL(gather_read_kernel<2>, grid, block, 0, s, (const uint4 *)a,
                         (const uint4 *)b, chunk_offsets16, n_chunks, never, sink);
      break;
    case 4096:
      hipLaunchKernelGGL(gather_read_kernel<4>, grid, block, 0, s, (const uint4 *)a,
                         (const uint4 *)b, chunk_offsets16, n_chunks, never, sink);
      break;
    case 8192:
      hipLaunchKernelGGL(gather_read_kernel<8>, grid, block, 0, s, (const uint4 *)a,
                         (const uint4 *)b, chunk_offsets16, n_chunks, never, sink);
      break;
    default:
      return -3;
  }
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
