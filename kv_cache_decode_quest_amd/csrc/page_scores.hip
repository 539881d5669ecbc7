// page_scores.hip -- build_decode_view, part 1: Quest page upper bounds.
//
// For request r, KV head g, logical page j and each q head h of g's group:
//     U[h][j] = sum_d max(q_hd * min_jd, q_hd * max_jd)
// (Quest's bound on q.k over the page's min/max box; SparseEngine digest,
// Method key points: query-relevant page selection through the decode-time q).
// The KV head's score is the max (or sum) of U over its G q heads.
//
// bf16 path (matrix cores).  With q+ = max(q, 0) and q- = min(q, 0),
//     max(q*a, q*b) = q+ * b + q- * a     whenever a <= b,
// so U = [q- | q+] . [min | max]: a dot product of length 2D against the
// page's metadata row, which is stored exactly in that order ([min][D] then
// [max][D]).  A 16-page tile of one KV head is then a skinny GEMM
//     C[16 heads][16 pages] = A[16 heads][2D] * B[2D][16 pages]
// run as 2D/32 v_mfma_f32_16x16x32_bf16 steps.  Heads past G are zero rows.
// Every product of two bf16 values is exact in fp32 and the zero halves add
// exact zeros, so the only rounding is the fp32 accumulation.  The kernel is
// bound by streaming the metadata (512 B per page and KV head at D = 128);
// the matrix cores only remove the per-element select/multiply work that
// would otherwise load the vector ALUs at HBM speed.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 on a 64-lane wave: lane l holds
// row (l % 16) of A and column (l % 16) of B, each for the eight K slots of
// group l / 16; the 16x16 fp32 result gives lane l column l % 16, rows
// 4*(l/16) .. 4*(l/16)+3.  Both operands use the same (group, element) -> k
// assignment, so the sum over k is exact whatever order the unit uses inside.
#include "append_inline.h"
#include "quest_launch.h"

namespace quest {

constexpr int kScoreTilesPerWave = 1;
constexpr int kScoreWaves = 4;
constexpr int kScorePagesPerBlock = kScoreWaves * kScoreTilesPerWave * 16;

// Splits 16 B of bf16 q values into their negative and positive parts,
// halfword by halfword, by the sign bit (-0 goes to the negative part, where
// it still contributes an exact zero).
__device__ __forceinline__ void split_signs(uint4 w, uint4 &neg, uint4 &pos) {
  uint32_t in[4] = {w.x, w.y, w.z, w.w}, n[4], p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t m = ((in[i] & 0x80008000u) >> 15) * 0xffffu;
    n[i] = in[i] & m;
    p[i] = in[i] & ~m;
  }
  neg = make_uint4(n[0], n[1], n[2], n[3]);
  pos = make_uint4(p[0], p[1], p[2], p[3]);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 w) {
  return __builtin_bit_cast(bf16x8, w);
}

// New tokens to store before scoring (the fused on_kv_stored + scores path);
// all null in the plain scoring path.
struct FusedAppend {
  const uint16_t *k_new, *v_new;
  const int32_t *cu_new, *ctx_before;
  uint16_t *k_cache, *v_cache;
};

// per_head: no group reduction; q head h of KV head g writes its own score
// row r * Hq + g * G + h (selection per q head).
template <int D, bool kAppend>
__global__ __launch_bounds__(256) void page_scores_mfma_kernel(
    int Hkv, int G, int per_head, int64_t pool, int P, int max_pages, int reduce,
    const uint16_t *__restrict__ q, uint16_t *kmeta,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ ctx_lens,
    FusedAppend fa, float *__restrict__ scores) {
  constexpr int kChunks = 2 * D / 32;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;          // head row of A, page column of B
  const int grp = lane >> 4;          // K-slot group
  const int g = blockIdx.x % Hkv;
  const int block = blockIdx.x / Hkv;
  const int r = blockIdx.y;
  int ctx, row0 = 0, p0 = 0, n_new = 0;
  if constexpr (kAppend) {
    // ctx_before read first: the compiler then issues the three length
    // loads together (one scalar round trip instead of two in a row)
    p0 = fa.ctx_before[r];
    row0 = fa.cu_new[r];
    const int row1 = fa.cu_new[r + 1];
    n_new = row1 - row0;
    ctx = p0 + (n_new > 0 ? n_new : 0);
  } else {
    ctx = ctx_lens[r];
  }
  const int n = pages_in(ctx, P, max_pages);
  const int base = block * kScorePagesPerBlock;
  if (base >= n) return;

  const int32_t *pt = page_table + (int64_t)r * max_pages;
  float *out = scores + (per_head ? (int64_t)(r * Hkv + g) * G : (int64_t)r * Hkv + g) *
                            max_pages;

  // Metadata row of this lane's page in each of the wave's tiles; pages past
  // the request read physical page 0 and are never written back, and a page
  // whose id lies outside the pool reads physical page 0 and scores -inf.
  int page[kScoreTilesPerWave];
  int64_t row[kScoreTilesPerWave];
#pragma unroll
  for (int t = 0; t < kScoreTilesPerWave; ++t) {
    page[t] = base + (t * kScoreWaves + wave) * 16 + col;
    row[t] = pt[page[t] < n ? page[t] : 0];
  }
  // q of head `col` of the group.  All loads in this kernel are
  // unconditional, from clamped in-bounds addresses, with unwanted lanes
  // masked afterwards: a load under a branch makes the compiler drain every
  // outstanding load at the join, which would serialise the prefetch.  Order
  // of issue: page ids, q, then all metadata tiles of the wave.
  uint4 qw[kChunks];
  {
    const int head = col < G ? col : 0;
    const uint16_t *qh = q + ((int64_t)r * Hkv * G + (int64_t)g * G + head) * D;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int k0 = c * 32 + grp * 8;
      qw[c] = *(const uint4 *)(qh + (k0 < D ? k0 : k0 - D));
    }
  }

  if constexpr (kAppend) {
    // on_kv_stored for this work-group's pages and KV head: the new tokens'
    // K/V go to their slots and the pages' min/max rows are refreshed, then a
    // barrier makes the rows visible to the waves that score them.  Only the
    // work-groups that own a touched page do this (one per request and head
    // at decode); the page-id and q loads above are already in flight.
    if (n_new > 0 && p0 >= 0) {
      const int p1 = p0 + n_new;
      const int a0 = max(p0 / P, base);
      const int a1 = min((p1 - 1) / P, base + kScorePagesPerBlock - 1);
      if (a0 <= a1) {
        const int32_t *ptr = page_table + (int64_t)r * max_pages;
        for (int pg = a0; pg <= a1 && pg < max_pages; ++pg) {
          const int64_t phys = ptr[pg];
          if (phys < 0 || phys >= pool) continue;
          const AppendSpan a = append_span(phys, Hkv, g, P, pg, p0, p1, row0);
          for (int d = threadIdx.x; d < D; d += blockDim.x)
            append_channel<uint16_t>(a, d, Hkv, D, P, fa.k_new, fa.v_new, fa.k_cache,
                                     fa.v_cache, kmeta);
        }
        __syncthreads();
      }
    }
  }

  bool in_pool[kScoreTilesPerWave];
#pragma unroll
  for (int t = 0; t < kScoreTilesPerWave; ++t) {
    const int64_t phys = row[t];
    in_pool[t] = phys >= 0 && phys < pool;
    const bool ok = page[t] < n && in_pool[t];
    row[t] = (ok ? phys * Hkv + g : (int64_t)g) * (2 * D);
  }

  uint4 b[kScoreTilesPerWave][kChunks];
#pragma unroll
  for (int t = 0; t < kScoreTilesPerWave; ++t)
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
      b[t][c] = *(const uint4 *)(kmeta + row[t] + c * 32 + grp * 8);

  // A operand: [q- | q+] (zero rows past G).
  bf16x8 a[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int k0 = c * 32 + grp * 8;
    uint4 neg, pos;
    split_signs(qw[c], neg, pos);
    uint4 x = k0 < D ? neg : pos;
    if (col >= G) x = make_uint4(0, 0, 0, 0);
    a[c] = as_bf16x8(x);
  }

#pragma unroll
  for (int t = 0; t < kScoreTilesPerWave; ++t) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c], as_bf16x8(b[t][c]), acc, 0, 0, 0);
    // lane holds page `col`, heads 4*grp .. 4*grp+3
    if (per_head) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * grp + i < G && page[t] < n)
          out[(int64_t)(4 * grp + i) * max_pages + page[t]] =
              in_pool[t] ? acc[i] : -__builtin_huge_valf();
      continue;
    }
    // combine the group
    float v = reduce == 0 ? -__builtin_huge_valf() : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (4 * grp + i < G) v = reduce == 0 ? fmaxf(v, acc[i]) : v + acc[i];
    }
    const float o16 = __shfl_xor(v, 16, kWave);
    v = reduce == 0 ? fmaxf(v, o16) : v + o16;
    const float o32 = __shfl_xor(v, 32, kWave);
    v = reduce == 0 ? fmaxf(v, o32) : v + o32;
    if (grp == 0 && page[t] < n) out[page[t]] = in_pool[t] ? v : -__builtin_huge_valf();
  }
}

constexpr int kMaxGroup = 16;       // q heads per KV head the layout allows

// fp32 path: one thread per page, the group's q in LDS, padded with zero
// rows to kG heads (the power of two at or above G) so the loop over heads
// has no branch (a padded head's sum is never read).  Each term is the
// product on the side the sign of q selects (q * max for q >= 0, else
// q * min), the larger of the two exact products, so the choice itself
// rounds nothing; the compiler fuses it into the fp32 add (one rounding per
// term).  Every head sums over d in order.
// With cu_new non-null (the fused on_kv_stored + scores path) the request
// length is ctx_before + its new tokens, and the work-group whose pages hold
// new tokens first stores them for its KV head and refreshes those pages'
// min/max (the per-channel body of the standalone append, so the metadata is
// the same bit for bit); the barrier after the q load makes the rows visible
// to the threads that score them.  Else the length is ctx_lens.
template <int kG>
__global__ __launch_bounds__(256) void page_scores_valu_kernel(
    int Hkv, int G, int per_head, int D, int64_t pool, int P, int max_pages, int reduce,
    const float *__restrict__ q, float *kmeta,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ ctx_lens,
    const int32_t *__restrict__ cu_new, const int32_t *__restrict__ ctx_before,
    const float *__restrict__ k_new, const float *__restrict__ v_new, float *k_cache,
    float *v_cache, float *__restrict__ scores) {
  extern __shared__ __align__(16) float q_lds[];     // [kG][D]
  const int g = blockIdx.y, r = blockIdx.z;
  const float *qg = q + ((int64_t)r * Hkv * G + (int64_t)g * G) * D;
  for (int i = threadIdx.x; i < kG * D; i += blockDim.x) q_lds[i] = i < G * D ? qg[i] : 0.f;
  if (cu_new != nullptr && k_new != nullptr) {
    const int row0 = cu_new[r], n_new = cu_new[r + 1] - row0, p0 = ctx_before[r];
    if (n_new > 0 && p0 >= 0) {
      const int p1 = p0 + n_new;
      const int base = blockIdx.x * blockDim.x;
      const int a0 = max(p0 / P, base);
      const int a1 = min((p1 - 1) / P, base + (int)blockDim.x - 1);
      const int32_t *ptr = page_table + (int64_t)r * max_pages;
      for (int pg = a0; pg <= a1 && pg < max_pages; ++pg) {
        const int64_t phys = ptr[pg];
        if (phys < 0 || phys >= pool) continue;
        const AppendSpan a = append_span(phys, Hkv, g, P, pg, p0, p1, row0);
        for (int d = threadIdx.x; d < D; d += blockDim.x)
          append_channel<float>(a, d, Hkv, D, P, k_new, v_new, k_cache, v_cache, kmeta);
      }
    }
  }
  __syncthreads();
  const int ctx = cu_new ? ctx_before[r] + max(cu_new[r + 1] - cu_new[r], 0) : ctx_lens[r];
  const int n = pages_in(ctx, P, max_pages);
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const int64_t phys = page_table[(int64_t)r * max_pages + j];
  if (phys < 0 || phys >= pool) {                     // outside the pool: -inf
    if (per_head) {
      for (int h = 0; h < G; ++h)
        scores[((int64_t)(r * Hkv + g) * G + h) * max_pages + j] = -__builtin_huge_valf();
    } else {
      scores[((int64_t)r * Hkv + g) * max_pages + j] = -__builtin_huge_valf();
    }
    return;
  }
  const float *lo = kmeta + (phys * Hkv + g) * 2 * D;
  const float *hi = lo + D;
  float u[kG];
#pragma unroll
  for (int h = 0; h < kG; ++h) u[h] = 0.f;
  if ((((uintptr_t)kmeta) & 15u) == 0) {
    // 16 channels of min and of max in flight at once (D is 64 or 128, a
    // multiple of 16, and rows of 2D floats keep 16-byte alignment); q read
    // 4 channels of a head at a time
    for (int d0 = 0; d0 < D; d0 += 16) {
      float4 la[4], ha[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        la[i] = *(const float4 *)(lo + d0 + 4 * i);
        ha[i] = *(const float4 *)(hi + d0 + 4 * i);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 qv[kG];
#pragma unroll
        for (int h = 0; h < kG; ++h) qv[h] = *(const float4 *)&q_lds[h * D + d0 + 4 * i];
        const float a[4] = {la[i].x, la[i].y, la[i].z, la[i].w};
        const float b[4] = {ha[i].x, ha[i].y, ha[i].z, ha[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int h = 0; h < kG; ++h) {
            const float qd = e == 0 ? qv[h].x : (e == 1 ? qv[h].y : (e == 2 ? qv[h].z : qv[h].w));
            u[h] += qd >= 0.f ? qd * b[e] : qd * a[e];
          }
        }
      }
    }
  } else {
    for (int d = 0; d < D; ++d) {
      const float a = lo[d], b = hi[d];
#pragma unroll
      for (int h = 0; h < kG; ++h) {
        const float qd = q_lds[h * D + d];
        u[h] += qd >= 0.f ? qd * b : qd * a;
      }
    }
  }
  float v = reduce == 0 ? -__builtin_huge_valf() : 0.f;
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    if (h < G) {
      if (per_head) scores[((int64_t)(r * Hkv + g) * G + h) * max_pages + j] = u[h];
      v = reduce == 0 ? fmaxf(v, u[h]) : v + u[h];
    }
  }
  if (!per_head) scores[((int64_t)r * Hkv + g) * max_pages + j] = v;
}

static hipError_t launch_scores(const Dims &dm, int batch, const void *q, void *kmeta,
                                const int32_t *page_table, const int32_t *ctx_lens, int reduce,
                                const FusedAppend &fa, bool fused, float *scores,
                                hipStream_t stream) {
  if (dm.dtype == 1) {
    const int blocks = (dm.max_pages + kScorePagesPerBlock - 1) / kScorePagesPerBlock;
    dim3 grid((unsigned)(blocks * dm.Hkv), (unsigned)batch);
    dim3 block(64 * kScoreWaves);
#define QUEST_SCORES(DD, AA)                                                                \
  hipLaunchKernelGGL((page_scores_mfma_kernel<DD, AA>), grid, block, 0, stream, dm.Hkv, dm.G, \
                     (int)dm.per_head(),                                                    \
                     dm.pool, dm.P, dm.max_pages, reduce, (const uint16_t *)q,              \
                     (uint16_t *)kmeta, page_table, ctx_lens, fa, scores)
    if (dm.D == 128) {
      if (fused) QUEST_SCORES(128, true); else QUEST_SCORES(128, false);
    } else {
      if (fused) QUEST_SCORES(64, true); else QUEST_SCORES(64, false);
    }
#undef QUEST_SCORES
  } else {
    dim3 grid((unsigned)((dm.max_pages + 255) / 256), (unsigned)dm.Hkv, (unsigned)batch);
#define QUEST_SCORES32(KG)                                                                  \
  hipLaunchKernelGGL(page_scores_valu_kernel<KG>, grid, dim3(256),                          \
                     (size_t)(KG) * dm.D * sizeof(float), stream, dm.Hkv, dm.G,             \
                     (int)dm.per_head(), dm.D, dm.pool, dm.P, dm.max_pages, reduce,         \
                     (const float *)q, (float *)kmeta, page_table, ctx_lens,                \
                     fused ? fa.cu_new : nullptr, fused ? fa.ctx_before : nullptr,           \
                     fused ? (const float *)fa.k_new : nullptr,                             \
                     fused ? (const float *)fa.v_new : nullptr,                             \
                     fused ? (float *)fa.k_cache : nullptr,                                 \
                     fused ? (float *)fa.v_cache : nullptr, scores)
    if (dm.G <= 1) QUEST_SCORES32(1);
    else if (dm.G <= 2) QUEST_SCORES32(2);
    else if (dm.G <= 4) QUEST_SCORES32(4);
    else if (dm.G <= 8) QUEST_SCORES32(8);
    else QUEST_SCORES32(kMaxGroup);
#undef QUEST_SCORES32
  }
  return hipGetLastError();
}

hipError_t launch_page_scores(const Dims &dm, int batch, const void *q,
                              const void *kmeta, const int32_t *page_table,
                              const int32_t *ctx_lens, int reduce,
                              float *scores, hipStream_t stream) {
  const FusedAppend none{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  return launch_scores(dm, batch, q, const_cast<void *>(kmeta), page_table, ctx_lens, reduce,
                       none, false, scores, stream);
}

hipError_t launch_append_scores(const Dims &dm, int batch, const void *q, const void *k_new,
                                const void *v_new, const int32_t *cu_new,
                                const int32_t *ctx_before, int max_new,
                                const int32_t *page_table, void *k_cache, void *v_cache,
                                void *kmeta, int reduce, float *scores, hipStream_t stream) {
  (void)max_new;                    // each work-group finds its own touched pages
  const FusedAppend fa{(const uint16_t *)k_new, (const uint16_t *)v_new, cu_new, ctx_before,
                       (uint16_t *)k_cache, (uint16_t *)v_cache};
  return launch_scores(dm, batch, q, kmeta, page_table, nullptr, reduce, fa, true, scores,
                       stream);
}

}  // namespace quest
