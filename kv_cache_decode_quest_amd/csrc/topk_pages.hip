// topk_pages.hip -- build_decode_view, part 2: the top-k pages of every
// (request, KV head) row within the request's token budget.
//
// k = min(max_k, clamp(floor(budget / P), 1, n)) pages of the row's n are
// kept: the largest scores, equal scores to the lower logical page.  That
// order is the order of the unique 64-bit key
//     (orderable(score) << 32) | (0xffffffff - page),
// so the selected set is unique and any exact top-k algorithm returns it.
//
// One work-group per row, radix select on the 32-bit orderable score keys:
//  1. block min/max of the keys: every key shares the bits above the highest
//     bit where min and max differ;
//  2. an (up to) 11-bit histogram on the next bits finds the bucket that holds
//     the k-th largest key, and how many keys above it are kept outright;
//  3. the bucket's keys (typically a handful) are gathered into LDS; if they
//     fit in one wave, each lane ranks its (key, page) pair against the others
//     in the 64-bit order; otherwise further 8-bit histogram passes over the
//     row narrow the bucket to a single key value;
//  4. a final pass writes the kept pages in ascending order: every page whose
//     key is above the threshold key, and the lowest-index pages among those
//     equal to it up to the count still needed.  Each thread owns a
//     contiguous run of pages, and an exclusive scan of per-thread counts gives
//     each its output position.
#include "quest_device.h"
#include "quest_launch.h"

namespace quest {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kBins1 = 2048;

// Larger score <-> larger key; -0.0 and +0.0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive block scan of one value per thread (kTopkThreads threads).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v, lane);
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  uint32_t off = 0;
  for (int w = 0; w < wave; ++w) off += wave_tot[w];
  __syncthreads();
  return off + incl - v;
}

struct TopkShared {
  uint32_t hist[kBins1];
  uint32_t wave_a[kTopkWaves], wave_b[kTopkWaves];
  uint32_t cand_key[kWave];
  int32_t cand_idx[kWave];
  uint32_t cand_count;
  uint32_t prefix;     // known high bits of the threshold key
  uint32_t krem;       // keys still to take at or below the known prefix
};

// Finds, in hist[0..bins), the bucket holding the krem-th largest element
// (buckets scanned from the top).  Wave 0 only.  Returns via sh.
__device__ void pick_bucket(TopkShared &sh, int bins, uint32_t krem, uint32_t prefix,
                            int shift) {
  const int lane = threadIdx.x & 63;
  const int per = (bins + kWave - 1) / kWave;       // buckets per lane, top first
  uint32_t tot = 0;
  for (int i = 0; i < per; ++i) {
    const int b = bins - 1 - (lane * per + i);
    if (b >= 0) tot += sh.hist[b];
  }
  const uint32_t incl = wave_incl_scan(tot, lane);
  const uint32_t excl = incl - tot;
  if (excl < krem && krem <= incl) {
    uint32_t cum = excl;
    for (int i = 0; i < per; ++i) {
      const int b = bins - 1 - (lane * per + i);
      if (b < 0) break;
      const uint32_t c = sh.hist[b];
      if (cum + c >= krem) {
        sh.prefix = prefix | ((uint32_t)b << shift);
        sh.krem = krem - cum;
        break;
      }
      cum += c;
    }
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_pages_kernel(
    int Hkv, int P, int max_pages, int max_k, const float *__restrict__ scores,
    const int32_t *__restrict__ ctx_lens, const int32_t *__restrict__ budget_tokens,
    int32_t *__restrict__ sel_pages, int32_t *__restrict__ num_sel) {
  __shared__ TopkShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  const int r = row / Hkv;
  const int n = pages_in(ctx_lens[r], P, max_pages);
  int k = 0;
  if (n > 0) {
    k = budget_tokens[r] / P;
    k = k < 1 ? 1 : (k > n ? n : k);
    k = k < max_k ? k : max_k;
  }
  const float *s = scores + (int64_t)row * max_pages;
  int32_t *out = sel_pages + (int64_t)row * max_k;
  if (tid == 0) num_sel[row] = k;
  for (int i = k + tid; i < max_k; i += kTopkThreads) out[i] = -1;
  if (k == n) {                                       // the whole row (or nothing)
    for (int i = tid; i < n; i += kTopkThreads) out[i] = i;
    return;
  }

  // 1. min and max key
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int j = tid; j < n; j += kTopkThreads) {
    const uint32_t u = order_key(s[j]);
    lo = min(lo, u);
    hi = max(hi, u);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor(lo, o, kWave));
    hi = max(hi, (uint32_t)__shfl_xor(hi, o, kWave));
  }
  if (lane == 0) {
    sh.wave_a[wave] = lo;
    sh.wave_b[wave] = hi;
  }
  for (int i = tid; i < kBins1; i += kTopkThreads) sh.hist[i] = 0;
  if (tid == 0) sh.cand_count = 0;
  __syncthreads();
  lo = sh.wave_a[0];
  hi = sh.wave_b[0];
  for (int w = 1; w < kTopkWaves; ++w) {
    lo = min(lo, sh.wave_a[w]);
    hi = max(hi, sh.wave_b[w]);
  }

  uint32_t thresh, krem;
  if (lo == hi) {                                     // every key equal
    thresh = lo;
    krem = (uint32_t)k;
  } else {
    // 2. first histogram on the bits just below the common prefix
    const int hb = 31 - __builtin_clz(lo ^ hi);
    const int shift1 = hb >= 10 ? hb - 10 : 0;
    const int bins = 1 << (hb - shift1 + 1);
    const uint32_t bmask = (uint32_t)bins - 1u;
    for (int j = tid; j < n; j += kTopkThreads) {
      const uint32_t u = order_key(s[j]);
      atomicAdd(&sh.hist[(u >> shift1) & bmask], 1u);
    }
    __syncthreads();
    const uint32_t common = (hb == 31) ? 0u : (hi >> (hb + 1)) << (hb + 1);
    if (wave == 0) pick_bucket(sh, bins, (uint32_t)k, common, shift1);
    __syncthreads();
    uint32_t prefix = sh.prefix;
    krem = sh.krem;
    int lowbit = shift1;             // bits >= lowbit of the threshold are known

    // 3. gather the bucket's keys; rank them in one wave if they fit
    if (lowbit > 0) {
      for (int j = tid; j < n; j += kTopkThreads) {
        const uint32_t u = order_key(s[j]);
        if ((u >> lowbit) == (prefix >> lowbit)) {
          const uint32_t slot = atomicAdd(&sh.cand_count, 1u);
          if (slot < (uint32_t)kWave) {
            sh.cand_key[slot] = u;
            sh.cand_idx[slot] = j;
          }
        }
      }
      __syncthreads();
      const uint32_t c = sh.cand_count;
      if (c <= (uint32_t)kWave) {
        if (wave == 0) {
          const bool mine = (uint32_t)lane < c;
          const uint64_t me = mine ? (((uint64_t)sh.cand_key[lane] << 32) |
                                      (0xffffffffu - (uint32_t)sh.cand_idx[lane]))
                                   : 0ull;
          uint32_t rank = 0;
          for (uint32_t m = 0; m < c; ++m) {
            const uint64_t other = ((uint64_t)sh.cand_key[m] << 32) |
                                   (0xffffffffu - (uint32_t)sh.cand_idx[m]);
            rank += other > me;
          }
          if (mine && rank == krem - 1) {
            // threshold = this pair; count the equal-key pairs at or above it
            const uint32_t tkey = sh.cand_key[lane];
            const int32_t tidx = sh.cand_idx[lane];
            uint32_t eq = 0;
            for (uint32_t m = 0; m < c; ++m)
              eq += (sh.cand_key[m] == tkey && sh.cand_idx[m] <= tidx);
            sh.prefix = tkey;
            sh.krem = eq;
          }
        }
        __syncthreads();
        prefix = sh.prefix;
        krem = sh.krem;
        lowbit = 0;
      }
    }
    // 3b. many keys in the bucket: narrow it 8 bits at a time over the row
    while (lowbit > 0) {
      const int w = lowbit < 8 ? lowbit : 8;
      const int shift = lowbit - w;
      const uint32_t wmask = (1u << w) - 1u;
      for (int i = tid; i < (1 << w); i += kTopkThreads) sh.hist[i] = 0;
      __syncthreads();
      for (int j = tid; j < n; j += kTopkThreads) {
        const uint32_t u = order_key(s[j]);
        if ((u >> lowbit) == (prefix >> lowbit)) atomicAdd(&sh.hist[(u >> shift) & wmask], 1u);
      }
      __syncthreads();
      if (wave == 0) pick_bucket(sh, 1 << w, krem, prefix, shift);
      __syncthreads();
      prefix = sh.prefix;
      krem = sh.krem;
      lowbit = shift;
    }
    thresh = prefix;
  }

  // 4. ascending output: keys above the threshold, then the first `krem`
  //    pages whose key equals it.
  const int chunk = (n + kTopkThreads - 1) / kTopkThreads;
  const int j0 = tid * chunk;
  const int j1 = min(n, j0 + chunk);
  uint32_t gt = 0, eq = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t u = order_key(s[j]);
    gt += u > thresh;
    eq += u == thresh;
  }
  const uint32_t gt_before = block_excl_scan(gt, sh.wave_a);
  uint32_t eq_before = block_excl_scan(eq, sh.wave_b);
  uint32_t pos = gt_before + min(eq_before, krem);
  for (int j = j0; j < j1; ++j) {
    const uint32_t u = order_key(s[j]);
    const bool take = u > thresh || (u == thresh && eq_before++ < krem);
    if (take) {
      if (pos < (uint32_t)k) out[pos] = j;      // never past the row
      ++pos;
    }
  }
}

hipError_t launch_topk(const Dims &dm, int batch, const float *scores,
                       const int32_t *ctx_lens, const int32_t *budget_tokens,
                       int max_k, int32_t *sel_pages, int32_t *num_sel,
                       hipStream_t stream) {
  dim3 grid((unsigned)(batch * dm.Hkv));
  hipLaunchKernelGGL(topk_pages_kernel, grid, dim3(kTopkThreads), 0, stream, dm.Hkv, dm.P,
                     dm.max_pages, max_k, scores, ctx_lens, budget_tokens, sel_pages,
                     num_sel);
  return hipGetLastError();
}

}  // namespace quest
