// topk_pages.hip -- build_decode_view, part 2: the top-k pages of every
// (request, KV head) row within the request's token budget.
//
// k = min(max_k, clamp(floor(budget / P), 1, n)) pages of the row's n are
// kept: the largest scores, equal scores to the lower logical page.  That
// order is the order of the unique 64-bit key
//     (orderable(score) << 32) | (0xffffffff - page),
// so the selected set is unique and any exact top-k algorithm returns it.
//
// One work-group per row, radix select on the 32-bit orderable score keys
// (staged in LDS for rows of up to 8192 pages):
//  1. block min/max of the keys: every key shares the bits above the highest
//     bit where min and max differ;
//  2. refinement passes: an (up to) 11-bit histogram of the keys that match
//     the known prefix, on the next bits, finds the bucket holding the k-th
//     largest key and how many keys above it are kept outright; the bucket's
//     bits join the prefix;
//  3. as soon as the bucket holds at most 64 keys, they are gathered into LDS
//     and one wave ranks its (key, page) pairs in the 64-bit order, which
//     fixes the threshold pair; otherwise refinement continues down to the
//     last bit;
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
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
static_assert(kBins == 2 * kTopkThreads, "each thread owns two histogram buckets");

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

struct TopkShared {
  uint32_t hist[kBins];
  uint32_t wave_tot[kTopkWaves];
  uint32_t cand_key[kWave];
  int32_t cand_idx[kWave];
  uint32_t cand_count;
  uint32_t prefix;     // known high bits of the threshold key
  uint32_t krem;       // keys still to take at or below the known prefix
  uint32_t bucket;     // keys in the chosen bucket
  uint32_t lo, hi;
};

// Inclusive scan over the block in thread order.  Ends with a barrier, so
// wave_tot may be reused right after.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, TopkShared &sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v, lane);
  if (lane == kWave - 1) sh.wave_tot[wave] = incl;
  __syncthreads();
  uint32_t off = 0;
  for (int w = 0; w < wave; ++w) off += sh.wave_tot[w];
  __syncthreads();
  return off + incl;
}

// The bucket (of `bins`) that holds the krem-th largest counted key, scanning
// buckets from the top; thread t owns buckets bins-1-2t and bins-2-2t, read
// from consecutive LDS words.  Results in sh.prefix / sh.krem / sh.bucket.
__device__ __forceinline__ void pick_bucket(TopkShared &sh, int bins, uint32_t krem,
                                            uint32_t prefix, int shift) {
  const int b1 = bins - 1 - 2 * (int)threadIdx.x, b0 = b1 - 1;
  const uint32_t c1 = b1 >= 0 ? sh.hist[b1] : 0u;
  const uint32_t c0 = b0 >= 0 ? sh.hist[b0] : 0u;
  const uint32_t incl = block_incl_scan(c1 + c0, sh);
  const uint32_t excl = incl - c1 - c0;
  if (excl < krem && krem <= incl) {
    const bool upper = excl + c1 >= krem;
    const int b = upper ? b1 : b0;
    sh.prefix = prefix | ((uint32_t)b << shift);
    sh.krem = krem - (upper ? excl : excl + c1);
    sh.bucket = upper ? c1 : c0;
  }
  __syncthreads();
}

// Rows of up to kStagedKeys pages are read from HBM once, into LDS, as
// orderable keys; every later pass reads LDS.  Longer rows read their scores
// from global memory in every pass.
constexpr int kStagedKeys = 8192;
constexpr int kLoadUnroll = kStagedKeys / kTopkThreads;

template <bool kStaged>
__global__ __launch_bounds__(kTopkThreads) void topk_pages_kernel(
    int Hkv, int P, int max_pages, int max_k, const float *__restrict__ scores,
    const int32_t *__restrict__ ctx_lens, const int32_t *__restrict__ budget_tokens,
    int32_t *__restrict__ sel_pages, int32_t *__restrict__ num_sel) {
  __shared__ TopkShared sh;
  __shared__ uint32_t staged[kStaged ? kStagedKeys : 1];
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
  auto key = [&](int j) -> uint32_t {
    if constexpr (kStaged) return staged[j];
    else return order_key(s[j]);
  };

  // 1. min and max key (and, for short rows, the keys into LDS: all loads of
  //    a thread are issued together from clamped addresses)
  uint32_t lo = 0xffffffffu, hi = 0u;
  if constexpr (kStaged) {
    float v[kLoadUnroll];
#pragma unroll
    for (int i = 0; i < kLoadUnroll; ++i) {
      const int j = tid + i * kTopkThreads;
      v[i] = s[j < n ? j : 0];
    }
#pragma unroll
    for (int i = 0; i < kLoadUnroll; ++i) {
      const int j = tid + i * kTopkThreads;
      const uint32_t u = order_key(v[i]);
      if (j < n) {
        staged[j] = u;
        lo = min(lo, u);
        hi = max(hi, u);
      }
    }
  } else {
    for (int j = tid; j < n; j += kTopkThreads) {
      const uint32_t u = order_key(s[j]);
      lo = min(lo, u);
      hi = max(hi, u);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor(lo, o, kWave));
    hi = max(hi, (uint32_t)__shfl_xor(hi, o, kWave));
  }
  if (tid == 0) {
    sh.lo = 0xffffffffu;
    sh.hi = 0u;
    sh.cand_count = 0;
  }
  sh.hist[2 * tid] = 0;
  sh.hist[2 * tid + 1] = 0;
  __syncthreads();
  if (lane == 0) {
    atomicMin(&sh.lo, lo);
    atomicMax(&sh.hi, hi);
  }
  __syncthreads();
  lo = sh.lo;
  hi = sh.hi;

  uint32_t thresh, krem = (uint32_t)k;
  if (lo == hi) {                                     // every key equal
    thresh = lo;
  } else {
    // 2./3. refine the threshold key, 11 bits at a time
    const int hb = 31 - __builtin_clz(lo ^ hi);
    int lowbit = hb + 1;                              // bits >= lowbit are known
    uint32_t prefix = (uint32_t)(((uint64_t)hi >> lowbit) << lowbit);
    bool first_pass = true;
    for (;;) {
      const int w = lowbit < kDigitBits ? lowbit : kDigitBits;
      const int shift = lowbit - w;
      const uint32_t bmask = (1u << w) - 1u;
      if (!first_pass) {
        sh.hist[2 * tid] = 0;
        sh.hist[2 * tid + 1] = 0;
        __syncthreads();
      }
      first_pass = false;
      const uint64_t want = (uint64_t)prefix >> lowbit;
      for (int j = tid; j < n; j += kTopkThreads) {
        const uint32_t u = key(j);
        if (((uint64_t)u >> lowbit) == want) atomicAdd(&sh.hist[(u >> shift) & bmask], 1u);
      }
      __syncthreads();
      pick_bucket(sh, 1 << w, krem, prefix, shift);
      prefix = sh.prefix;
      krem = sh.krem;
      const uint32_t count = sh.bucket;
      lowbit = shift;
      if (lowbit == 0) {                              // the threshold key itself
        thresh = prefix;
        break;
      }
      if (count <= (uint32_t)kWave) {
        // gather the bucket and rank it in one wave
        const uint32_t want2 = prefix >> lowbit;
        for (int j = tid; j < n; j += kTopkThreads) {
          const uint32_t u = key(j);
          if ((u >> lowbit) == want2) {
            const uint32_t slot = atomicAdd(&sh.cand_count, 1u);
            if (slot < (uint32_t)kWave) {
              sh.cand_key[slot] = u;
              sh.cand_idx[slot] = j;
            }
          }
        }
        __syncthreads();
        if (wave == 0) {
          const uint32_t c = count;
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
        thresh = sh.prefix;
        krem = sh.krem;
        break;
      }
    }
  }

  // 4. ascending output: keys above the threshold, then the first `krem`
  //    pages whose key equals it.  One scan of (above, equal) counts packed
  //    in 16-bit halves when the row fits, two scans otherwise.
  const int chunk = (n + kTopkThreads - 1) / kTopkThreads;
  const int j0 = tid * chunk;
  const int j1 = min(n, j0 + chunk);
  uint32_t gt = 0, eq = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t u = key(j);
    gt += u > thresh;
    eq += u == thresh;
  }
  uint32_t gt_before, eq_before;
  if (n < 65536) {
    const uint32_t packed = (gt << 16) | eq;
    const uint32_t before = block_incl_scan(packed, sh) - packed;
    gt_before = before >> 16;
    eq_before = before & 0xffffu;
  } else {
    gt_before = block_incl_scan(gt, sh) - gt;
    eq_before = block_incl_scan(eq, sh) - eq;
  }
  uint32_t pos = gt_before + min(eq_before, krem);
  for (int j = j0; j < j1; ++j) {
    const uint32_t u = key(j);
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
  if (dm.max_pages <= kStagedKeys)
    hipLaunchKernelGGL(topk_pages_kernel<true>, grid, dim3(kTopkThreads), 0, stream, dm.Hkv,
                       dm.P, dm.max_pages, max_k, scores, ctx_lens, budget_tokens, sel_pages,
                       num_sel);
  else
    hipLaunchKernelGGL(topk_pages_kernel<false>, grid, dim3(kTopkThreads), 0, stream, dm.Hkv,
                       dm.P, dm.max_pages, max_k, scores, ctx_lens, budget_tokens, sel_pages,
                       num_sel);
  return hipGetLastError();
}

}  // namespace quest
