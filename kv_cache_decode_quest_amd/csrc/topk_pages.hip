// topk_pages.hip -- build_decode_view, part 2: the top-k pages of every
// (request, KV head) row within the request's token budget.
//
// k = min(max_k, clamp(floor(budget / P), 1, n)) pages of the row's n are
// kept: the largest scores, equal scores to the lower logical page.  That
// order is the order of the unique 64-bit key
//     (orderable(score) << 32) | (0xffffffff - page),
// so the selected set is unique and any exact top-k algorithm returns it.
//
// One 1024-thread work-group per row, radix select on the 32-bit orderable
// score keys (held in registers for rows of up to 8192 pages).  The work is a
// handful of barrier-separated phases, each short; wave-level scans and
// reductions use the DPP network and ballots, not LDS round trips.
//  1. min and max key: every key shares the bits above the highest bit where
//     they differ;
//  2. refinement: an (up to) 11-bit histogram of the keys matching the known
//     prefix, on the next bits, gives the bucket holding the k-th largest key
//     and the count kept above it; repeated until the bucket holds at most 64
//     keys (usually once) or the key is fully known;
//  3. the bucket's keys are gathered into LDS and every wave ranks the
//     (key, page) pairs in the 64-bit order, which fixes the threshold;
//  4. each wave walks a contiguous range of pages with ballots: a count pass,
//     one barrier to exchange the per-wave counts, then a write pass that puts
//     every page above the threshold, and the lowest-index pages equal to it
//     up to the count still needed, at its ascending position.
#include "quest_device.h"
#include "quest_launch.h"

namespace quest {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
constexpr int kBinsPerWave = kBins / kTopkWaves;     // 128: two per lane
static_assert(kBinsPerWave == 2 * kWave, "each lane owns two histogram buckets");

// Larger score <-> larger key; -0.0 and +0.0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct TopkShared {
  uint32_t hist[kBins];
  uint32_t wave_a[kTopkWaves], wave_b[kTopkWaves];
  uint32_t cand_key[kWave];
  int32_t cand_idx[kWave];
  uint32_t cand_count;
  uint32_t prefix;     // known high bits of the threshold key
  uint32_t krem;       // keys still to take at or below the known prefix
  uint32_t bucket;     // keys in the chosen bucket
};

// The bucket (of `bins` <= kBins) holding the krem-th largest counted key,
// buckets ranked from the top: wave w owns the 128 buckets below the top
// 128*w, lane l two of them.  Results in sh.prefix / sh.krem / sh.bucket.
__device__ __forceinline__ void pick_bucket(TopkShared &sh, int bins, uint32_t krem,
                                            uint32_t prefix, int shift) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int b1 = bins - 1 - kBinsPerWave * wave - 2 * lane, b0 = b1 - 1;
  const uint32_t c1 = b1 >= 0 ? sh.hist[b1] : 0u;
  const uint32_t c0 = b0 >= 0 ? sh.hist[b0] : 0u;
  const uint32_t incl = wave_incl_sum(c1 + c0);
  if (lane == kWave - 1) sh.wave_a[wave] = incl;
  __syncthreads();
  uint32_t above = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) above += (w < wave) ? sh.wave_a[w] : 0u;
  const uint32_t excl = above + incl - c1 - c0;
  if (excl < krem && krem <= excl + c1 + c0) {
    const bool upper = excl + c1 >= krem;
    sh.prefix = prefix | ((uint32_t)(upper ? b1 : b0) << shift);
    sh.krem = krem - (upper ? excl : excl + c1);
    sh.bucket = upper ? c1 : c0;
  }
  __syncthreads();
}

// Rows of up to kRegKeys pages are read from HBM once, into registers: wave w
// holds pages [512 w, 512 w + 512), lane l pages 512 w + 64 i + l (i < 8), the
// same wave-contiguous order the output pass needs, so no pass re-reads
// memory.  Longer rows read their scores from global memory in every pass.
constexpr int kPerThread = 8;
constexpr int kRegKeys = kPerThread * kTopkThreads;      // 8192
constexpr int kRegSpan = kPerThread * kWave;              // pages per wave

template <bool kRegs>
__global__ __launch_bounds__(kTopkThreads) void topk_pages_kernel(
    int Hkv, int P, int max_pages, int max_k, const float *__restrict__ scores,
    const int32_t *__restrict__ ctx_lens, const int32_t *__restrict__ budget_tokens,
    int32_t *__restrict__ sel_pages, int32_t *__restrict__ num_sel) {
  __shared__ TopkShared sh;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int row = blockIdx.x;
  const int r = row / Hkv;
  const float *s = scores + (int64_t)row * max_pages;
  // Register rows: the whole score row is loaded in the same round trip as
  // the request's length and budget (entries past the length are ignored).
  float sv[kRegs ? kPerThread : 1];
  if constexpr (kRegs) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int j = wave * kRegSpan + i * kWave + lane;
      sv[i] = s[j < max_pages ? j : 0];
    }
  }
  const int n = pages_in(ctx_lens[r], P, max_pages);
  int k = 0;
  if (n > 0) {
    k = budget_tokens[r] / P;
    k = k < 1 ? 1 : (k > n ? n : k);
    k = k < max_k ? k : max_k;
  }
  int32_t *out = sel_pages + (int64_t)row * max_k;
  if (tid == 0) num_sel[row] = k;
  for (int i = k + tid; i < max_k; i += kTopkThreads) out[i] = -1;
  if (k == n) {                                       // the whole row (or nothing)
    for (int i = tid; i < n; i += kTopkThreads) out[i] = i;
    return;
  }
  // The thread's keys: registers, or global memory for long rows.  Invalid
  // slots (past the row) never count; their key is 0.
  uint32_t u[kRegs ? kPerThread : 1];
  if constexpr (kRegs) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int j = wave * kRegSpan + i * kWave + lane;
      u[i] = j < n ? order_key(sv[i]) : 0u;
    }
  }
  auto valid = [&](int i) { return wave * kRegSpan + i * kWave + lane < n; };

  // 1. min and max key
  uint32_t lo = 0xffffffffu, hi = 0u;
  if constexpr (kRegs) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
      if (valid(i)) {
        lo = min(lo, u[i]);
        hi = max(hi, u[i]);
      }
  } else {
    for (int j = tid; j < n; j += kTopkThreads) {
      const uint32_t x = order_key(s[j]);
      lo = min(lo, x);
      hi = max(hi, x);
    }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    sh.wave_a[wave] = lo;
    sh.wave_b[wave] = hi;
  }
  sh.hist[2 * tid] = 0;
  sh.hist[2 * tid + 1] = 0;
  if (tid == 0) sh.cand_count = 0;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    lo = min(lo, sh.wave_a[w]);
    hi = max(hi, sh.wave_b[w]);
  }

  uint32_t thresh, krem = (uint32_t)k;
  if (lo == hi) {                                     // every key equal
    thresh = lo;
  } else {
    // 2. refine the threshold key, 11 bits at a time
    const int hb = 31 - __builtin_clz(lo ^ hi);
    int lowbit = hb + 1;                              // bits >= lowbit are known
    uint32_t prefix = (uint32_t)(((uint64_t)hi >> lowbit) << lowbit);
    uint32_t count;
    for (bool first_pass = true;; first_pass = false) {
      const int w = lowbit < kDigitBits ? lowbit : kDigitBits;
      const int shift = lowbit - w;
      const uint32_t bmask = (1u << w) - 1u;
      if (!first_pass) {
        sh.hist[2 * tid] = 0;
        sh.hist[2 * tid + 1] = 0;
        __syncthreads();
      }
      const uint64_t want = (uint64_t)prefix >> lowbit;
      if constexpr (kRegs) {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i)
          if (valid(i) && ((uint64_t)u[i] >> lowbit) == want)
            atomicAdd(&sh.hist[(u[i] >> shift) & bmask], 1u);
      } else {
        for (int j = tid; j < n; j += kTopkThreads) {
          const uint32_t x = order_key(s[j]);
          if (((uint64_t)x >> lowbit) == want) atomicAdd(&sh.hist[(x >> shift) & bmask], 1u);
        }
      }
      __syncthreads();
      pick_bucket(sh, 1 << w, krem, prefix, shift);
      prefix = sh.prefix;
      krem = sh.krem;
      count = sh.bucket;
      lowbit = shift;
      if (lowbit == 0 || count <= (uint32_t)kWave) break;
    }
    if (lowbit == 0) {                                // the threshold key itself
      thresh = prefix;
    } else {
      // 3. gather the bucket; every wave ranks it (no barrier needed after)
      const uint32_t want2 = prefix >> lowbit;
      auto gather = [&](uint32_t x, int j) {
        if ((x >> lowbit) == want2) {
          const uint32_t slot = atomicAdd(&sh.cand_count, 1u);
          if (slot < (uint32_t)kWave) {
            sh.cand_key[slot] = x;
            sh.cand_idx[slot] = j;
          }
        }
      };
      if constexpr (kRegs) {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i)
          if (valid(i)) gather(u[i], wave * kRegSpan + i * kWave + lane);
      } else {
        for (int j = tid; j < n; j += kTopkThreads) gather(order_key(s[j]), j);
      }
      __syncthreads();
      const bool mine = (uint32_t)lane < count;
      const uint32_t mkey = mine ? sh.cand_key[lane] : 0u;
      const int32_t midx = mine ? sh.cand_idx[lane] : 0;
      const uint64_t me = ((uint64_t)mkey << 32) | (0xffffffffu - (uint32_t)midx);
      uint32_t rank = 0;
      for (uint32_t m = 0; m < count; ++m) {
        const uint64_t other = ((uint64_t)sh.cand_key[m] << 32) |
                               (0xffffffffu - (uint32_t)sh.cand_idx[m]);
        rank += other > me;
      }
      const uint64_t hit = __ballot(mine && rank == krem - 1);
      const int tl = (int)__ffsll((unsigned long long)hit) - 1;
      thresh = (uint32_t)__builtin_amdgcn_readlane((int)mkey, tl);
      const int32_t tidx = __builtin_amdgcn_readlane(midx, tl);
      // equal-key pairs at or above the threshold pair
      const uint64_t eq = __ballot(mine && mkey == thresh && midx <= tidx);
      krem = (uint32_t)__popcll(eq);
    }
  }

  // 4. ascending output.  Wave w owns pages [w*span, (w+1)*span), 64 at a time.
  const int span = kRegs ? kRegSpan : ((n + kTopkThreads - 1) / kTopkThreads) * kWave;
  const int w0 = wave * span;
  const int iters = kRegs ? kPerThread : span / kWave;
  const uint64_t below = (1ull << lane) - 1ull;
  auto key_at = [&](int i, int j) -> uint32_t {
    if constexpr (kRegs) return u[i];
    else return j < n ? order_key(s[j]) : 0u;
  };
  uint32_t gt_w = 0, eq_w = 0;
#pragma unroll
  for (int i = 0; i < iters; ++i) {
    const int j = w0 + i * kWave + lane;
    const uint32_t x = key_at(i, j);
    gt_w += (uint32_t)__popcll(__ballot(j < n && x > thresh));
    eq_w += (uint32_t)__popcll(__ballot(j < n && x == thresh));
  }
  __syncthreads();                                    // wave_a/b free again
  if (lane == 0) {
    sh.wave_a[wave] = gt_w;
    sh.wave_b[wave] = eq_w;
  }
  __syncthreads();
  uint32_t gt_b = 0, eq_b = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    gt_b += (w < wave) ? sh.wave_a[w] : 0u;
    eq_b += (w < wave) ? sh.wave_b[w] : 0u;
  }
#pragma unroll
  for (int i = 0; i < iters; ++i) {
    const int j = w0 + i * kWave + lane;
    const uint32_t x = key_at(i, j);
    const bool is_gt = j < n && x > thresh;
    const bool is_eq = j < n && x == thresh;
    const uint64_t mgt = __ballot(is_gt), meq = __ballot(is_eq);
    const uint32_t gt_before = gt_b + (uint32_t)__popcll(mgt & below);
    const uint32_t eq_before = eq_b + (uint32_t)__popcll(meq & below);
    if (is_gt || (is_eq && eq_before < krem)) {
      const uint32_t pos = gt_before + min(eq_before, krem);
      if (pos < (uint32_t)k) out[pos] = j;            // never past the row
    }
    gt_b += (uint32_t)__popcll(mgt);
    eq_b += (uint32_t)__popcll(meq);
  }
}

hipError_t launch_topk(const Dims &dm, int batch, const float *scores,
                       const int32_t *ctx_lens, const int32_t *budget_tokens,
                       int max_k, int32_t *sel_pages, int32_t *num_sel,
                       hipStream_t stream) {
  dim3 grid((unsigned)(batch * dm.Hkv));
  if (dm.max_pages <= kRegKeys)
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
