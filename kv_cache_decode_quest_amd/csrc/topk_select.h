// topk_select.h -- build_decode_view, part 2: the top-k pages of every
// (request, KV head) row within the request's token budget, as device code
// shared by the top-k kernel and the fused top-k + decode kernel.
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
// reductions use the DPP network and ballots, not LDS round trips, and
// cross-wave sums read one LDS word per lane.
//  1. the range the threshold key lies in: up to the largest key, from the
//     least key or, where that is larger, the least of the largest keys of
//     the threads that hold keys (each of those holds a key at least that
//     large, so when they are k or more, so is the threshold); every key in
//     the range shares the bits above the highest bit where its ends differ.
//     The second bound keeps low outliers (a partly filled last page, pages
//     outside the pool at -inf) from widening the first histogram's buckets;
//  2. refinement: an (up to) 11-bit histogram of the keys matching the known
//     prefix, on the next bits, gives the bucket holding the k-th largest key
//     and the count kept above it; repeated until the bucket holds at most 64
//     keys (one pass on rows of a few thousand normal scores) or the key is
//     fully known;
//  3. the bucket's keys are gathered into LDS (register rows also count, per
//     wave, the keys above the bucket) and one wave ranks the (key, page)
//     pairs in the 64-bit order, which fixes the threshold pair;
//  4. one ballot pass: a page is kept iff its pair is at or above the
//     threshold pair; a wave's first position is the above-bucket keys of
//     earlier waves plus the kept bucket keys at lower pages, and lane
//     positions are prefixes of the ballot masks (v_mbcnt).  Rows over 8192
//     pages, and thresholds resolved to a full key, take a two-pass form
//     instead: a count pass, one barrier to exchange the per-wave counts,
//     then a write pass that puts every page above the threshold key, and
//     the lowest-index pages equal to it up to the count still needed, at
//     its ascending position.
#pragma once
#include "quest_device.h"
#include "quest_plan.h"

namespace quest {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
constexpr int kBinsPerLane = kBins / kTopkThreads;   // each lane owns this many buckets
constexpr int kBinsPerWave = kBinsPerLane * kWave;
static_assert(kBinsPerLane * kTopkThreads == kBins && kTopkWaves <= 16, "bucket ownership");

// Larger score <-> larger key; -0.0 and +0.0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  u = u == 0x80000000u ? 0u : u;                     // -0.0 -> +0.0
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

struct TopkShared {
  uint32_t hist[kBins];
  uint32_t wave_a[kTopkWaves], wave_b[kTopkWaves], wave_c[kTopkWaves], wave_d[kTopkWaves];
  uint32_t cand_key[kWave];
  int32_t cand_idx[kWave];
  uint32_t cnt_gt[kTopkWaves], cnt_eq[kTopkWaves];   // per-wave output counts
  uint32_t cand_count;
  uint32_t prefix;     // known high bits of the threshold key
  uint32_t krem;       // keys still to take at or below the known prefix
  uint32_t bucket;     // keys in the chosen bucket
  uint32_t thresh;     // the threshold pair (key, page), once ranked
  int32_t tidx;
  uint32_t keq;        // keys equal to the threshold key that are kept
};

// Sum of vals[w] over the waves w before `wave` (vals: kTopkWaves entries in
// LDS): lane l < 16 reads vals[l], masked by l < wave, and row 0 sums its 16
// lanes on the DPP network.  Uniform result.
__device__ __forceinline__ uint32_t sum_of_earlier_waves(const uint32_t *vals, int wave) {
  const int lane = lane_id();
  uint32_t x = lane < wave ? vals[lane & (kTopkWaves - 1)] : 0u;
  x += dpp_row<kRowShr1>(0u, x);
  x += dpp_row<kRowShr2>(0u, x);
  x += dpp_row<kRowShr4>(0u, x);
  x += dpp_row<kRowShr8>(0u, x);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
}

// min of vals_lo[w] and vals_c[w], max of vals_hi[w] over all waves, the
// same way.
__device__ __forceinline__ void range_over_waves(const uint32_t *vals_lo,
                                                 const uint32_t *vals_hi,
                                                 const uint32_t *vals_c, uint32_t &lo,
                                                 uint32_t &hi, uint32_t &c) {
  const int lane = lane_id() & (kTopkWaves - 1);
  uint32_t a = vals_lo[lane], b = vals_hi[lane], f = vals_c[lane];
  a = min(a, dpp_row<kRowShr1>(a, a));
  b = max(b, dpp_row<kRowShr1>(b, b));
  f = min(f, dpp_row<kRowShr1>(f, f));
  a = min(a, dpp_row<kRowShr2>(a, a));
  b = max(b, dpp_row<kRowShr2>(b, b));
  f = min(f, dpp_row<kRowShr2>(f, f));
  a = min(a, dpp_row<kRowShr4>(a, a));
  b = max(b, dpp_row<kRowShr4>(b, b));
  f = min(f, dpp_row<kRowShr4>(f, f));
  a = min(a, dpp_row<kRowShr8>(a, a));
  b = max(b, dpp_row<kRowShr8>(b, b));
  f = min(f, dpp_row<kRowShr8>(f, f));
  lo = (uint32_t)__builtin_amdgcn_readlane((int)a, 15);
  hi = (uint32_t)__builtin_amdgcn_readlane((int)b, 15);
  c = (uint32_t)__builtin_amdgcn_readlane((int)f, 15);
}

// The bucket (of `bins` <= kBins) holding the krem-th largest counted key,
// buckets ranked from the top: wave w owns the kBinsPerWave buckets below the
// top kBinsPerWave*w, lane l kBinsPerLane of them.  Results in sh.prefix /
// sh.krem / sh.bucket.
__device__ __forceinline__ void pick_bucket(TopkShared &sh, int bins, uint32_t krem,
                                            uint32_t prefix, int shift) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int top = bins - 1 - kBinsPerWave * wave - kBinsPerLane * lane;
  uint32_t c[kBinsPerLane], total = 0;
#pragma unroll
  for (int e = 0; e < kBinsPerLane; ++e) {
    c[e] = top - e >= 0 ? sh.hist[top - e] : 0u;
    total += c[e];
  }
  const uint32_t incl = wave_incl_sum(total);
  if (lane == kWave - 1) sh.wave_a[wave] = incl;
  __syncthreads();
  uint32_t run = sum_of_earlier_waves(sh.wave_a, wave) + incl - total;   // keys above `top`
#pragma unroll
  for (int e = 0; e < kBinsPerLane; ++e) {
    if (run < krem && krem <= run + c[e]) {
      sh.prefix = prefix | ((uint32_t)(top - e) << shift);
      sh.krem = krem - run;
      sh.bucket = c[e];
    }
    run += c[e];
  }
  __syncthreads();
}

// Rows of up to kRegKeys pages are read from HBM once, into registers: wave w
// holds pages [S w, S w + S) with S = reg_span(max_pages), lane l pages
// S w + 64 i + l (i < S / 64), the same wave-contiguous order the output pass
// needs, so no pass re-reads memory.  S spreads the row's stride over all
// waves in whole 64-page slots, so short rows keep every wave busy.  Longer
// rows read their scores from global memory in every pass.
constexpr int kPerThread = kRegKeys / kTopkThreads;

__host__ __device__ constexpr int reg_span(int max_pages) {
  const int slots = ((max_pages + kTopkWaves - 1) / kTopkWaves + kWave - 1) / kWave;
  return (slots < kPerThread ? (slots > 0 ? slots : 1) : kPerThread) * kWave;
}

// k = min(max_k, clamp(floor(budget / P), 1, n)) of the row's n pages (n =
// 0 and k = 0 for a request with no token); P a power of two.
__device__ __forceinline__ void row_size(int ctx, int budget, int log2p, int max_pages,
                                         int max_k, int &n, int &k) {
  n = ctx <= 0 ? 0 : min((ctx + (1 << log2p) - 1) >> log2p, max_pages);
  k = 0;
  if (n > 0) {
    k = budget >> log2p;                              // floor; negatives clamp to 1 below
    k = k < 1 ? 1 : (k > n ? n : k);
    k = k < max_k ? k : max_k;
  }
}

// The selection of one row by a kTopkThreads work-group; every thread calls
// it.  s: the row's scores in global memory; sv: this thread's scores of a
// register row (wave w, lane l, slot i holds page span w + 64 i + l for
// i < span / 64; span = reg_span(row stride));
// n pages, k of them kept (0 <= k <= n).  emit(pos, page) is called once for
// each kept page with its position pos in [0, k) of the ascending page list.
// kForced: the first n_sink and the last n_recent pages rank above every
// scored page, the lower page first among them (without, n_sink and
// n_recent are ignored).
template <bool kRegs, bool kForced, typename Emit>
__device__ __forceinline__ void select_row(TopkShared &sh, const float *__restrict__ s,
                                           const float (&sv)[kRegs ? kPerThread : 1], int span,
                                           int n, int k, int n_sink, int n_recent, Emit emit) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  if (k == n) {                                       // the whole row (or nothing)
    for (int i = tid; i < n; i += kTopkThreads) emit(i, i);
    return;
  }
  // Forced pages are emitted here; the radix select below runs over the
  // scored pages [a, b) for the kk places they leave.
  int a = 0, b = n, kk = k;
  if constexpr (kForced) {
    const int ns = min(n_sink, n), nr = min(n_recent, n - ns);
    a = ns;
    b = n - nr;
    if (k <= ns + nr) {                               // only forced pages: the lowest k
      for (int i = tid; i < k; i += kTopkThreads) emit(i, i < ns ? i : b + (i - ns));
      return;
    }
    kk = k - ns - nr;
    for (int i = tid; i < ns; i += kTopkThreads) emit(i, i);               // sink pages
    for (int i = tid; i < nr; i += kTopkThreads) emit(ns + kk + i, b + i); // recent pages
    if (kk == b - a) {                                // and every scored page
      for (int i = tid; i < kk; i += kTopkThreads) emit(a + i, a + i);
      return;
    }
  }
  auto in_row = [&](int j) { return (!kForced || j >= a) && j < b; };
  // The page of register slot i (slots past the span hold none: -1).
  const int nslots = span / kWave;
  auto slot_page = [&](int i) { return i < nslots ? wave * span + i * kWave + lane : -1; };
  // The thread's keys: registers, or global memory for long rows.  Slots
  // outside the scored range never count; their key is 0.
  uint32_t u[kRegs ? kPerThread : 1];
  if constexpr (kRegs) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int j = slot_page(i);
      u[i] = j >= 0 && in_row(j) ? order_key(sv[i]) : 0u;
    }
  }
  auto valid = [&](int i) { const int j = slot_page(i); return j >= 0 && in_row(j); };

  // 1. min and max key, and the least of the largest keys of the threads
  // that hold keys, with the number of those threads
  uint32_t lo = 0xffffffffu, hi = 0u;
  bool holds = false;
  if constexpr (kRegs) {
    // slots outside the range hold key 0, which never raises hi
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      lo = min(lo, valid(i) ? u[i] : 0xffffffffu);
      hi = max(hi, u[i]);
      holds = holds || valid(i);
    }
  } else {
    for (int j = a + tid; j < b; j += kTopkThreads) {
      const uint32_t x = order_key(s[j]);
      lo = min(lo, x);
      hi = max(hi, x);
    }
    holds = a + tid < b;
  }
  uint32_t top = holds ? hi : 0xffffffffu;
  const uint32_t holders = (uint32_t)__popcll(__ballot(holds));
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  top = wave_min_u32(top);
  if (lane == 0) {
    sh.wave_a[wave] = lo;
    sh.wave_b[wave] = hi;
    sh.wave_c[wave] = top;
    sh.wave_d[wave] = holders;
  }
#pragma unroll
  for (int e = 0; e < kBinsPerLane; ++e) sh.hist[kBinsPerLane * tid + e] = 0;
  if (tid == 0) sh.cand_count = 0;
  __syncthreads();
  range_over_waves(sh.wave_a, sh.wave_b, sh.wave_c, lo, hi, top);
  const uint32_t n_holders = sum_of_earlier_waves(sh.wave_d, kTopkWaves);

  uint32_t thresh, krem = (uint32_t)kk;
  if (lo == hi) {                                     // every key equal: the lowest kk pages
    for (int i = tid; i < kk; i += kTopkThreads) emit(a + i, a + i);
    return;
  }
  // Each of the n_holders threads holding keys holds one >= top, so for
  // kk <= n_holders the threshold key is >= top too.
  const uint32_t floor_key = (uint32_t)kk <= n_holders ? max(lo, top) : lo;
  // 2. refine the threshold key, 11 bits at a time.  floor_key == hi: at
  // least kk keys equal hi, which is then the threshold key.
  int lowbit = floor_key == hi ? 0 : 32 - __builtin_clz(floor_key ^ hi);   // bits >= lowbit known
  uint32_t prefix = (uint32_t)(((uint64_t)hi >> lowbit) << lowbit);
  uint32_t count = 0;
  for (bool first_pass = true; lowbit > 0; first_pass = false) {
    const int w = lowbit < kDigitBits ? lowbit : kDigitBits;
    const int shift = lowbit - w;
    const uint32_t bmask = (1u << w) - 1u;
    const uint32_t himask = lowbit >= 32 ? 0u : (0xffffffffu << lowbit);
    if (!first_pass) {
#pragma unroll
      for (int e = 0; e < kBinsPerLane; ++e) sh.hist[kBinsPerLane * tid + e] = 0;
      __syncthreads();
    }
    if constexpr (kRegs) {
#pragma unroll
      for (int i = 0; i < kPerThread; ++i)
        if (valid(i) && ((u[i] ^ prefix) & himask) == 0u)
          atomicAdd(&sh.hist[(u[i] >> shift) & bmask], 1u);
    } else {
      for (int j = a + tid; j < b; j += kTopkThreads) {
        const uint32_t x = order_key(s[j]);
        if (((x ^ prefix) & himask) == 0u) atomicAdd(&sh.hist[(x >> shift) & bmask], 1u);
      }
    }
    __syncthreads();
    pick_bucket(sh, 1 << w, krem, prefix, shift);
    prefix = sh.prefix;
    krem = sh.krem;
    count = __builtin_amdgcn_readfirstlane(sh.bucket);
    lowbit = shift;
    if (lowbit == 0 || count <= (uint32_t)kWave) break;
  }
  if (lowbit == 0) {                                  // the threshold key itself
    thresh = prefix;
  } else {
    // 3. gather the bucket (at most 64 keys) into LDS; wave 0 ranks the
    // (key, page) pairs in the 64-bit order and publishes the threshold pair.
    // Register rows also count, per wave, the keys above the bucket: all of
    // them are kept.
    const uint32_t himask = 0xffffffffu << lowbit;    // 1 <= lowbit <= 31 here
    const uint32_t bucket_top = prefix | ~himask;     // largest key of the bucket
    auto gather = [&](uint32_t x, int j) {
      if (((x ^ prefix) & himask) == 0u) {
        const uint32_t slot = atomicAdd(&sh.cand_count, 1u);
        if (slot < (uint32_t)kWave) {
          sh.cand_key[slot] = x;
          sh.cand_idx[slot] = j;
        }
      }
    };
    if constexpr (kRegs) {
      uint32_t above = 0;
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) {
        if (valid(i)) gather(u[i], slot_page(i));
        above += (uint32_t)__popcll(__ballot(valid(i) && u[i] > bucket_top));
      }
      if (lane == 0) sh.cnt_gt[wave] = above;
    } else {
      for (int j = a + tid; j < b; j += kTopkThreads) gather(order_key(s[j]), j);
    }
    __syncthreads();
    if (wave == 0) {
      const bool mine = (uint32_t)lane < count;
      const uint32_t mkey = mine ? sh.cand_key[lane] : 0u;
      const int32_t midx = mine ? sh.cand_idx[lane] : 0;
      // rank = candidates before this one: a larger key, or the same key
      // at a lower page
      uint32_t rank = 0;
      for (uint32_t m = 0; m < count; ++m) {
        const uint32_t ok = (uint32_t)__builtin_amdgcn_readlane((int)mkey, (int)m);
        const int32_t oi = __builtin_amdgcn_readlane(midx, (int)m);
        rank += (ok > mkey || (ok == mkey && oi < midx)) ? 1u : 0u;
      }
      const uint64_t hit = __ballot(mine && rank == krem - 1);
      const int tl = (int)__ffsll((unsigned long long)hit) - 1;
      const uint32_t th = (uint32_t)__builtin_amdgcn_readlane((int)mkey, tl);
      const int32_t tidx = __builtin_amdgcn_readlane(midx, tl);
      // equal-key pairs at or above the threshold pair
      const uint64_t eq = __ballot(mine && mkey == th && midx <= tidx);
      if (lane == 0) {
        sh.thresh = th;
        sh.tidx = tidx;
        sh.keq = (uint32_t)__popcll(eq);
      }
    }
    __syncthreads();
    thresh = sh.thresh;
    if constexpr (kRegs) {
      // 4a. ascending output in one pass.  A page is kept iff its (key, page)
      // pair is at or above the threshold pair.  This wave's first position:
      // the kept pages of earlier waves = their keys above the bucket plus
      // the kept candidates at a lower page than this wave's range.
      const int32_t tidx = (int32_t)sh.tidx;
      const int w0 = wave * span;
      const bool cmine = (uint32_t)lane < count;
      const uint32_t ck = cmine ? sh.cand_key[lane] : 0u;
      const int32_t ci = cmine ? sh.cand_idx[lane] : 0;
      const bool ckept = cmine && (ck > thresh || (ck == thresh && ci <= tidx));
      uint32_t pos0 = sum_of_earlier_waves(sh.cnt_gt, wave) +
                      (uint32_t)__popcll(__ballot(ckept && ci < w0));
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) {
        const int j = slot_page(i);
        const uint32_t x = u[i];
        const bool kept = valid(i) && (x > thresh || (x == thresh && j <= tidx));
        const uint64_t m = __ballot(kept);
        if (kept) {
          const uint32_t pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)m, pos0));
          if (pos < (uint32_t)kk) emit(a + (int)pos, j);   // never past the row
        }
        pos0 += (uint32_t)__popcll(m);
      }
      return;
    }
    krem = sh.keq;
  }

  // 4b. ascending output for long rows, and for ties at a fully known key.
  // Wave w owns pages [w*span, (w+1)*span), 64 at a time: a pass of ballots
  // counts the wave's kept pages (above the threshold key, and equal to it),
  // one barrier exchanges the counts, and a second pass writes every kept
  // page at its position, with lane prefixes of the ballot masks from
  // v_mbcnt.  Register rows keep the masks from the first pass; long rows
  // recompute them.
  const int wspan = kRegs ? span : ((n + kTopkThreads - 1) / kTopkThreads) * kWave;
  const int w0 = wave * wspan;
  const int iters = kRegs ? kPerThread : wspan / kWave;
  auto page_of = [&](int i) { return kRegs ? slot_page(i) : w0 + i * kWave + lane; };
  auto masks = [&](int i, uint64_t &mg, uint64_t &me) {
    const int j = page_of(i);
    const bool live = j >= 0 && in_row(j);
    uint32_t x;
    if constexpr (kRegs) x = u[i];
    else x = live ? order_key(s[j]) : 0u;
    mg = __ballot(live && x > thresh);
    me = __ballot(live && x == thresh);
  };
  constexpr int kSaved = kRegs ? kPerThread : 1;
  uint64_t sg[kSaved], se[kSaved];
  uint32_t gt_w = 0, eq_w = 0;
  auto count_pass = [&](int i) {
    uint64_t mg, me;
    masks(i, mg, me);
    if constexpr (kRegs) {
      sg[i] = mg;
      se[i] = me;
    }
    gt_w += (uint32_t)__popcll(mg);
    eq_w += (uint32_t)__popcll(me);
  };
  // (loops holding ballots unroll only at a trip count known when compiled)
  if constexpr (kRegs) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) count_pass(i);
  } else {
    for (int i = 0; i < iters; ++i) count_pass(i);
  }
  if (lane == 0) {
    sh.cnt_gt[wave] = gt_w;
    sh.cnt_eq[wave] = eq_w;
  }
  __syncthreads();
  uint32_t gt_b = sum_of_earlier_waves(sh.cnt_gt, wave);
  uint32_t eq_b = sum_of_earlier_waves(sh.cnt_eq, wave);
  auto write_pass = [&](int i) {
    uint64_t mg, me;
    if constexpr (kRegs) {
      mg = sg[i];
      me = se[i];
    } else {
      masks(i, mg, me);
    }
    // kept pages of this wave before this lane, plus those of earlier waves
    const uint32_t gt_before =
        __builtin_amdgcn_mbcnt_hi((uint32_t)(mg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mg, gt_b));
    const uint32_t eq_before =
        __builtin_amdgcn_mbcnt_hi((uint32_t)(me >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)me, eq_b));
    const bool is_gt = (mg >> lane) & 1ull;
    const bool is_eq = (me >> lane) & 1ull;
    if (is_gt || (is_eq && eq_before < krem)) {
      const uint32_t pos = gt_before + min(eq_before, krem);
      if (pos < (uint32_t)kk) emit(a + (int)pos, page_of(i));   // never past the row
    }
    gt_b += (uint32_t)__popcll(mg);
    eq_b += (uint32_t)__popcll(me);
  };
  if constexpr (kRegs) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) write_pass(i);
  } else {
    for (int i = 0; i < iters; ++i) write_pass(i);
  }
}

}  // namespace quest
