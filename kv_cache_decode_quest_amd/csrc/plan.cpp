// plan.cpp -- launch plans of the split-K decode and of the fused top-k +
// decode kernel (declared in quest_plan.h).  Host arithmetic only: no HIP
// call, so the C ABI can size workspaces and report plans without a GPU.
#include "quest_plan.h"

#include <stdint.h>

#include <algorithm>

namespace quest {

namespace {

// fp32: work-groups the plan aims for (the fp32 kernel walks its pages one at
// a time, so its splits start at one page and the grid sets how many).
constexpr long kTargetWorkGroups = 2048;
// bf16: at most kPlanSplits splits per row, or as many as give every CU a
// split when the batch has fewer than kLiveGrid / kPlanSplits rows, so long
// rows take several rounds per split instead of multiplying the work-group
// merges and the partials the merge kernel reads (a dense 8008-page row of
// batch 8: 8 splits of 32 rounds; the ragged batch's longest rows, 383
// pages of 32 tokens: 8 splits of 3 rounds); otherwise one round per split,
// the unit the live-split decode spreads over its work-groups.  Measured on
// the ragged batch, at most 4 / 6 / 8 / 12 / 32 splits per row: 130.3 /
// 111.3 / 108.4 / 110.5 / 116.8 us per step; rows of up to 8 rounds (batch 8
// x 128000 at a 4096-token budget, the 48-layer step, the 32k layer) keep
// one round per split.
constexpr long kPlanSplits = 8;

// Shapes whose 16-wave decode fits the 128 registers a 1024-thread
// work-group leaves each lane (the others spill, and stay two launches).
bool fused_shape(int P, int D) { return D == 64 || (D == 128 && P == 16); }

}  // namespace

DecodePlan decode_plan(const Dims &dm, int batch, int max_k) {
  DecodePlan p{1, max_k > 0 ? max_k : 1};
  if (batch <= 0 || max_k <= 0) return p;
  long pps;
  if (dm.dtype == 1) {
    // A round: the bf16 kernel's waves take pages_per_wave pages each at
    // once.  One round per split, or as many as keep the splits within the
    // cap.
    const long per_round = (long)kDecodeWaves * pages_per_wave(dm.P, dm.D);
    const long one_round = (max_k + per_round - 1) / per_round;
    const long rows = (long)batch * dm.R;
    const long cap = std::max(kPlanSplits,
                              std::min((long)kMaxSplits, (kLiveGrid + rows - 1) / rows));
    pps = per_round * ((one_round + cap - 1) / cap);
  } else {
    // fp32: one page per split, more only past the grid the plan aims for
    // (or kMaxSplits per row).
    const long rows = (long)batch * dm.R;
    const long want = std::min((long)kMaxSplits,
                               std::max(1L, (kTargetWorkGroups + rows - 1) / rows));
    pps = (max_k + want - 1) / want;
  }
  p.pages_per_split = (int)pps;
  p.n_split = (int)((max_k + pps - 1) / pps);
  return p;
}

bool decode_live(const Dims &dm, int batch) {
  return dm.dtype == 1 && batch > 0 && (long)batch * dm.R <= kLiveRows;
}

int decode_grid(const Dims &dm, int batch, int max_k) {
  const long splits = (long)batch * dm.R * decode_plan(dm, batch, max_k).n_split;
  return (int)(decode_live(dm, batch) ? std::min(splits, (long)kLiveGrid) : splits);
}

size_t decode_workspace_bytes(const Dims &dm, int batch, int max_k) {
  if (batch <= 0) return 0;
  const DecodePlan p = decode_plan(dm, batch, max_k);
  return (size_t)batch * dm.R * p.n_split * dm.Gcols * (dm.D + 2) * sizeof(float);
}

// The fused kernel's plan: as many splits per row as keep the grid within
// one resident work-group per CU, each a whole number of the decode's
// rounds, and never more splits than decode_plan gives (whose partials the
// caller's workspace is sized for; a small batch with a large max_k takes
// more rounds per split instead).  A row of one split writes its output
// directly (no merge launch).
DecodePlan fused_plan(const Dims &dm, int batch, int max_k) {
  const long rows = (long)batch * dm.R;
  const long per_round = (long)kDecodeWaves * pages_per_wave(dm.P, dm.D);
  const long cap = std::max(1L, std::min(kFusedMaxWorkGroups / std::max(1L, rows),
                                         (long)decode_plan(dm, batch, max_k).n_split));
  long pps = (max_k + cap - 1) / cap;
  pps = (pps + per_round - 1) / per_round * per_round;
  DecodePlan p;
  // a split this long is never fused (more than kMaxFusedPages); the clamp
  // only keeps the reported size from wrapping when max_k nears INT32_MAX
  p.pages_per_split = (int)std::min(pps, (long)INT32_MAX);
  p.n_split = (int)((max_k + pps - 1) / pps);
  return p;
}

bool topk_decode_fused(const Dims &dm, int batch, int max_k) {
  if (dm.dtype != 1 || dm.max_pages > kRegKeys || !fused_shape(dm.P, dm.D) || max_k <= 0 ||
      batch <= 0)
    return false;
  const DecodePlan p = fused_plan(dm, batch, max_k);
  return p.pages_per_split <= kMaxFusedPages &&
         (long)batch * dm.R * p.n_split <= kFusedMaxWorkGroups;
}

}  // namespace quest
