// plan.cpp -- launch plans of the split-K decode and of the fused top-k +
// decode kernel (declared in quest_plan.h).  Host arithmetic only: no HIP
// call, so the C ABI can size workspaces and report plans without a GPU.
#include "quest_plan.h"

#include <algorithm>

namespace quest {

namespace {

// Work-groups the plan aims for: four per resident slot (two work-groups per
// CU at the decode's LDS size), so rows of very different selection sizes
// (a ragged batch: every row's grid is sized by the largest) still spread
// over the CUs; and at most kPlanSplits splits per bf16 row, so long rows
// take several rounds per split instead of multiplying the partials the
// merge reads (a dense 8008-page row: 32 splits of 8 rounds).  Measured on
// the ragged batch (32 requests, page 32, 10% budgets): 134 us per step
// against 162 us at 1024 work-groups; the dense reference unchanged.
constexpr long kTargetWorkGroups = 2048;
constexpr long kPlanSplits = 32;

// Shapes whose 16-wave decode fits the 128 registers a 1024-thread
// work-group leaves each lane (the others spill, and stay two launches).
bool fused_shape(int P, int D) { return D == 64 || (D == 128 && P == 16); }

}  // namespace

DecodePlan decode_plan(const Dims &dm, int batch, int max_k) {
  DecodePlan p{1, max_k > 0 ? max_k : 1};
  if (batch <= 0 || max_k <= 0) return p;
  // A round: the bf16 kernel's waves take pages_per_wave pages each at once;
  // the fp32 kernel walks its pages one at a time (each a chain of loads and
  // barriers), so its splits start at one page.
  const long per_round = dm.dtype == 1 ? (long)kDecodeWaves * pages_per_wave(dm.P, dm.D) : 1;
  const long rows = (long)batch * dm.R;
  long want_splits = std::max(1L, (kTargetWorkGroups + rows - 1) / rows);
  if (dm.dtype == 1) want_splits = std::min(want_splits, kPlanSplits);
  long rounds = 1;
  while ((max_k + per_round * rounds - 1) / (per_round * rounds) >
         std::min((long)kMaxSplits, want_splits) && per_round * rounds < max_k)
    ++rounds;
  const long pps = per_round * rounds;
  p.pages_per_split = (int)pps;
  p.n_split = (int)((max_k + pps - 1) / pps);
  return p;
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
  p.pages_per_split = (int)pps;
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
