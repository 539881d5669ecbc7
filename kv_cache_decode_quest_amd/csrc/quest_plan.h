// quest_plan.h -- shapes and launch plans of the decode kernels: plain host
// arithmetic (no HIP call, no device code), shared by the C ABI's validation
// and workspace sizing (quest_abi.cpp), the launchers, and the kernels'
// compile-time constants.  plan.cpp holds the functions.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace quest {

struct Dims {
  int Hq, Hkv, G, D, P;
  int dtype;          // 0 fp32, 1 bf16
  int64_t pool;       // physical pages
  int max_pages;      // page-table row stride
  // Selection rows: a request has R rows of scores / selections, row x holds
  // q heads x*Gcols .. x*Gcols+Gcols-1 and reads KV head x / gdiv.  Shared
  // per KV head: R = Hkv, Gcols = G, gdiv = 1; per q head: R = Hq, Gcols = 1,
  // gdiv = G.
  int R, Gcols, gdiv;
  bool per_head() const { return R != Hkv || Gcols != G; }
};

struct DecodePlan {
  int n_split;          // splits per (request, selection row)
  int pages_per_split;  // selected pages one work-group attends
};

// Waves of a bf16 decode work-group, and the most splits a row may have.
constexpr int kDecodeWaves = 8;
constexpr int kMaxSplits = 256;

// Pages one wave of the 8-wave bf16 decode loads at once (one round): 32 KB
// of K and V per wave in flight at D = 128 (4 pages of 16 tokens, 2 of 32, 1
// of 64), so the page registers stay within budget.  8-token pages go two to
// a 16-token tile (twice the pages of 16-token ones).
constexpr int pages_per_wave(int P, int D) {
  return P < 16 ? 2 * pages_per_wave(16, D) : ((P * D <= 2048) ? 4 : (P * D <= 4096 ? 2 : 1));
}

// Rows of up to kRegKeys pages are selected from registers (one read of the
// score row); the fused top-k + decode kernel needs such rows.
constexpr int kRegKeys = 8192;
// The fused kernel keeps at most kMaxFusedPages page ids per split in LDS
// and runs at most one work-group per CU of an MI355X.
constexpr int kMaxFusedPages = 256;
constexpr long kFusedMaxWorkGroups = 256;

// The standalone decode's plan.  Pure arithmetic; batch > 0 and max_k > 0
// give n_split >= 1.
DecodePlan decode_plan(const Dims &dm, int batch, int max_k);

// The bf16 standalone decode runs only the splits that hold selected pages
// ("live" splits: ceil(count / pages_per_split) of each row): every
// work-group lists them from the rows' selection counts in LDS; with U live
// splits the first A = ceil(U / ceil(U / kLiveGrid)) work-groups take equal
// shares (work-group b: splits b, b + A, b + 2A, ...) and the rest exit.
// Used while the rows' list fits (kLiveRows rows).
// kLiveGrid is one work-group on each of an MI355X's 256 CUs: the 8-wave
// decode needs about 200 registers per lane (two waves per SIMD), so one
// work-group is resident per CU and the whole grid runs at once.
constexpr int kLiveRows = 1024;
constexpr int kLiveGrid = 256;
bool decode_live(const Dims &dm, int batch);
// Work-groups of the standalone decode launch.
int decode_grid(const Dims &dm, int batch, int max_k);

// Bytes of split partials the decode (standalone or fused) writes: the
// caller's workspace must hold this many.
size_t decode_workspace_bytes(const Dims &dm, int batch, int max_k);

// Whether the combined top-k + decode runs as one fused kernel, and its
// plan.  The fused plan never has more splits than decode_plan, so the
// workspace of decode_workspace_bytes holds its partials.
bool topk_decode_fused(const Dims &dm, int batch, int max_k);
DecodePlan fused_plan(const Dims &dm, int batch, int max_k);

}  // namespace quest
