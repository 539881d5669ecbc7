/*
 * abi_sanitize_driver.c -- drives every entry point of include/quest.h through
 * the library's host code (quest_abi.cpp, plan.cpp) with the kernel launchers
 * replaced by host stand-ins (abi_sanitize_stubs.cpp), so the validation,
 * plan and workspace arithmetic run under the address and
 * undefined-behaviour sanitizers with no GPU (tests/test_abi_sanitize.py).
 *
 * Checks: a valid call returns QUEST_OK and reaches exactly one launcher; each
 * documented rejection returns its status and launches nothing; a seeded
 * sweep of layouts and sizes (extremes included) never launches on a
 * rejected call, and every accepted decode plan covers max_k with no empty
 * split, within 256 splits, with the fused plan never wider than the
 * workspace's.  Device pointers are fake, aligned addresses: nothing is
 * dereferenced on the host.  Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "quest.h"

extern int stub_launches;
extern int stub_last_batch;
extern int stub_last_max_k;
extern void *stub_last_workspace;

#define D(addr) ((void *)(uintptr_t)(addr))
static void *const P = D(0x100000);            /* aligned fake device pointers */
static int32_t *const I = (int32_t *)D(0x200000);
static float *const F = (float *)D(0x300000);
static void *const WS = D(0x400000);
static void *const MIS = D(0x100002);           /* misaligned */

static int failures = 0;
#define CHECK(cond, what)                                                        \
  do {                                                                           \
    if (!(cond)) {                                                               \
      fprintf(stderr, "abi driver: %s (line %d)\n", what, __LINE__);             \
      ++failures;                                                                \
    }                                                                            \
  } while (0)

static quest_layout layout(int hq, int hkv, int d, int p, int dt, int64_t pool, int maxp) {
  quest_layout L;
  memset(&L, 0, sizeof L);
  L.abi_version = QUEST_ABI_VERSION;
  L.num_q_heads = hq;
  L.num_kv_heads = hkv;
  L.head_dim = d;
  L.page_size = p;
  L.dtype = dt;
  L.num_pool_pages = pool;
  L.max_pages_per_seq = maxp;
  L.selection = QUEST_SELECT_PER_KV_HEAD;
  return L;
}

/* Status of a call and whether it reached a launcher exactly when it
 * succeeded with a nonzero batch. */
static void expect(int st, int want, int before, int batch, const char *what) {
  const int launched = stub_launches - before;
  if (st != want) {
    fprintf(stderr, "abi driver: %s: status %d, expected %d\n", what, st, want);
    ++failures;
  }
  const int want_launch = (want == QUEST_OK && batch > 0) ? 1 : 0;
  if (launched != want_launch) {
    fprintf(stderr, "abi driver: %s: %d launches, expected %d\n", what, launched,
            want_launch);
    ++failures;
  }
}

static int append_call(const quest_layout *L, int batch, void *k_new) {
  return quest_append_kv(L, batch, k_new, P, I, I, 1, I, P, P, P, NULL);
}
static int scores_call(const quest_layout *L, int batch, int reduce, void *q) {
  return quest_page_scores(L, batch, q, P, I, I, reduce, F, NULL);
}
static int append_score_call(const quest_layout *L, int batch, int max_new) {
  return quest_append_score(L, batch, P, P, P, I, I, max_new, I, P, P, P, 0, F, NULL);
}
static int topk_call(const quest_layout *L, int batch, int max_k, int ns, int nr) {
  return quest_topk_pages_forced(L, batch, F, I, I, max_k, ns, nr, I, I, NULL);
}
static int decode_call(const quest_layout *L, int batch, int max_k, void *ws, size_t wsb,
                       float scale) {
  return quest_sparse_decode(L, batch, P, P, P, I, I, I, I, max_k, scale, P, ws, wsb, NULL);
}
static int combined_call(const quest_layout *L, int batch, int max_k, void *ws, size_t wsb) {
  return quest_topk_sparse_decode(L, batch, P, P, P, I, I, F, I, max_k, 0, 0, 0.1f, I, I, P,
                                  ws, wsb, NULL);
}
static int step_call(const quest_layout *L, int batch, int max_k, void *ws, size_t wsb) {
  return quest_decode_step(L, batch, P, P, P, I, I, 1, I, P, P, P, 0, I, I, max_k, 0, 0, 0.1f,
                           F, I, I, P, ws, wsb, NULL);
}
static int noalloc_call(const quest_layout *L, int batch, int max_k) {
  return quest_decode_step_noalloc(L, batch, P, P, P, I, I, 1, I, P, P, P, 0, I, I, max_k, 0, 0,
                                   0.1f, F, I, I, P, NULL);
}

static uint64_t rng = 0x243f6a8885a308d3ull;
static uint32_t next(void) {
  rng = rng * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(rng >> 33);
}
/* An entry of v[0..n): three times in four one of the first `valid` (the
 * supported values), else any (extremes and rejected values). */
static int pick(const int *v, int valid, int n) {
  return (next() % 4 != 0) ? v[next() % (uint32_t)valid] : v[next() % (uint32_t)n];
}

int main(void) {
  int b;
  CHECK(quest_abi_version() == QUEST_ABI_VERSION, "abi version");
  for (int st = -8; st <= 0; ++st) CHECK(quest_status_string(st) != NULL, "status string");

  const quest_layout L = layout(32, 4, 128, 16, QUEST_BF16, 8 * 8009, 8009);
  const size_t need = quest_sparse_decode_workspace_bytes(&L, 8, 256);
  CHECK(need > 0, "workspace bytes");

  /* valid calls reach one launcher each */
  b = stub_launches; expect(append_call(&L, 8, P), QUEST_OK, b, 8, "append");
  b = stub_launches; expect(scores_call(&L, 8, QUEST_REDUCE_MAX, P), QUEST_OK, b, 8, "scores");
  b = stub_launches; expect(append_score_call(&L, 8, 1), QUEST_OK, b, 8, "append+scores");
  b = stub_launches; expect(topk_call(&L, 8, 256, 1, 2), QUEST_OK, b, 8, "top-k forced");
  b = stub_launches;
  expect(quest_topk_pages(&L, 8, F, I, I, 256, I, I, NULL), QUEST_OK, b, 8, "top-k");
  b = stub_launches; expect(decode_call(&L, 8, 256, WS, need, 0.1f), QUEST_OK, b, 8, "decode");
  CHECK(stub_last_workspace == WS && stub_last_max_k == 256, "decode arguments passed on");
  b = stub_launches; expect(combined_call(&L, 8, 256, WS, need), QUEST_OK, b, 8, "combined");
  b = stub_launches; expect(step_call(&L, 8, 256, WS, need), QUEST_OK, b, 8, "step");
  b = stub_launches; expect(noalloc_call(&L, 8, 256), QUEST_OK, b, 8, "step, no allocation");
  CHECK(stub_last_workspace != NULL && stub_last_workspace != WS, "static scratch passed on");

  /* batch 0 launches nothing, even with NULL pointers */
  b = stub_launches;
  expect(quest_append_kv(&L, 0, NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL),
         QUEST_OK, b, 0, "append, batch 0");
  b = stub_launches; expect(decode_call(&L, 0, 4, NULL, 0, 0.1f), QUEST_OK, b, 0, "decode, batch 0");
  b = stub_launches; expect(noalloc_call(&L, 0, 4), QUEST_OK, b, 0, "no allocation, batch 0");

  /* documented rejections launch nothing */
  b = stub_launches; expect(append_call(NULL, 8, P), QUEST_ERR_NULL, b, 8, "NULL layout");
  b = stub_launches; expect(append_call(&L, 8, NULL), QUEST_ERR_NULL, b, 8, "NULL k_new");
  {
    quest_layout bad = L;
    bad.abi_version = 2;
    b = stub_launches; expect(scores_call(&bad, 8, 0, P), QUEST_ERR_ABI, b, 8, "abi mismatch");
    bad = L; bad.num_q_heads = 30;
    b = stub_launches; expect(scores_call(&bad, 8, 0, P), QUEST_ERR_SHAPE, b, 8, "Hq % Hkv");
    bad = L; bad.head_dim = 96;
    b = stub_launches; expect(scores_call(&bad, 8, 0, P), QUEST_ERR_UNSUPPORTED, b, 8, "D 96");
    bad = L; bad.page_size = 48;
    b = stub_launches; expect(scores_call(&bad, 8, 0, P), QUEST_ERR_UNSUPPORTED, b, 8, "P 48");
    bad = L; bad.num_q_heads = 4 * 17;
    b = stub_launches; expect(scores_call(&bad, 8, 0, P), QUEST_ERR_UNSUPPORTED, b, 8, "G 17");
    bad = L; bad.dtype = 7;
    b = stub_launches; expect(scores_call(&bad, 8, 0, P), QUEST_ERR_UNSUPPORTED, b, 8, "dtype");
    bad = L; bad.selection = 5;
    b = stub_launches; expect(scores_call(&bad, 8, 0, P), QUEST_ERR_UNSUPPORTED, b, 8, "selection");
    bad = L; bad.max_pages_per_seq = INT32_MAX;
    b = stub_launches; expect(scores_call(&bad, 8, 0, P), QUEST_ERR_SHAPE, b, 8, "row too long");
    bad = L; bad.num_pool_pages = 0;
    b = stub_launches; expect(scores_call(&bad, 8, 0, P), QUEST_ERR_SHAPE, b, 8, "empty pool");
  }
  b = stub_launches; expect(scores_call(&L, 8, 2, P), QUEST_ERR_UNSUPPORTED, b, 8, "reduce 2");
  b = stub_launches; expect(scores_call(&L, 8, 0, MIS), QUEST_ERR_SHAPE, b, 8, "misaligned q");
  b = stub_launches; expect(scores_call(&L, 65536, 0, P), QUEST_ERR_SHAPE, b, 65536, "batch 65536");
  b = stub_launches; expect(scores_call(&L, -1, 0, P), QUEST_ERR_SHAPE, b, -1, "batch -1");
  b = stub_launches; expect(append_score_call(&L, 8, -1), QUEST_ERR_SHAPE, b, 8, "max_new -1");
  b = stub_launches; expect(topk_call(&L, 8, 0, 0, 0), QUEST_ERR_SHAPE, b, 8, "max_k 0");
  b = stub_launches; expect(topk_call(&L, 8, 16, -1, 0), QUEST_ERR_SHAPE, b, 8, "n_sink -1");
  b = stub_launches;
  expect(decode_call(&L, 8, 256, WS, need - 1, 0.1f), QUEST_ERR_WORKSPACE, b, 8, "small workspace");
  b = stub_launches;
  expect(decode_call(&L, 8, 256, D(0x400004), need, 0.1f), QUEST_ERR_WORKSPACE, b, 8,
         "misaligned workspace");
  b = stub_launches;
  expect(decode_call(&L, 8, 256, WS, need, 1.0f / 0.0f), QUEST_ERR_SHAPE, b, 8, "scale inf");
  b = stub_launches;
  expect(combined_call(&L, 8, 256, NULL, need), QUEST_ERR_WORKSPACE, b, 8, "combined, no workspace");
  b = stub_launches;
  expect(step_call(&L, 8, 256, WS, need - 16), QUEST_ERR_WORKSPACE, b, 8, "step, small workspace");
  b = stub_launches;
  expect(noalloc_call(&L, 1100, 16), QUEST_ERR_SCRATCH, b, 1100, "no allocation, beyond scratch");

  /* plan queries */
  {
    int32_t ns = 0, pps = 0, fu = -1;
    CHECK(quest_sparse_decode_plan(&L, 8, 256, &ns, &pps) == QUEST_OK, "plan");
    CHECK(ns * pps >= 256 && (ns - 1) * pps < 256, "plan covers max_k");
    CHECK(quest_topk_sparse_decode_plan(&L, 8, 256, &fu, &ns, &pps) == QUEST_OK, "combined plan");
    CHECK(fu == 1 && ns == 8 && pps == 32, "combined plan at batch 8 x 128000");
    CHECK(quest_topk_sparse_decode_plan(&L, 8, 256, NULL, &ns, &pps) == QUEST_ERR_NULL,
          "combined plan, NULL output");
    CHECK(quest_topk_sparse_decode_fused(&L, 8, 256) == 1, "fused at batch 8 x 128000");
    CHECK(quest_topk_sparse_decode_fused(&L, 8, 0) == QUEST_ERR_SHAPE, "fused, max_k 0");
  }

  /* seeded sweep, extremes included: no sanitizer report, no launch on a
   * rejected call, every accepted plan consistent */
  static const int hq[] = {1, 2, 4, 8, 12, 16, 32, 64, 256, 0, -4, 33};
  static const int hkv[] = {1, 2, 4, 8, 16, 0, -1, 3};
  static const int dims[] = {64, 128, 0, -64, 96, 256};
  static const int pages[] = {8, 16, 32, 64, 0, -16, 48, 128};
  static const int dts[] = {QUEST_F32, QUEST_BF16, 2, -1};
  static const int maxps[] = {1, 2, 63, 64, 65, 8009, 8192, 8193, 1 << 20, 1 << 28,
                              INT32_MAX, 0, -5};
  static const int batches[] = {0, 1, 2, 7, 8, 64, 255, 1024, 65535, 65536, -1, 1 << 30};
  static const int maxks[] = {1, 2, 16, 31, 32, 33, 255, 256, 257, 2048, 8192, 100000,
                              INT32_MAX, 0, -3};
  static const int64_t pools[] = {1, 64064, ((int64_t)1) << 40, INT64_MAX, 0, -1};
  int accepted = 0;
  for (int it = 0; it < 40000; ++it) {
    quest_layout S = layout(pick(hq, 9, 12), pick(hkv, 5, 8), pick(dims, 2, 6),
                            pick(pages, 4, 8), pick(dts, 2, 4), pools[next() % 6],
                            pick(maxps, 10, 13));
    S.selection = (next() % 5 == 0) ? QUEST_SELECT_PER_Q_HEAD : QUEST_SELECT_PER_KV_HEAD;
    const int batch = pick(batches, 10, 12), max_k = pick(maxks, 13, 15);
    const size_t wsb = quest_sparse_decode_workspace_bytes(&S, batch, max_k);
    int32_t ns = 0, pps = 0, fu = 0, fns = 0, fpps = 0;
    const int pst = quest_sparse_decode_plan(&S, batch, max_k, &ns, &pps);
    const int fst = quest_topk_sparse_decode_plan(&S, batch, max_k, &fu, &fns, &fpps);
    CHECK(pst == fst, "plan statuses agree");
    if (pst == QUEST_OK) {
      CHECK(pps >= 1 && ns >= 1 && ns <= 256, "plan bounds");
      CHECK((int64_t)ns * pps >= max_k && (int64_t)(ns - 1) * pps < max_k, "plan covers max_k");
      if (batch > 0) {
        /* the decode's grid (rows x splits work-groups, 512 threads for bf16
         * and 256 for fp32; the live-split form launches fewer) and the
         * merge's (one 128-thread work-group per q head) stay within 2^32
         * work-items */
        const int64_t rows = (int64_t)batch * (S.selection == QUEST_SELECT_PER_Q_HEAD
                                                   ? S.num_q_heads : S.num_kv_heads);
        const int64_t threads = S.dtype == QUEST_BF16 ? 512 : 256;
        CHECK(rows * ns * threads < ((int64_t)1 << 32), "decode grid within 2^32 work-items");
        CHECK((int64_t)batch * S.num_q_heads * 128 < ((int64_t)1 << 32),
              "merge grid within 2^32 work-items");
      }
      if (fu) {
        CHECK(fns <= ns, "fused plan within the workspace's splits");
        CHECK((int64_t)fns * fpps >= max_k && (int64_t)(fns - 1) * fpps < max_k,
              "fused plan covers max_k");
      }
    }
    b = stub_launches;
    const int st = decode_call(&S, batch, max_k, WS, wsb, 0.1f);
    const int launched = stub_launches - b;
    CHECK(launched == ((st == QUEST_OK && batch > 0) ? 1 : 0), "decode launches iff accepted");
    if (st == QUEST_OK && batch > 0) {
      ++accepted;
      CHECK(wsb > 0 && pst == QUEST_OK, "an accepted decode has a workspace and a plan");
    }
    b = stub_launches;
    const int st2 = step_call(&S, batch, max_k, WS, wsb);
    CHECK(stub_launches - b == ((st2 == QUEST_OK && batch > 0) ? 1 : 0),
          "step launches iff accepted");
    b = stub_launches;
    const int st3 = noalloc_call(&S, batch, max_k);
    CHECK(stub_launches - b == ((st3 == QUEST_OK && batch > 0) ? 1 : 0),
          "no-allocation step launches iff accepted");
    if (st3 == QUEST_OK && batch > 0) CHECK(wsb <= QUEST_STATIC_SCRATCH_BYTES, "within scratch");
    b = stub_launches;
    const int st4 = scores_call(&S, batch, (int)(next() % 3), P);
    CHECK(stub_launches - b == ((st4 == QUEST_OK && batch > 0) ? 1 : 0),
          "scores launch iff accepted");
  }
  CHECK(accepted > 2000, "the sweep accepted enough calls");
  if (failures) {
    fprintf(stderr, "abi driver: %d failures\n", failures);
    return 1;
  }
  printf("abi driver ok: %d launches, %d accepted sweep decodes\n", stub_launches, accepted);
  return 0;
}
