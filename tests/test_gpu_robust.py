"""GPU test of page-table entries outside the pool.  A live page whose id lies
outside [0, num_pool_pages) scores -inf, is never stored to and gives no
token to the attention; no kernel touches memory outside the pool for it.

The K, V and metadata pools are allocated with guard pages past the declared
pool, and every bad entry points into that guard region.  A missing bounds
check would then touch allocated memory only, and would show up as changed
guard bytes, or as results that depend on what the guard pages hold (two runs
with different guard contents must agree bit for bit).  Requests whose
tables are intact must match a run without bad entries bit for bit."""
from __future__ import annotations

import pytest
import torch

from kv_cache_decode_quest_amd import quest, workloads
from kv_cache_decode_quest_amd.workloads import WORKLOADS, scaled
from parity import log

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
GUARD = 3                    # guard pages past the declared pool
STEPS = 2                    # decode steps, one appended token per request each
BAD = (1, 3)                 # requests with out-of-pool entries
FULL = 1                     # ... of which this one selects every page

CASES = {
    # bf16, page 16, D 128: the fused top-k + decode kernel
    "bf16_p16": scaled(WORKLOADS["layer32k"], batch=4, ctx=2999, budget_tokens=512,
                       steps=STEPS),
    # bf16, page 32, permuted pages: the top-k kernel, then the live-split decode
    "bf16_p32": scaled(WORKLOADS["ragged"], batch=4, ctx_range=(1500, 4000),
                       budget_page_div=4, steps=STEPS),
    # fp32, page 16, D 64: the fp32 kernels
    "f32": scaled(WORKLOADS["tiny"], batch=4, ctx=1499, budget_tokens=256, steps=STEPS),
}


def pages_of(ctx, P):
    return (int(ctx) + P - 1) // P


def run(w, lay, table, guard_fill, budgets, max_k):
    """Prefill through the intact table, then STEPS decode steps
    (quest_decode_step) through `table`.  Returns the pools with their guard
    pages and the last step's buffers."""
    pool, P, D, Hkv, dt = lay.num_pool_pages, w.page_size, w.head_dim, w.num_kv_heads, w.torch_dtype
    L = quest.make_layout(w.num_q_heads, Hkv, D, P, dt, pool, lay.max_pages)
    full = [torch.zeros((pool + GUARD, Hkv, P, D), dtype=dt, device=DEV),
            torch.zeros((pool + GUARD, Hkv, D, P), dtype=dt, device=DEV),
            torch.zeros((pool + GUARD, Hkv, 2, D), dtype=dt, device=DEV)]
    for t in full:
        t[pool:] = guard_fill
    k_cache, v_cache, kmeta = (t[:pool] for t in full)
    k_new, v_new, cu, ctx_before = workloads.prefill_tokens(w, lay, DEV)
    quest.quest_append_kv(L, k_new, v_new, cu, ctx_before, int(lay.ctx0.max()), lay.page_table,
                          k_cache, v_cache, kmeta)
    bufs = quest.alloc_decode_buffers(L, w.batch, max_k, DEV)
    bufs.scores.fill_(0.0)           # entries past a request are never written
    cu1 = torch.arange(w.batch + 1, dtype=torch.int32, device=DEV)
    ctx = lay.ctx0.clone()
    for s in range(STEPS):
        q, kn, vn = workloads.step_tokens(w, DEV, 0, s)
        quest.quest_decode_step(L, q, kn, vn, cu1, ctx, 1, table, k_cache, v_cache, kmeta,
                                ctx + 1, budgets, max_k, workloads.default_sm_scale(w),
                                bufs.scores, bufs.sel_pages, bufs.num_sel, bufs.out,
                                bufs.workspace)
        ctx = ctx + 1
    torch.cuda.synchronize()
    return full, bufs


def bits(t):
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


@pytest.mark.parametrize("name", list(CASES))
def test_out_of_pool_page_ids(name, gpu_lib):
    w = CASES[name]
    P = w.page_size
    lay = workloads.make_layout(w, DEV)
    pool = lay.num_pool_pages
    ctx0 = lay.ctx0.cpu().tolist()
    n_end = [pages_of(c + STEPS, P) for c in ctx0]
    budgets = workloads.budget_tokens(w, lay.ctx0 + STEPS)
    budgets[FULL] = n_end[FULL] * P                       # every page of this request
    max_k = max(n_end)
    # bad entries: two earlier pages and every page the decode steps append to
    table = lay.page_table.clone()
    bad_pages = {}
    for r in BAD:
        logical = sorted({1, n_end[r] // 2} | {p // P for p in range(ctx0[r], ctx0[r] + STEPS)})
        for i, j in enumerate(logical):
            table[r, j] = pool + i % GUARD
        bad_pages[r] = logical
    L = quest.make_layout(w.num_q_heads, w.num_kv_heads, w.head_dim, P, w.torch_dtype, pool,
                          lay.max_pages)
    log(f"out-of-pool {name}: pool {pool} (+{GUARD} guard pages), bad pages {bad_pages}, "
        f"max_k {max_k}, plan {quest.quest_topk_sparse_decode_plan(L, w.batch, max_k)}")

    clean_fill, fill_a, fill_b = 1.0, 2.0, -3.0e4
    clean, cb = run(w, lay, lay.page_table, clean_fill, budgets, max_k)
    pools_a, ba = run(w, lay, table, fill_a, budgets, max_k)
    pools_b, bb = run(w, lay, table, fill_b, budgets, max_k)

    # 1. nothing was stored past the pool
    for pools, fill in ((clean, clean_fill), (pools_a, fill_a), (pools_b, fill_b)):
        for t in pools:
            assert bool((t[pool:] == fill).all()), "a guard page was written"
    # 2. nothing was read past the pool: the results do not depend on the guard
    for x, y in ((ba.scores, bb.scores), (ba.sel_pages, bb.sel_pages),
                 (ba.num_sel, bb.num_sel), (ba.out, bb.out)):
        assert torch.equal(bits(x), bits(y))
    for x, y in zip(pools_a, pools_b):
        assert torch.equal(bits(x[:pool]), bits(y[:pool]))
    # 3. out-of-pool pages score -inf and are never preferred over a scored page
    for r in BAD:
        for j in bad_pages[r]:
            assert bool((ba.scores[r, :, j] == float("-inf")).all()), (r, j)
    r = BAD[1]
    for row in range(ba.sel_pages.shape[1]):
        k = int(ba.num_sel[r, row])
        assert 0 < k < n_end[r] - len(bad_pages[r])
        sel = set(ba.sel_pages[r, row, :k].tolist())
        assert not sel & set(bad_pages[r]), (r, row)
    # the full-budget request selects its bad pages too: the decode skips them
    assert bool((ba.num_sel[FULL] == n_end[FULL]).all())
    assert bool(torch.isfinite(ba.out.float()).all())
    # 4. requests with intact tables match the run without bad entries
    for r in range(w.batch):
        if r in BAD:
            continue
        n = n_end[r]
        assert torch.equal(bits(ba.scores[r, :, :n]), bits(cb.scores[r, :, :n])), r
        assert torch.equal(ba.num_sel[r], cb.num_sel[r]), r
        assert torch.equal(ba.sel_pages[r], cb.sel_pages[r]), r
        assert torch.equal(bits(ba.out[r]), bits(cb.out[r])), r
