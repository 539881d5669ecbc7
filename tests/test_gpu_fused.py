"""GPU parity of quest_topk_sparse_decode (top-k and attention in one kernel
where the shape allows, two kernels otherwise).

Its selection must equal quest_topk_pages_forced's bit for bit (that kernel
is itself held to the oracle in test_gpu_parity.py), its outputs must meet
the oracle at the usual tolerance, and where it falls back to two kernels its
outputs must equal quest_sparse_decode's bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from helpers import to_f64
from kv_cache_decode_quest_amd import quest, workloads
from kv_cache_decode_quest_amd.workloads import WORKLOADS, scaled
from parity import SMALL, Layer, check_request_output, log, topk_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

CASES = {name: w for name, w in SMALL.items() if w.dtype == "bf16"}
CASES["bench128k_b4"] = scaled(WORKLOADS["bench128k"], batch=4, ctx=20000,
                               budget_tokens=2048, steps=1)
# 64 requests x 4 KV heads = 256 rows: one work-group per row, no merge
CASES["rows256"] = workloads.Workload("rows256", 64, 32, 4, 128, 16, "bf16",
                                      ctx_range=(1, 1500), budget_tokens=320, steps=1,
                                      seed=91, poison=float("nan"))
# Several rounds per split (the later rounds' page ids come from the split's
# LDS list): 256 rows of 128 pages, one split of 4 rounds and no merge (the
# 48-layer step's plan); 32 rows of 1024 pages, 8 splits of 4 rounds; and
# one request of 4 KV heads keeping 2048 pages, 64 one-round splits per row
# (the decode plan's split count, which sizes the workspace)
CASES["rounds4_rows256"] = workloads.Workload("rounds4_rows256", 64, 32, 4, 128, 16, "bf16",
                                              ctx_range=(1000, 6000), budget_tokens=2048,
                                              steps=1, seed=93, poison=float("nan"),
                                              permute_pages=True)
CASES["rounds4_rows32"] = workloads.Workload("rounds4_rows32", 8, 32, 4, 128, 16, "bf16",
                                             ctx_range=(16500, 22000), budget_tokens=16384,
                                             steps=1, seed=94)
CASES["batch1_long"] = workloads.Workload("batch1_long", 1, 32, 4, 128, 16, "bf16",
                                             ctx=40000, budget_tokens=32768, steps=1, seed=95)
# rounds of the fused plan per split, where a case asserts it
ROUNDS = {"rounds4_rows256": 4, "rounds4_rows32": 4, "batch1_long": 1}
# 40 requests: 160 rows, one split each
CASES["rows160_d64"] = workloads.Workload("rows160_d64", 40, 16, 4, 64, 32, "bf16",
                                          ctx_range=(0, 3000), budget_tokens=640, steps=1,
                                          seed=92, permute_pages=True)


def pages_per_round(P, D):
    """Pages an 8-wave decode round takes (the fused kernel's 16 waves take
    the same): 32 KB of K/V per wave at D 128."""
    if P < 16:
        return 2 * pages_per_round(16, D)
    return 8 * (4 if P * D <= 2048 else (2 if P * D <= 4096 else 1))


def expect_fused(w, L, max_k):
    """The documented rule: bf16, rows of at most 8192 pages, D 64 or (D 128,
    P 16), each row split into at most min(256 / rows, the decode plan's
    splits) parts of whole rounds, of at most 256 pages."""
    rows = w.batch * quest.selection_rows(L)
    cap = max(1, min(256 // rows, quest.quest_sparse_decode_plan(L, w.batch, max_k)["num_splits"]))
    per_round = pages_per_round(w.page_size, w.head_dim)
    pps = -(-(-(-max_k // cap)) // per_round) * per_round
    n_split = -(-max_k // pps)
    return (w.dtype == "bf16" and L.max_pages_per_seq <= 8192
            and (w.head_dim == 64 or (w.head_dim == 128 and w.page_size == 16))
            and pps <= 256 and rows * n_split <= 256)


def one_bf16_ulp(a, b):
    """|a - b| within one bf16 rounding step of the larger magnitude (the
    two paths sum the same fp32 terms in a different order)."""
    return np.abs(a - b) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-6


def run_case(w, n_sink=0, n_recent=0, per_q_head=False):
    lay = Layer(w, DEV)
    if per_q_head:
        lay.L = quest.make_layout(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                                  w.torch_dtype, lay.lay.num_pool_pages, lay.lay.max_pages,
                                  per_q_head=True)
    sm = workloads.default_sm_scale(w)
    for step in range(w.steps):
        q, k_new, v_new = lay.step_inputs(step)
        bufs = lay.buffers(extra=1)
        lay.append_score_step(q, k_new, v_new, bufs)       # scores and the plain top-k
        budgets = lay.budgets()
        if n_sink or n_recent:
            quest.quest_topk_pages_forced(lay.L, bufs.scores, lay.ctx, budgets, bufs.max_k,
                                          n_sink, n_recent, bufs.sel_pages, bufs.num_sel)
        lay.attend(q, bufs)
        fb = lay.buffers(bufs.max_k)
        fb.sel_pages.fill_(-7)
        quest.quest_topk_sparse_decode(lay.L, q, lay.k_cache, lay.v_cache, lay.pt, lay.ctx,
                                       bufs.scores, budgets, bufs.max_k, sm, fb.sel_pages,
                                       fb.num_sel, fb.out, fb.workspace, n_sink, n_recent)
        torch.cuda.synchronize()
        fused = quest.quest_topk_sparse_decode_fused(lay.L, w.batch, bufs.max_k)
        assert fused == expect_fused(w, lay.L, bufs.max_k)
        plan = quest.quest_topk_sparse_decode_plan(lay.L, w.batch, bufs.max_k)
        log(f"{w.name} step {step}: max_k {bufs.max_k}, plan {plan}")
        if w.name in ROUNDS:
            assert fused and plan["pages_per_split"] == \
                ROUNDS[w.name] * pages_per_round(w.page_size, w.head_dim), plan
        assert torch.equal(fb.num_sel, bufs.num_sel)
        assert torch.equal(fb.sel_pages, bufs.sel_pages)
        two, one = to_f64(bufs.out), to_f64(fb.out)
        if not fused:
            assert torch.equal(fb.out.view(torch.int16), bufs.out.view(torch.int16))
        else:
            assert np.all(one_bf16_ulp(one, two)), float(np.abs(one - two).max())
        sel, nsel = fb.sel_pages.cpu().numpy(), fb.num_sel.cpu().numpy()
        for r in range(w.batch):
            ref = lay.oracle_request(q, r, per_q_head=per_q_head, n_sink=n_sink,
                                     n_recent=n_recent)
            check_request_output(lay, q, r, sel[r], nsel[r], one[r], ref,
                                 f"{w.name} fused r{r}", per_q_head=per_q_head)
            if int(lay.ctx[r]) == 0:
                assert np.all(one[r] == 0.0)
    return lay


@pytest.mark.parametrize("name", list(CASES))
def test_fused_matches_two_calls_and_oracle(name, gpu_lib):
    run_case(CASES[name])


@pytest.mark.parametrize("name", ["layer32k_small", "g12_d64", "p8_d64"])
def test_fused_per_q_head(name, gpu_lib):
    run_case(SMALL[name], per_q_head=True)


def test_fused_forced_pages(gpu_lib):
    """Sink and recent pages: the selection equals quest_topk_pages_forced's
    and the outputs that of the decode of that selection; the outputs also
    meet the oracle's decode with the same forcing."""
    w = scaled(WORKLOADS["layer32k"], batch=3, ctx=4000, budget_tokens=512, steps=1)
    lay = run_case(w, n_sink=1, n_recent=2)
    q = lay.step_inputs(0)[0]
    bufs = lay.buffers()
    quest.quest_page_scores(lay.L, q, lay.kmeta, lay.pt, lay.ctx, bufs.scores)
    quest.quest_topk_sparse_decode(lay.L, q, lay.k_cache, lay.v_cache, lay.pt, lay.ctx,
                                   bufs.scores, lay.budgets(), bufs.max_k,
                                   workloads.default_sm_scale(w), bufs.sel_pages, bufs.num_sel,
                                   bufs.out, bufs.workspace, 1, 2)
    torch.cuda.synchronize()
    assert quest.quest_topk_sparse_decode_fused(lay.L, w.batch, bufs.max_k)
    sel, nsel = bufs.sel_pages.cpu().numpy(), bufs.num_sel.cpu().numpy()
    out = to_f64(bufs.out)
    for r in range(w.batch):
        ref = lay.oracle_request(q, r, n_sink=1, n_recent=2)
        check_request_output(lay, q, r, sel[r], nsel[r], out[r], ref, f"fused forced r{r}")


def test_fused_bench_shape_equals_two_calls(gpu_lib):
    """The benchmark's own shape (batch 8 x 128000 tokens, budget 4096): one
    fused launch of 256 work-groups; the selection equals the top-k kernel's
    and the outputs the two-kernel path's within one bf16 step."""
    w = WORKLOADS["bench128k"]
    lay = Layer(w, DEV, host=False)
    q, k_new, v_new = lay.step_inputs(0)
    bufs = lay.buffers(extra=1)
    lay.append_score_step(q, k_new, v_new, bufs)
    lay.attend(q, bufs)
    fb = lay.buffers(bufs.max_k)
    quest.quest_topk_sparse_decode(lay.L, q, lay.k_cache, lay.v_cache, lay.pt, lay.ctx,
                                   bufs.scores, lay.budgets(), bufs.max_k,
                                   workloads.default_sm_scale(w), fb.sel_pages, fb.num_sel,
                                   fb.out, fb.workspace)
    torch.cuda.synchronize()
    assert quest.quest_topk_sparse_decode_fused(lay.L, w.batch, bufs.max_k)
    assert torch.equal(fb.num_sel, bufs.num_sel)
    assert torch.equal(fb.sel_pages, bufs.sel_pages)
    one, two = to_f64(fb.out), to_f64(bufs.out)
    assert np.all(one_bf16_ulp(one, two)), float(np.abs(one - two).max())


@pytest.mark.parametrize("n_max,P,D,max_k,forced", [
    (300, 16, 128, 298, (0, 0)), (300, 16, 128, 298, (1, 2)), (2050, 32, 64, 400, (0, 0)),
    (8008, 16, 128, 256, (0, 0)), (8008, 16, 128, 256, (4, 4)), (900, 8, 64, 300, (0, 0)),
    (500, 64, 64, 200, (2, 1))])
def test_fused_selection_on_constructed_rows(n_max, P, D, max_k, forced, gpu_lib):
    """The fused kernel's selection on score rows built to reach every branch
    of the row selection (distinct keys, heavy ties, all equal, signed zeros,
    adjacent floats, more than 64 keys tied at the threshold, wide and narrow
    ranges; k = 1, n - 1, n, truncation by max_k; forced pages) equals the
    oracle's, and its outputs equal the two-call path's within one bf16 step."""
    gen = torch.Generator().manual_seed(7000 + n_max + P)
    rows = topk_rows(n_max, gen)
    Hkv, G = 2, 8
    B = (len(rows) + 1) // 2
    while len(rows) < B * Hkv:
        rows.append(torch.randn(n_max, generator=gen))
    scores = torch.stack(rows).reshape(B, Hkv, n_max).contiguous().to(DEV)
    ctx_choices = [n_max * P, n_max * P - P + 1, 1, P + 1, (n_max // 2) * P, n_max * P - 3]
    bud_choices = [3 * P, (n_max - 1) * P, 5, 0, n_max * P * 2, P * (n_max // 3) + 7]
    ctx = torch.tensor([ctx_choices[b % 6] for b in range(B)], dtype=torch.int32, device=DEV)
    bud = torch.tensor([bud_choices[b % 6] for b in range(B)], dtype=torch.int32, device=DEV)
    pool = B * n_max
    L = quest.make_layout(G * Hkv, Hkv, D, P, torch.bfloat16, pool, n_max)
    assert quest.quest_topk_sparse_decode_fused(L, B, max_k)
    pt = torch.arange(pool, dtype=torch.int32, device=DEV).view(B, n_max)
    g = torch.Generator(device=DEV).manual_seed(8000 + n_max)
    k_cache = torch.randn((pool, Hkv, P, D), generator=g, device=DEV).to(torch.bfloat16)
    v_cache = torch.randn((pool, Hkv, D, P), generator=g, device=DEV).to(torch.bfloat16)
    q = torch.randn((B, G * Hkv, D), generator=g, device=DEV).to(torch.bfloat16)
    sm = D ** -0.5
    ns, nr = forced
    two = quest.alloc_decode_buffers(L, B, max_k, DEV)
    one = quest.alloc_decode_buffers(L, B, max_k, DEV)
    one.sel_pages.fill_(12345)
    quest.quest_topk_pages_forced(L, scores, ctx, bud, max_k, ns, nr, two.sel_pages, two.num_sel)
    quest.quest_sparse_decode(L, q, k_cache, v_cache, pt, ctx, two.sel_pages, two.num_sel, max_k,
                              sm, two.out, two.workspace)
    quest.quest_topk_sparse_decode(L, q, k_cache, v_cache, pt, ctx, scores, bud, max_k, sm,
                                   one.sel_pages, one.num_sel, one.out, one.workspace, ns, nr)
    torch.cuda.synchronize()
    sel, nsel = one.sel_pages.cpu().numpy(), one.num_sel.cpu().numpy()
    s64 = scores.cpu().double().numpy()
    for b in range(B):
        n = min(-(-int(ctx[b]) // P), n_max)
        k = min(oracle.pages_for_budget(int(bud[b]), int(ctx[b]), P), max_k)
        for h in range(Hkv):
            want = oracle.select(np.ascontiguousarray(s64[b, h, :n]), k, ns, nr)
            assert nsel[b, h] == k, (b, h)
            assert np.array_equal(sel[b, h, :k], want), (b, h, n, k)
            assert np.all(sel[b, h, k:] == -1)
    assert torch.equal(one.sel_pages, two.sel_pages)
    a, c = to_f64(one.out), to_f64(two.out)
    assert np.all(one_bf16_ulp(a, c)), float(np.abs(a - c).max())


def range_floor_rows(n_max, gen):
    """Four score rows per request: low outliers (-inf and -1e30 among normal
    scores), most keys tied at the row's maximum, one -inf among normal
    scores, and plain normal scores."""
    low = torch.randn(n_max, generator=gen) + 30.0
    low[torch.randperm(n_max, generator=gen)[: n_max // 400]] = float("-inf")
    low[torch.randint(0, n_max, (3,), generator=gen)] = -1e30
    top = torch.full((n_max,), 2.0)
    top[torch.randperm(n_max, generator=gen)[: n_max // 8]] = \
        torch.randn(n_max // 8, generator=gen) - 4.0
    one = torch.randn(n_max, generator=gen)
    one[int(torch.randint(0, n_max, (1,), generator=gen))] = float("-inf")
    return [low, top, one, torch.randn(n_max, generator=gen)]


@pytest.mark.parametrize("n_max,ns,ks,fused", [
    (8008, (8008, 7800), (1, 64, 256, 1000, 1024, 1025), True),
    (10000, (10000, 7800), (1, 64, 256, 1000, 1024, 1025), False),
    (2049, (2049, 1500), (1, 64, 128, 500, 704, 705), True)])
def test_selection_range_floor(n_max, ns, ks, fused, gpu_lib):
    """The threshold's range starts at the least of the largest keys of the
    selection threads that hold keys, when k is at most their number (which
    leaves low outliers out of the first histogram), else at the least key.
    Rows that fill the table stride or end inside a wave's span (at stride
    2049, 704 threads hold pages of a full row and 512 of a 1500-page one; at
    8008 and 10000 all 1024), k on both sides of the holders' count: the
    top-k kernel's selection, and the fused kernel's where the shape allows
    it, equal the oracle's; the fused outputs equal the two-call path's within
    one bf16 step."""
    P, D, Hkv, G = 16, 128, 4, 8
    gen = torch.Generator().manual_seed(9100 + n_max)
    B = len(ks) * len(ns)
    rows = [r for _ in range(B) for r in range_floor_rows(n_max, gen)]
    scores = torch.stack(rows).reshape(B, Hkv, n_max).contiguous().to(DEV)
    ctx = torch.tensor([ns[b % 2] * P - (b % 3) for b in range(B)], dtype=torch.int32,
                       device=DEV)
    bud = torch.tensor([ks[b // 2] * P + (b % 5) for b in range(B)], dtype=torch.int32,
                       device=DEV)
    max_k = max(ks)
    pool = n_max                                   # every request reads the same pages
    L = quest.make_layout(G * Hkv, Hkv, D, P, torch.bfloat16, pool, n_max)
    assert quest.quest_topk_sparse_decode_fused(L, B, max_k) == fused
    two = quest.alloc_decode_buffers(L, B, max_k, DEV)
    quest.quest_topk_pages(L, scores, ctx, bud, max_k, two.sel_pages, two.num_sel)
    log(f"range floor n_max {n_max}: {B} requests x {Hkv} heads, k {ks}")
    outs = [two]
    if fused:
        pt = torch.arange(pool, dtype=torch.int32, device=DEV).repeat(B, 1).contiguous()
        g = torch.Generator(device=DEV).manual_seed(9200 + n_max)
        k_cache = torch.randn((pool, Hkv, P, D), generator=g, device=DEV).to(torch.bfloat16)
        v_cache = torch.randn((pool, Hkv, D, P), generator=g, device=DEV).to(torch.bfloat16)
        q = torch.randn((B, G * Hkv, D), generator=g, device=DEV).to(torch.bfloat16)
        sm = D ** -0.5
        one = quest.alloc_decode_buffers(L, B, max_k, DEV)
        one.sel_pages.fill_(12345)
        quest.quest_sparse_decode(L, q, k_cache, v_cache, pt, ctx, two.sel_pages, two.num_sel,
                                  max_k, sm, two.out, two.workspace)
        quest.quest_topk_sparse_decode(L, q, k_cache, v_cache, pt, ctx, scores, bud, max_k, sm,
                                       one.sel_pages, one.num_sel, one.out, one.workspace)
        outs.append(one)
    torch.cuda.synchronize()
    s64 = scores.cpu().double().numpy()
    for bufs in outs:
        sel, nsel = bufs.sel_pages.cpu().numpy(), bufs.num_sel.cpu().numpy()
        for b in range(B):
            n = -(-int(ctx[b]) // P)
            k = min(oracle.pages_for_budget(int(bud[b]), int(ctx[b]), P), max_k)
            assert k == ks[b // 2]
            for h in range(Hkv):
                want = oracle.select(np.ascontiguousarray(s64[b, h, :n]), k)
                assert nsel[b, h] == k, (b, h)
                assert np.array_equal(sel[b, h, :k], want), (b, h, n, k)
                assert np.all(sel[b, h, k:] == -1)
    if fused:
        a, c = to_f64(outs[1].out), to_f64(outs[0].out)
        assert np.all(one_bf16_ulp(a, c)), float(np.abs(a - c).max())
