"""GPU parity: every step of the HIP path against the fp64 oracle.

Inputs are the seeded synthetic workloads (scaled down so the oracle finishes
in seconds, still spanning several tiles and a ragged tail), plus the full
benchmark shape on sampled requests.  Tolerances are documented in
tests/parity.py.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from helpers import to_f64, to_oracle
from kv_cache_decode_quest_amd import quest, workloads
from kv_cache_decode_quest_amd.workloads import WORKLOADS, scaled
from parity import (SMALL, Layer, check_kmeta, check_out, check_pool_bytes,
                    check_request_output, check_scores, compare_selection, log, topk_rows)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

def run_and_check(w, layer=0, reduce="max", fused=False):
    log(f"workload {w.name} layer {layer} reduce {reduce} fused {fused}: batch {w.batch} ctx "
        f"{workloads.context_lengths(w).tolist()[:8]}")
    lay = Layer(w, DEV, layer=layer)
    check_pool_bytes(lay)
    for r in range(w.batch):
        ctx = int(lay.ctx[r])
        if ctx:
            check_kmeta(lay, r, oracle.request_bounds(lay.shape, lay.host[0], lay.pt_host[r], ctx))
    flagged = 0
    for step in range(w.steps):
        q, k_new, v_new = lay.step_inputs(step)
        if fused:
            bufs = lay.buffers(extra=1)
            lay.append_score_step(q, k_new, v_new, bufs, reduce)
        else:
            lay.append_step(k_new, v_new)
            bufs = lay.buffers()
            lay.view(q, bufs, reduce)
        lay.attend(q, bufs)
        torch.cuda.synchronize()
        check_pool_bytes(lay)
        km = to_f64(lay.kmeta)
        scores = bufs.scores.cpu().numpy().astype(np.float64)
        sel = bufs.sel_pages.cpu().numpy()
        nsel = bufs.num_sel.cpu().numpy()
        out = to_f64(bufs.out)
        # the oracle's own selection, fed to the decode kernel directly
        sel_o = torch.full_like(bufs.sel_pages, -1)
        nsel_o = torch.zeros_like(bufs.num_sel)
        refs = []
        for r in range(w.batch):
            ref = lay.oracle_request(q, r, reduce)
            refs.append(ref)
            for g in range(w.num_kv_heads):
                sel_o[r, g, :len(ref["sel"][g])] = torch.from_numpy(ref["sel"][g])
                nsel_o[r, g] = len(ref["sel"][g])
        bufs2 = lay.buffers(bufs.max_k)
        lay.attend(q, bufs2, sel_o.to(DEV), nsel_o.to(DEV))
        torch.cuda.synchronize()
        out2 = to_f64(bufs2.out)
        qh = to_f64(q)
        for r, ref in enumerate(refs):
            if ref["bounds"].shape[0]:
                check_kmeta(lay, r, ref["bounds"], km)
                check_scores(scores[r], ref["scores"], qh[r], ref["bounds"], w.group)
            check_out(out2[r], ref["out"], w.torch_dtype, f"{w.name} r{r} (oracle selection)")
            flagged += check_request_output(lay, q, r, sel[r], nsel[r], out[r], ref,
                                            f"{w.name} r{r}")
            if int(lay.ctx[r]) == 0:
                assert np.all(out[r] == 0.0)
    log(f"workload {w.name}: ok, flagged rows {flagged}")
    return flagged


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_steps_match_oracle(name, gpu_lib):
    w = SMALL[name]
    for layer in range(w.layers):
        run_and_check(w, layer)


@pytest.mark.parametrize("name", ["tiny", "layer32k_small", "ragged_small", "edges",
                                  "edges_d64_p32", "f32_g1"])
def test_fused_append_score_matches_oracle(name, gpu_lib):
    run_and_check(SMALL[name], fused=True)


def test_group_sum_variant(gpu_lib):
    run_and_check(SMALL["layer32k_small"], reduce="sum")


def check_store_against_oracle(lay, k_c, v_c, km):
    """Pools equal the oracle's store of the same tokens byte for byte, and
    every live page's metadata equals the oracle's from-scratch min/max."""
    assert to_oracle(k_c).tobytes() == lay.host[0].tobytes(), "K pool differs from the oracle"
    assert to_oracle(v_c).tobytes() == lay.host[1].tobytes(), "V pool differs from the oracle"
    kmh = to_f64(km)
    for r in range(lay.w.batch):
        ctx = int(lay.ctx[r])
        if ctx:
            check_kmeta(lay, r, oracle.request_bounds(lay.shape, lay.host[0], lay.pt_host[r], ctx),
                        kmh)


def test_incremental_append_equals_bulk(gpu_lib):
    """Pool and metadata after token-by-token appends equal the bulk append's,
    and both equal the oracle's store and from-scratch page bounds."""
    w = scaled(WORKLOADS["ragged"], batch=3, ctx_range=(20, 200), steps=0)
    bulk = Layer(w, DEV)
    k_c, v_c = workloads.empty_pool(w, bulk.lay, DEV)
    km = torch.full_like(bulk.kmeta, -3.0)
    k_new, v_new, cu, _ = workloads.prefill_tokens(w, bulk.lay, DEV)
    cuh = cu.cpu().tolist()
    lens = [cuh[r + 1] - cuh[r] for r in range(w.batch)]
    ctx = torch.zeros(w.batch, dtype=torch.int32, device=DEV)
    for t in range(max(lens)):
        counts = [1 if t < n else 0 for n in lens]
        rows = [cuh[r] + t for r in range(w.batch) if counts[r]]
        sub_cu = torch.tensor([0] + np.cumsum(counts).tolist(), dtype=torch.int32, device=DEV)
        idx = torch.tensor(rows, dtype=torch.int64, device=DEV)
        quest.quest_append_kv(bulk.L, k_new[idx].contiguous(), v_new[idx].contiguous(), sub_cu,
                              ctx, 1, bulk.pt, k_c, v_c, km)
        ctx = ctx + torch.tensor(counts, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    assert torch.equal(ctx.cpu(), bulk.ctx.cpu())
    assert torch.equal(k_c.view(torch.int16), bulk.k_cache.view(torch.int16))
    assert torch.equal(v_c.view(torch.int16), bulk.v_cache.view(torch.int16))
    for r in range(w.batch):
        n = -(-int(bulk.ctx[r]) // w.page_size)
        phys = bulk.pt[r, :n].long()
        assert torch.equal(km[phys].view(torch.int16), bulk.kmeta[phys].view(torch.int16))
    check_store_against_oracle(bulk, k_c, v_c, km)


@pytest.mark.parametrize("page_size,chunk,ctx_range", [
    (8, 37, (200, 900)), (16, 37, (200, 900)), (32, 37, (200, 900)), (64, 37, (200, 900)),
    (16, 4096, (5000, 13000))])
def test_unaligned_and_chunked_append_match(page_size, chunk, ctx_range, gpu_lib):
    """The same tokens stored three ways give identical pools and metadata,
    equal to the oracle's store and from-scratch page bounds: one bulk append
    (16-byte vector path), chunks of `chunk` tokens per request per call
    (37: chunks that start and end inside pages; 4096: the prefill chunk
    size, page-aligned, with a partial last chunk), and one bulk append from
    source tensors shifted off 16-byte alignment (the scalar path)."""
    w = scaled(WORKLOADS["ragged"], batch=3, ctx_range=ctx_range, steps=0, page_size=page_size)
    ref = Layer(w, DEV)
    k_new, v_new, cu, _ = workloads.prefill_tokens(w, ref.lay, DEV)
    cuh = cu.cpu().tolist()
    lens = [cuh[r + 1] - cuh[r] for r in range(w.batch)]

    def fresh():
        k_c, v_c = workloads.empty_pool(w, ref.lay, DEV)
        return k_c, v_c, torch.full_like(ref.kmeta, -3.0)

    def same(k_c, v_c, km):
        assert torch.equal(k_c.view(torch.int16), ref.k_cache.view(torch.int16))
        assert torch.equal(v_c.view(torch.int16), ref.v_cache.view(torch.int16))
        for r in range(w.batch):
            n = -(-lens[r] // w.page_size)
            phys = ref.pt[r, :n].long()
            assert torch.equal(km[phys].view(torch.int16), ref.kmeta[phys].view(torch.int16))
        check_store_against_oracle(ref, k_c, v_c, km)

    # chunks of `chunk` tokens per request
    k_c, v_c, km = fresh()
    step = chunk
    for t0 in range(0, max(lens), step):
        counts = [max(0, min(step, n - t0)) for n in lens]
        rows = [cuh[r] + t0 + i for r in range(w.batch) for i in range(counts[r])]
        sub_cu = torch.tensor([0] + np.cumsum(counts).tolist(), dtype=torch.int32, device=DEV)
        ctx0 = torch.tensor([min(t0, n) for n in lens], dtype=torch.int32, device=DEV)
        idx = torch.tensor(rows, dtype=torch.int64, device=DEV)
        quest.quest_append_kv(ref.L, k_new[idx].contiguous(), v_new[idx].contiguous(), sub_cu,
                              ctx0, step, ref.pt, k_c, v_c, km)
    torch.cuda.synchronize()
    same(k_c, v_c, km)

    # source tensors one element off 16-byte alignment
    k_c, v_c, km = fresh()
    shape = tuple(k_new.shape)
    k_buf = torch.empty(k_new.numel() + 1, dtype=k_new.dtype, device=DEV)
    v_buf = torch.empty(v_new.numel() + 1, dtype=v_new.dtype, device=DEV)
    k_off, v_off = k_buf[1:].view(shape), v_buf[1:].view(shape)
    k_off.copy_(k_new)
    v_off.copy_(v_new)
    assert k_off.data_ptr() % 16 != 0
    zero = torch.zeros(w.batch, dtype=torch.int32, device=DEV)
    quest.quest_append_kv(ref.L, k_off, v_off, cu, zero, max(lens), ref.pt, k_c, v_c, km)
    torch.cuda.synchronize()
    same(k_c, v_c, km)


def test_empty_and_one_token_requests(gpu_lib):
    """A request with no token selects nothing and outputs zeros; the others
    match the oracle (decode without a preceding append)."""
    w = SMALL["edges"]
    lay = Layer(w, DEV)
    q, _, _ = lay.step_inputs(0)
    bufs = lay.buffers()
    lay.view(q, bufs)
    lay.attend(q, bufs)
    torch.cuda.synchronize()
    assert int(lay.ctx[0]) == 0
    assert bufs.num_sel[0].cpu().tolist() == [0] * w.num_kv_heads
    assert torch.all(bufs.sel_pages[0] == -1)
    assert torch.all(bufs.out[0] == 0)
    out = to_f64(bufs.out)
    sel, nsel = bufs.sel_pages.cpu().numpy(), bufs.num_sel.cpu().numpy()
    for r in range(1, w.batch):
        ref = lay.oracle_request(q, r)
        for g in range(w.num_kv_heads):
            assert compare_selection(sel[r, g], int(nsel[r, g]), ref["sel"][g],
                                     ref["scores"][g]) == "exact"
        check_out(out[r], ref["out"], w.torch_dtype, f"edges r{r}")


@pytest.mark.parametrize("n_max,P", [(64, 16), (300, 16), (2050, 32), (8008, 16), (10000, 16),
                                     (500, 64), (900, 8)])
def test_topk_exact(n_max, P, gpu_lib):
    gen = torch.Generator().manual_seed(5000 + n_max)
    rows = topk_rows(n_max, gen)
    Hkv = 2
    B = (len(rows) + 1) // 2
    while len(rows) < B * Hkv:
        rows.append(torch.randn(n_max, generator=gen))
    scores = torch.stack(rows).reshape(B, Hkv, n_max).contiguous()
    # request lengths and budgets exercise k = 1, n-1, n, n+1, truncation by max_k
    ctx_choices = [n_max * P, n_max * P - P + 1, 1, P + 1, (n_max // 2) * P, n_max * P - 3]
    bud_choices = [3 * P, (n_max - 1) * P, 5, 0, n_max * P * 2, P * (n_max // 3) + 7]
    ctx = torch.tensor([ctx_choices[b % 6] for b in range(B)], dtype=torch.int32)
    bud = torch.tensor([bud_choices[b % 6] for b in range(B)], dtype=torch.int32)
    max_k = max(1, n_max - 2)          # caps the budget-covers-all rows
    L = quest.make_layout(8 * Hkv, Hkv, 128, P, torch.bfloat16, 1, n_max)
    sel = torch.full((B, Hkv, max_k), 12345, dtype=torch.int32, device=DEV)
    nsel = torch.full((B, Hkv), -7, dtype=torch.int32, device=DEV)
    quest.quest_topk_pages(L, scores.to(DEV), ctx.to(DEV), bud.to(DEV), max_k, sel, nsel)
    torch.cuda.synchronize()
    sel, nsel = sel.cpu().numpy(), nsel.cpu().numpy()
    s64 = scores.double().numpy()
    for b in range(B):
        n = min(-(-int(ctx[b]) // P), n_max)
        k = min(oracle.pages_for_budget(int(bud[b]), int(ctx[b]), P), max_k)
        for g in range(Hkv):
            want = oracle.select(np.ascontiguousarray(s64[b, g, :n]), k)
            assert nsel[b, g] == k, (b, g)
            assert np.array_equal(sel[b, g, :k], want), (b, g, n, k)
            assert np.all(sel[b, g, k:] == -1)


@pytest.mark.parametrize("n_max,P", [(300, 16), (2050, 32), (10000, 16)])
def test_topk_forced_exact(n_max, P, gpu_lib):
    """Forced sink / recent pages: the same rows as test_topk_exact, every
    (n_sink, n_recent) pair below, compared with the oracle's selection
    (budgets include k smaller than the forced set)."""
    gen = torch.Generator().manual_seed(6000 + n_max)
    rows = topk_rows(n_max, gen)
    Hkv = 2
    B = (len(rows) + 1) // 2
    while len(rows) < B * Hkv:
        rows.append(torch.randn(n_max, generator=gen))
    scores = torch.stack(rows).reshape(B, Hkv, n_max).contiguous()
    ctx_choices = [n_max * P, n_max * P - P + 1, 1, P + 1, (n_max // 2) * P, n_max * P - 3]
    bud_choices = [3 * P, (n_max - 1) * P, 5, 0, n_max * P * 2, P * (n_max // 3) + 7]
    ctx = torch.tensor([ctx_choices[b % 6] for b in range(B)], dtype=torch.int32)
    bud = torch.tensor([bud_choices[(b + 1) % 6] for b in range(B)], dtype=torch.int32)
    max_k = max(1, n_max - 2)
    L = quest.make_layout(8 * Hkv, Hkv, 128, P, torch.bfloat16, 1, n_max)
    s64 = scores.double().numpy()
    for ns, nr in ((1, 0), (0, 1), (1, 2), (4, 4), (n_max, 0)):
        sel = torch.full((B, Hkv, max_k), 12345, dtype=torch.int32, device=DEV)
        nsel = torch.full((B, Hkv), -7, dtype=torch.int32, device=DEV)
        quest.quest_topk_pages_forced(L, scores.to(DEV), ctx.to(DEV), bud.to(DEV), max_k, ns,
                                      nr, sel, nsel)
        torch.cuda.synchronize()
        sel_h, nsel_h = sel.cpu().numpy(), nsel.cpu().numpy()
        for b in range(B):
            n = min(-(-int(ctx[b]) // P), n_max)
            k = min(oracle.pages_for_budget(int(bud[b]), int(ctx[b]), P), max_k)
            for g in range(Hkv):
                want = oracle.select(np.ascontiguousarray(s64[b, g, :n]), k, ns, nr)
                assert nsel_h[b, g] == k, (ns, nr, b, g)
                assert np.array_equal(sel_h[b, g, :k], want), (ns, nr, b, g, n, k)
                assert np.all(sel_h[b, g, k:] == -1)


def test_forced_pages_decode(gpu_lib):
    """One decode step with a sink page and two recent pages always kept:
    selections and outputs against the oracle's decode with the same forcing."""
    w = scaled(WORKLOADS["layer32k"], batch=3, ctx=4000, budget_tokens=512, steps=1)
    lay = Layer(w, DEV)
    q, k_new, v_new = lay.step_inputs(0)
    lay.append_step(k_new, v_new)
    bufs = lay.buffers()
    quest.quest_page_scores(lay.L, q, lay.kmeta, lay.pt, lay.ctx, bufs.scores)
    quest.quest_topk_pages_forced(lay.L, bufs.scores, lay.ctx, lay.budgets(), bufs.max_k, 1, 2,
                                  bufs.sel_pages, bufs.num_sel)
    lay.attend(q, bufs)
    torch.cuda.synchronize()
    sel, nsel = bufs.sel_pages.cpu().numpy(), bufs.num_sel.cpu().numpy()
    out = to_f64(bufs.out)
    for r in range(w.batch):
        ref = lay.oracle_request(q, r, n_sink=1, n_recent=2)
        n = -(-int(lay.ctx[r]) // w.page_size)
        for g in range(w.num_kv_heads):
            assert {0, n - 2, n - 1} <= set(sel[r, g, :nsel[r, g]].tolist())
        check_request_output(lay, q, r, sel[r], nsel[r], out[r], ref, f"forced r{r}")


@pytest.mark.parametrize("name,fused", [("layer32k_small", False), ("layer32k_small", True),
                                        ("edges_d64_p32", True), ("f32_g1", False)])
def test_per_q_head_selection(name, fused, gpu_lib):
    """Every q head scores and selects its own pages (no GQA sharing):
    per-head scores within the fp32 summation bound, per-head selections
    exact, and outputs against the oracle's per-q-head decode."""
    w = SMALL[name]
    lay = Layer(w, DEV)
    lay.L = quest.make_layout(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                              w.torch_dtype, lay.lay.num_pool_pages, lay.lay.max_pages,
                              per_q_head=True)
    q, k_new, v_new = lay.step_inputs(0)
    bufs = lay.buffers(extra=1)
    assert tuple(bufs.scores.shape[:2]) == (w.batch, w.num_q_heads)
    if fused:
        lay.append_score_step(q, k_new, v_new, bufs)
    else:
        lay.append_step(k_new, v_new)
        lay.view(q, bufs)
    lay.attend(q, bufs)
    torch.cuda.synchronize()
    scores = bufs.scores.cpu().numpy().astype(np.float64)
    sel, nsel = bufs.sel_pages.cpu().numpy(), bufs.num_sel.cpu().numpy()
    out = to_f64(bufs.out)
    qh = to_f64(q)
    G = w.num_q_heads // w.num_kv_heads
    for r in range(w.batch):
        ref = lay.oracle_request(q, r, per_q_head=True)
        n = ref["scores"].shape[1]
        if n:
            mag = np.maximum(np.abs(ref["bounds"][:, :, 0, :]), np.abs(ref["bounds"][:, :, 1, :]))
            kv_of = np.arange(w.num_q_heads) // G
            tol = 2.0 * (w.head_dim + 2) * 2.0 ** -24 * np.einsum(
                "hd,jhd->hj", np.abs(qh[r]), mag[:, kv_of, :]) + 1e-30
            assert np.all(np.abs(scores[r, :, :n] - ref["scores"]) <= tol)
        check_request_output(lay, q, r, sel[r], nsel[r], out[r], ref, f"{name} per-head r{r}",
                             per_q_head=True)


def test_topk_empty_request(gpu_lib):
    L = quest.make_layout(8, 1, 128, 16, torch.bfloat16, 1, 10)
    scores = torch.randn((2, 1, 10), device=DEV)
    ctx = torch.tensor([0, 5], dtype=torch.int32, device=DEV)
    bud = torch.tensor([64, 64], dtype=torch.int32, device=DEV)
    sel = torch.full((2, 1, 4), 9, dtype=torch.int32, device=DEV)
    nsel = torch.full((2, 1), 9, dtype=torch.int32, device=DEV)
    quest.quest_topk_pages(L, scores, ctx, bud, 4, sel, nsel)
    torch.cuda.synchronize()
    assert nsel.cpu().tolist() == [[0], [1]]
    assert sel[0].cpu().tolist() == [[-1, -1, -1, -1]]
    assert sel[1].cpu().tolist() == [[0, -1, -1, -1]]


def test_deterministic_and_budget_covering_all_is_dense(gpu_lib):
    w = scaled(WORKLOADS["layer32k"], batch=2, ctx=1000, budget_tokens=10 ** 6, steps=1)
    lay = Layer(w, DEV)
    q, k_new, v_new = lay.step_inputs(0)
    lay.append_step(k_new, v_new)
    n = -(-1001 // 16)
    outs = []
    for _ in range(2):
        bufs = lay.buffers(max_k=n)
        lay.view(q, bufs)
        lay.attend(q, bufs)
        torch.cuda.synchronize()
        assert torch.equal(bufs.num_sel.cpu(), torch.full((2, 4), n, dtype=torch.int32))
        outs.append(bufs.out.clone())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    sm = workloads.default_sm_scale(w)
    for r in range(2):
        dense = oracle.request_dense(lay.shape, np.ascontiguousarray(to_oracle(q[r])),
                                     lay.host[0], lay.host[1], lay.pt_host[r], 1001, sm)
        check_out(to_f64(outs[0][r]), dense, torch.bfloat16, "dense")


@pytest.mark.parametrize("budget,max_ks", [(1024, (64, 200, 501)), (8000, (501, 520, 1100))])
def test_split_count_invariance(budget, max_ks, gpu_lib):
    """Changing max_k changes the split plan (2, 7, 16, 17 and 18 splits per
    row, so the merge's round trips hold 8, 16 or 32 splits, with and without
    empty ones): the selections stay the same and every plan's outputs meet
    the oracle."""
    w = scaled(WORKLOADS["layer32k"], batch=2, ctx=8000, budget_tokens=budget, steps=1)
    lay = Layer(w, DEV)
    q, k_new, v_new = lay.step_inputs(0)
    lay.append_step(k_new, v_new)
    refs = [lay.oracle_request(q, r) for r in range(w.batch)]
    k = budget // w.page_size
    results = []
    for max_k in max_ks:
        bufs = lay.buffers(max_k=max_k)
        plan = quest.quest_sparse_decode_plan(lay.L, w.batch, max_k)
        log(f"split invariance: budget {budget}, max_k {max_k}, plan {plan}")
        lay.view(q, bufs)
        lay.attend(q, bufs)
        torch.cuda.synchronize()
        sel, nsel, out = bufs.sel_pages.cpu().numpy(), bufs.num_sel.cpu().numpy(), to_f64(bufs.out)
        assert (nsel == k).all()
        for r in range(w.batch):
            check_request_output(lay, q, r, sel[r], nsel[r], out[r], refs[r],
                                 f"split invariance max_k {max_k} r{r}")
        results.append((plan, out, bufs.sel_pages[:, :, :k].cpu()))
    assert len({p["num_splits"] for p, _, _ in results}) == len(max_ks)
    for _, out, sel in results[1:]:
        assert torch.equal(sel, results[0][2])
        check_out(out, results[0][1], torch.bfloat16, "split invariance")


def test_full_bench_shape_sampled(gpu_lib):
    """The benchmark's own shape (batch 8 x 128000, budget 4096), requests 0
    and 7 checked against the oracle in full after each of two decode steps:
    step 0 through the four separate calls (append, scores, top-k, decode),
    step 1 through exactly the sequence bench.py times (quest_append_score,
    then quest_topk_sparse_decode: one fused top-k + decode launch of 8
    splits per row and the merge)."""
    w = scaled(WORKLOADS["bench128k"], steps=2)
    log("full-size benchmark shape: building the cache")
    lay = Layer(w, DEV, host_requests=[0, 7])
    log("cache built")
    for step in range(w.steps):
        q, k_new, v_new = lay.step_inputs(step)
        bufs = lay.buffers(extra=1)
        if step == 0:
            lay.append_step(k_new, v_new)
            lay.view(q, bufs)
            lay.attend(q, bufs)
        else:
            lay.append_score_step(q, k_new, v_new, bufs, topk=False)
            lay.select_attend(q, bufs)
            plan = quest.quest_topk_sparse_decode_plan(lay.L, w.batch, bufs.max_k)
            assert plan == {"fused": True, "num_splits": 8, "pages_per_split": 32}, plan
        torch.cuda.synchronize()
        km = to_f64(lay.kmeta)
        scores = bufs.scores.cpu().numpy().astype(np.float64)
        sel, nsel = bufs.sel_pages.cpu().numpy(), bufs.num_sel.cpu().numpy()
        out = to_f64(bufs.out)
        qh = to_f64(q)
        for r in (0, 7):
            log(f"step {step}: oracle request {r}")
            ref = lay.oracle_request(q, r)
            check_kmeta(lay, r, ref["bounds"], km)
            check_scores(scores[r], ref["scores"], qh[r], ref["bounds"], w.group)
            assert ref["k"] == 256
            check_request_output(lay, q, r, sel[r], nsel[r], out[r], ref,
                                 f"bench step {step} r{r}")


def test_live_splits_ignore_stale_partials(gpu_lib):
    """The decode writes partials only for the splits that hold selected
    pages, and the merge reads only those: with the workspace filled with NaN,
    or holding a larger previous call's partials, a call with few (and no)
    selected pages per row still matches the oracle's attention over its
    selection; a request with no token outputs zeros."""
    w = workloads.Workload("live_splits", 5, 32, 4, 128, 32, "bf16",
                           ctx_list=(0, 40, 700, 2000, 3100), budget_tokens=4000, steps=1,
                           seed=97, permute_pages=True, poison=float("nan"))
    lay = Layer(w, DEV)
    q, _, _ = lay.step_inputs(0)
    max_k = 125
    plan = quest.quest_sparse_decode_plan(lay.L, w.batch, max_k)
    assert plan["num_splits"] > 4, plan
    bufs = lay.buffers(max_k=max_k)
    quest.quest_page_scores(lay.L, q, lay.kmeta, lay.pt, lay.ctx, bufs.scores)
    sm = workloads.default_sm_scale(w)
    outs = []
    for budget, fill in ((4000, None), (64, None), (32, float("nan")), (1000, float("nan"))):
        bud = torch.full((w.batch,), budget, dtype=torch.int32, device=DEV)
        quest.quest_topk_pages(lay.L, bufs.scores, lay.ctx, bud, max_k, bufs.sel_pages,
                               bufs.num_sel)
        if fill is not None:
            bufs.workspace.fill_(fill)
        lay.attend(q, bufs)
        torch.cuda.synchronize()
        out = to_f64(bufs.out)
        sel, nsel = bufs.sel_pages.cpu().numpy(), bufs.num_sel.cpu().numpy()
        assert np.isfinite(out).all(), budget
        assert np.all(out[0] == 0.0) and np.all(nsel[0] == 0)
        for r in range(1, w.batch):
            gpu_sel = [np.asarray(sel[r, g, :nsel[r, g]], np.int32) for g in range(w.num_kv_heads)]
            want = oracle.request_attend(lay.shape, np.ascontiguousarray(to_oracle(q[r])),
                                         lay.host[0], lay.host[1], lay.pt_host[r],
                                         int(lay.ctx[r]), gpu_sel, sm)
            check_out(out[r], want, torch.bfloat16, f"live splits budget {budget} r{r}")
        outs.append(out)
    log(f"live splits: plan {plan}")


@pytest.mark.parametrize("P,D", [(8, 128), (16, 128), (32, 64), (64, 128)])
def test_append_ties_and_signed_zeros(P, D, gpu_lib):
    """Keys drawn from {-0, +0, -1, +1}: every channel of a page is full of
    ties, both zeros among them.  Stored four ways (one bulk append, chunks
    of 5 tokens that start and end inside pages, one token per call, and the
    scalar path from a source one element off 16-byte alignment), the
    metadata equals the oracle's from-scratch bounds bit for bit, the sign
    of zero included (a scan in position order with strict comparisons keeps
    the first-seen of equal values), and the pools equal the oracle's store."""
    Hq, Hkv, B = 8, 2, 3
    lens = [3 * P + 5, 2 * P, 7]
    gen = torch.Generator().manual_seed(4400 + P + D)
    n_pages = [-(-n // P) for n in lens]
    max_pages = max(n_pages) + 1
    pool = sum(n_pages) + 3
    ids = torch.randperm(pool, generator=gen).to(torch.int32)
    pt = torch.zeros((B, max_pages), dtype=torch.int32)
    o = 0
    for r in range(B):
        pt[r, :n_pages[r]] = ids[o:o + n_pages[r]]
        o += n_pages[r]
    N = sum(lens)
    vals = torch.tensor([-0.0, 0.0, -1.0, 1.0])
    k_new = vals[torch.randint(0, 4, (N, Hkv, D), generator=gen)].to(torch.bfloat16)
    v_new = torch.randn((N, Hkv, D), generator=gen).to(torch.bfloat16)
    cuh = [0] + np.cumsum(lens).tolist()
    L = quest.make_layout(Hq, Hkv, D, P, torch.bfloat16, pool, max_pages)
    shape = oracle.Shape(Hq, Hkv, D, P, pool, oracle.BF16)
    kh = np.zeros((pool, Hkv, P, D), np.uint16)
    vh = np.zeros((pool, Hkv, D, P), np.uint16)
    pt_h = pt.numpy()
    for r in range(B):
        oracle.store_tokens(shape, np.ascontiguousarray(to_oracle(k_new[cuh[r]:cuh[r + 1]])),
                            np.ascontiguousarray(to_oracle(v_new[cuh[r]:cuh[r + 1]])), 0,
                            pt_h[r], kh, vh)
    want = [oracle.request_bounds(shape, kh, pt_h[r], lens[r]) for r in range(B)]
    assert any(np.any((w == 0) & np.signbit(w)) for w in want)    # -0 kept somewhere
    assert any(np.any((w == 0) & ~np.signbit(w)) for w in want)   # and +0
    pt_d, kn, vn = pt.to(DEV), k_new.to(DEV), v_new.to(DEV)

    def fresh():
        return (torch.zeros((pool, Hkv, P, D), dtype=torch.bfloat16, device=DEV),
                torch.zeros((pool, Hkv, D, P), dtype=torch.bfloat16, device=DEV),
                torch.full((pool, Hkv, 2, D), 5.0, dtype=torch.bfloat16, device=DEV))

    def in_chunks(step, src_k=kn, src_v=vn):
        k_c, v_c, km = fresh()
        for t0 in range(0, max(lens), step):
            counts = [max(0, min(step, n - t0)) for n in lens]
            rows = [cuh[r] + t0 + i for r in range(B) for i in range(counts[r])]
            sub_cu = torch.tensor([0] + np.cumsum(counts).tolist(), dtype=torch.int32, device=DEV)
            ctx0 = torch.tensor([min(t0, n) for n in lens], dtype=torch.int32, device=DEV)
            idx = torch.tensor(rows, dtype=torch.int64, device=DEV)
            quest.quest_append_kv(L, src_k[idx].contiguous(), src_v[idx].contiguous(), sub_cu,
                                  ctx0, step, pt_d, k_c, v_c, km)
        return k_c, v_c, km

    ways = {"bulk": in_chunks(max(lens)), "chunks5": in_chunks(5), "tokens": in_chunks(1)}
    k_buf = torch.empty(kn.numel() + 1, dtype=kn.dtype, device=DEV)
    v_buf = torch.empty(vn.numel() + 1, dtype=vn.dtype, device=DEV)
    k_off, v_off = k_buf[1:].view(kn.shape), v_buf[1:].view(vn.shape)
    k_off.copy_(kn)
    v_off.copy_(vn)
    assert k_off.data_ptr() % 16 != 0
    k_c, v_c, km = fresh()
    quest.quest_append_kv(L, k_off, v_off, torch.tensor(cuh, dtype=torch.int32, device=DEV),
                          torch.zeros(B, dtype=torch.int32, device=DEV), max(lens), pt_d, k_c,
                          v_c, km)
    ways["scalar"] = (k_c, v_c, km)
    torch.cuda.synchronize()
    for name, (k_c, v_c, km) in ways.items():
        assert to_oracle(k_c).tobytes() == kh.tobytes(), name
        assert to_oracle(v_c).tobytes() == vh.tobytes(), name
        kmh = to_f64(km)
        for r in range(B):
            got = kmh[pt_h[r, :n_pages[r]]]
            assert np.array_equal(got, want[r]), (name, r)
            assert np.array_equal(np.signbit(got), np.signbit(want[r])), (name, r)


@pytest.mark.parametrize("dtype,D,P", [(torch.bfloat16, 128, 16), (torch.bfloat16, 64, 32),
                                       (torch.float32, 64, 16)])
def test_append_score_several_tokens(dtype, D, P, gpu_lib):
    """quest_append_score storing several new tokens per request in one call
    (0, 1, 5, 17 and 40; first positions inside pages, at a page start, and
    just before the first page of the next scoring work-group's range: 1024
    tokens at page 16 for the matrix-core kernel's 64-page groups, 4096 for
    the fp32 kernel's 256-page groups): pools equal the oracle's store byte
    for byte, every live page's metadata equals the oracle's from-scratch
    bounds, and the scores meet the oracle's within the fp32 summation
    bound."""
    Hq, Hkv = 8, 2
    G = Hq // Hkv
    span = (64 if dtype == torch.bfloat16 else 256) * P     # tokens per scoring work-group
    before = [span - 3, 7, P, span - 10, 2 * P + 1, 0]
    new = [5, 17, 40, 40, 0, 1]
    B = len(before)
    gen = torch.Generator().manual_seed(4500 + D + P)
    n_pages = [-(-(b + n) // P) for b, n in zip(before, new)]
    max_pages = max(n_pages) + 2
    pool = sum(n_pages) + 5
    ids = torch.randperm(pool, generator=gen).to(torch.int32)
    pt = torch.zeros((B, max_pages), dtype=torch.int32)
    o = 0
    for r in range(B):
        pt[r, :n_pages[r]] = ids[o:o + n_pages[r]]
        o += n_pages[r]
    elem = oracle.BF16 if dtype == torch.bfloat16 else oracle.F32
    shape = oracle.Shape(Hq, Hkv, D, P, pool, elem)
    L = quest.make_layout(Hq, Hkv, D, P, dtype, pool, max_pages)
    pt_h = pt.numpy()
    # prompts (bulk append) and the new tokens (one quest_append_score call)
    k0 = torch.randn((sum(before), Hkv, D), generator=gen).to(dtype)
    v0 = torch.randn((sum(before), Hkv, D), generator=gen).to(dtype)
    k1 = torch.randn((sum(new), Hkv, D), generator=gen).to(dtype)
    v1 = torch.randn((sum(new), Hkv, D), generator=gen).to(dtype)
    q = torch.randn((B, Hq, D), generator=gen).to(dtype)
    cu0 = [0] + np.cumsum(before).tolist()
    cu1 = [0] + np.cumsum(new).tolist()
    kh = np.zeros((pool, Hkv, P, D), shape.storage_dtype())
    vh = np.zeros((pool, Hkv, D, P), shape.storage_dtype())
    for r in range(B):
        if before[r]:
            oracle.store_tokens(shape, np.ascontiguousarray(to_oracle(k0[cu0[r]:cu0[r + 1]])),
                                np.ascontiguousarray(to_oracle(v0[cu0[r]:cu0[r + 1]])), 0,
                                pt_h[r], kh, vh)
        if new[r]:
            oracle.store_tokens(shape, np.ascontiguousarray(to_oracle(k1[cu1[r]:cu1[r + 1]])),
                                np.ascontiguousarray(to_oracle(v1[cu1[r]:cu1[r + 1]])),
                                before[r], pt_h[r], kh, vh)
    k_c = torch.zeros((pool, Hkv, P, D), dtype=dtype, device=DEV)
    v_c = torch.zeros((pool, Hkv, D, P), dtype=dtype, device=DEV)
    km = torch.full((pool, Hkv, 2, D), 3.0, dtype=dtype, device=DEV)
    pt_d = pt.to(DEV)
    zeros = torch.zeros(B, dtype=torch.int32, device=DEV)
    quest.quest_append_kv(L, k0.to(DEV), v0.to(DEV), torch.tensor(cu0, dtype=torch.int32,
                          device=DEV), zeros, max(before), pt_d, k_c, v_c, km)
    scores = torch.full((B, Hkv, max_pages), 7.0, dtype=torch.float32, device=DEV)
    quest.quest_append_score(L, q.to(DEV), k1.to(DEV), v1.to(DEV),
                             torch.tensor(cu1, dtype=torch.int32, device=DEV),
                             torch.tensor(before, dtype=torch.int32, device=DEV), max(new), pt_d,
                             k_c, v_c, km, scores)
    torch.cuda.synchronize()
    assert to_oracle(k_c).tobytes() == kh.tobytes()
    assert to_oracle(v_c).tobytes() == vh.tobytes()
    kmh, sc = to_f64(km), scores.cpu().numpy().astype(np.float64)
    qh = to_oracle(q)
    for r in range(B):
        ctx = before[r] + new[r]
        if ctx == 0:
            continue
        bounds = oracle.request_bounds(shape, kh, pt_h[r], ctx)
        got = kmh[pt_h[r, :n_pages[r]]]
        assert np.array_equal(got, bounds), r
        ref = oracle.request_scores(shape, np.ascontiguousarray(qh[r]), bounds)
        check_scores(sc[r], ref, to_f64(q[r]), bounds, G)
