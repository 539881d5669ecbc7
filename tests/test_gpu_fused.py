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
from helpers import to_f64, to_oracle
from kv_cache_decode_quest_amd import quest, workloads
from kv_cache_decode_quest_amd.workloads import WORKLOADS, scaled
from parity import Layer, check_out, compare_selection, log
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

CASES = {name: w for name, w in SMALL.items() if w.dtype == "bf16"}
CASES["bench128k_b4"] = scaled(WORKLOADS["bench128k"], batch=4, ctx=20000,
                               budget_tokens=2048, steps=1)


def expect_fused(w, L, max_k):
    """The documented rule: bf16, rows of at most 8192 pages, D 64 or (D 128,
    P 16), at most 256 pages per split and 256 work-groups."""
    plan = quest.quest_sparse_decode_plan(L, w.batch, max_k)
    rows = w.batch * quest.selection_rows(L)
    return (w.dtype == "bf16" and L.max_pages_per_seq <= 8192
            and (w.head_dim == 64 or (w.head_dim == 128 and w.page_size == 16))
            and plan["pages_per_split"] <= 256 and rows * plan["num_splits"] <= 256)


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
        log(f"{w.name} step {step}: fused kernel {fused}, max_k {bufs.max_k}")
        assert torch.equal(fb.num_sel, bufs.num_sel)
        assert torch.equal(fb.sel_pages, bufs.sel_pages)
        two, one = to_f64(bufs.out), to_f64(fb.out)
        if not fused:
            assert torch.equal(fb.out.view(torch.int16), bufs.out.view(torch.int16))
        else:
            assert np.all(one_bf16_ulp(one, two)), float(np.abs(one - two).max())
        if n_sink or n_recent:
            continue
        sel, nsel = bufs.sel_pages.cpu().numpy(), bufs.num_sel.cpu().numpy()
        for r in range(w.batch):
            ref = lay.oracle_request(q, r, per_q_head=per_q_head)
            rows = len(ref["sel"])
            flags = [compare_selection(sel[r, x], int(nsel[r, x]), ref["sel"][x],
                                       ref["scores"][x]) for x in range(rows)]
            if "flagged" not in flags:
                check_out(one[r], ref["out"], w.torch_dtype, f"{w.name} fused r{r}")
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
        ref = oracle.decode_request(lay.shape, np.ascontiguousarray(to_oracle(q[r])), lay.host[0],
                                    lay.host[1], lay.pt_host[r], int(lay.ctx[r]),
                                    int(lay.budgets()[r]), workloads.default_sm_scale(w),
                                    n_sink=1, n_recent=2)
        flags = [compare_selection(sel[r, g], int(nsel[r, g]), ref["sel"][g], ref["scores"][g])
                 for g in range(w.num_kv_heads)]
        if "flagged" not in flags:
            check_out(out[r], ref["out"], torch.bfloat16, f"fused forced r{r}")


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
