"""GPU parity of quest_decode_step, the whole decode step of one layer in one
ABI call.

Two identical caches step side by side: one through quest_append_score +
quest_topk_sparse_decode (each held to the oracle elsewhere), one through
quest_decode_step.  Scores, metadata, caches, selections and outputs must be
equal bit for bit after every step, and the outputs must meet the oracle at
the usual tolerance.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from helpers import to_f64
from kv_cache_decode_quest_amd import quest, workloads
from kv_cache_decode_quest_amd.workloads import WORKLOADS, scaled
from parity import Layer, check_request_output, log

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

W = workloads.Workload
CASES = {
    # 8-token pages (two kernels for the top-k and decode)
    "p8": W("p8", 3, 32, 4, 128, 8, "bf16", ctx_range=(100, 3000), budget_tokens=512, steps=2,
            seed=305),
    # 8 requests x 4 KV heads = 32 rows, 8 splits of 32 pages
    "rows32": scaled(WORKLOADS["bench128k"], batch=8, ctx=9000, budget_tokens=4096, steps=3),
    # 12 rows, ragged lengths, permuted pages
    "rows12_ragged": W("rows12_ragged", 3, 32, 4, 128, 16, "bf16", ctx_range=(300, 7000),
                       budget_tokens=1024, steps=3, permute_pages=True, poison=float("nan"),
                       seed=301),
    # 2 rows, G 16 (no column packing)
    "rows2_g16": W("rows2_g16", 1, 32, 2, 128, 16, "bf16", ctx=5000, budget_tokens=2048,
                   steps=2, seed=302),
    # 256 rows: one split per row, the output written without a merge
    "rows256": W("rows256", 64, 32, 4, 128, 16, "bf16", ctx_range=(1, 1500),
                 budget_tokens=320, steps=2, poison=float("nan"), seed=303),
    # a request with no token, short requests, a budget past the context
    "edges": W("edges", 5, 16, 2, 128, 16, "bf16", ctx_list=(0, 1, 16, 17, 2500),
               budget_tokens=256, steps=2, seed=304),
}


def run_case(w, reduce="max", n_sink=0, n_recent=0, check_oracle=True):
    two = Layer(w, DEV, host=check_oracle)
    one = Layer(w, DEV, host=False)
    sm = workloads.default_sm_scale(w)
    max_k = two.max_k()
    max_k = max(max_k, int((workloads.budget_tokens(w, two.ctx + w.steps).max()) // w.page_size))
    bt = two.buffers(max_k)
    bo = one.buffers(max_k)
    cu = torch.arange(w.batch + 1, dtype=torch.int32, device=DEV)
    for step in range(w.steps):
        q, k_new, v_new = two.step_inputs(step)
        ctx_b = two.ctx.clone()
        two.append_score_step(q, k_new, v_new, bt, reduce=reduce, topk=False)
        budgets = two.budgets()
        quest.quest_topk_sparse_decode(two.L, q, two.k_cache, two.v_cache, two.pt, two.ctx,
                                       bt.scores, budgets, max_k, sm, bt.sel_pages, bt.num_sel,
                                       bt.out, bt.workspace, n_sink, n_recent)
        bo.sel_pages.fill_(-7)
        bo.out.fill_(7.0)
        quest.quest_decode_step(one.L, q, k_new, v_new, cu, ctx_b, 1, one.pt, one.k_cache,
                                one.v_cache, one.kmeta, ctx_b + 1, budgets, max_k, sm,
                                bo.scores, bo.sel_pages, bo.num_sel, bo.out, bo.workspace,
                                reduce, n_sink, n_recent)
        one.ctx = ctx_b + 1
        torch.cuda.synchronize()
        log(f"{w.name} step {step}: max_k {max_k}, reduce {reduce}")
        assert torch.equal(one.kmeta.view(torch.int16), two.kmeta.view(torch.int16)), step
        assert torch.equal(one.k_cache.view(torch.int16), two.k_cache.view(torch.int16)), step
        assert torch.equal(one.v_cache.view(torch.int16), two.v_cache.view(torch.int16)), step
        for r in range(w.batch):
            nr = (int(one.ctx[r]) + w.page_size - 1) // w.page_size
            assert torch.equal(bo.scores[r, :, :nr].view(torch.int32),
                               bt.scores[r, :, :nr].view(torch.int32)), (step, r)
        assert torch.equal(bo.num_sel, bt.num_sel), step
        assert torch.equal(bo.sel_pages, bt.sel_pages), step
        assert torch.equal(bo.out.view(torch.int16), bt.out.view(torch.int16)), step
    if check_oracle:
        out = to_f64(bo.out)
        sel, nsel = bo.sel_pages.cpu().numpy(), bo.num_sel.cpu().numpy()
        for r in range(w.batch):
            ref = two.oracle_request(q, r, reduce=reduce, n_sink=n_sink, n_recent=n_recent)
            check_request_output(two, q, r, sel[r], nsel[r], out[r], ref, f"{w.name} step r{r}")
            if int(one.ctx[r]) == 0:
                assert np.all(out[r] == 0.0)


@pytest.mark.parametrize("name", list(CASES))
def test_decode_step_equals_two_calls(gpu_lib, name):
    w = CASES[name]
    run_case(w)


def test_decode_step_sum_and_forced(gpu_lib):
    w = CASES["rows12_ragged"]
    run_case(w, reduce="sum", check_oracle=True)
    run_case(w, n_sink=1, n_recent=2)
