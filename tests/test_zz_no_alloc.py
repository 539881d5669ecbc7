"""GPU test of quest_decode_step_noalloc, the decode step that allocates
nothing (its split partials live in the library's static device scratch):
two calls in a row, the second with a smaller input, each against
quest_decode_step with a caller workspace on an identical cache.  Both run
the same kernels on the same inputs, so everything must agree bit for bit;
the outputs also meet the oracle at the usual tolerance."""
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


def one_step(w, step=0):
    """One decode step of workload w through both entry points; returns the
    noalloc call's buffers after checking them."""
    ref = Layer(w, DEV)
    nal = Layer(w, DEV, host=False)
    sm = workloads.default_sm_scale(w)
    q, k_new, v_new = ref.step_inputs(step)
    cu = torch.arange(w.batch + 1, dtype=torch.int32, device=DEV)
    ctx_b = ref.ctx.clone()
    ctx_a = ctx_b + 1
    budgets = workloads.budget_tokens(w, ctx_a).to(DEV)
    max_k = max(1, int((budgets // w.page_size).max()))
    need = quest.quest_sparse_decode_workspace_bytes(ref.L, w.batch, max_k)
    assert 0 < need <= quest.STATIC_SCRATCH_BYTES
    br = quest.alloc_decode_buffers(ref.L, w.batch, max_k, DEV)
    bn = quest.alloc_decode_buffers(nal.L, w.batch, max_k, DEV)
    bn.out.fill_(7.0)
    bn.sel_pages.fill_(-7)
    quest.quest_decode_step(ref.L, q, k_new, v_new, cu, ctx_b, 1, ref.pt, ref.k_cache,
                            ref.v_cache, ref.kmeta, ctx_a, budgets, max_k, sm, br.scores,
                            br.sel_pages, br.num_sel, br.out, br.workspace)
    quest.quest_decode_step_noalloc(nal.L, q, k_new, v_new, cu, ctx_b, 1, nal.pt, nal.k_cache,
                                    nal.v_cache, nal.kmeta, ctx_a, budgets, max_k, sm, bn.scores,
                                    bn.sel_pages, bn.num_sel, bn.out)
    torch.cuda.synchronize()
    plan = quest.quest_topk_sparse_decode_plan(ref.L, w.batch, max_k)
    log(f"noalloc {w.name}: max_k {max_k}, plan {plan}, partials {need} bytes")
    assert torch.equal(bn.num_sel, br.num_sel)
    assert torch.equal(bn.sel_pages, br.sel_pages)
    assert torch.equal(bn.out.view(torch.int16), br.out.view(torch.int16))
    assert torch.equal(nal.kmeta.view(torch.int16), ref.kmeta.view(torch.int16))
    assert torch.equal(nal.k_cache.view(torch.int16), ref.k_cache.view(torch.int16))
    assert torch.equal(nal.v_cache.view(torch.int16), ref.v_cache.view(torch.int16))
    for r in range(w.batch):
        n = (int(ctx_a[r]) + w.page_size - 1) // w.page_size
        assert torch.equal(bn.scores[r, :, :n].view(torch.int32),
                           br.scores[r, :, :n].view(torch.int32)), r
    ref.host_append(k_new, v_new)      # the oracle's copy of the appended token
    assert torch.equal(ref.ctx, ctx_a)
    out = to_f64(bn.out)
    sel, nsel = bn.sel_pages.cpu().numpy(), bn.num_sel.cpu().numpy()
    for r in range(w.batch):
        oref = ref.oracle_request(q, r)
        check_request_output(ref, q, r, sel[r], nsel[r], out[r], oref, f"noalloc {w.name} r{r}")
    return plan


def test_noalloc_step_equals_workspace_step(gpu_lib):
    # first call: 32 selection rows of 8 fused splits (partials merged from
    # the scratch); second, smaller: 6 ragged requests at page 32 (the top-k
    # and decode kernels, two splits per row, merged from the scratch)
    big = scaled(WORKLOADS["bench128k"], batch=8, ctx=9000, budget_tokens=4096, steps=1)
    small = scaled(WORKLOADS["ragged"], batch=6, ctx_range=(400, 6000), steps=1)
    p1 = one_step(big)
    assert p1["fused"] and p1["num_splits"] == 8
    p2 = one_step(small)
    assert not p2["fused"] and p2["num_splits"] > 1
