"""GPU parity at the full sizes of the one-layer 32k, ragged and 48-layer workloads, checked
on sampled requests against the oracle (the benchmark shape itself is
covered by test_full_bench_shape_sampled), dense decode over every page at
the benchmark shape, plus hipGraph capture/replay of a decode step."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from helpers import to_f64, to_oracle
from kv_cache_decode_quest_amd import quest, workloads
from kv_cache_decode_quest_amd.workloads import WORKLOADS, scaled
from parity import (Layer, check_kmeta, check_out, check_request_output, check_scores,
                    log)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def check_requests(lay, q, bufs, requests):
    torch.cuda.synchronize()
    km = to_f64(lay.kmeta)
    scores = bufs.scores.cpu().numpy().astype(np.float64)
    sel, nsel = bufs.sel_pages.cpu().numpy(), bufs.num_sel.cpu().numpy()
    out = to_f64(bufs.out)
    qh = to_f64(q)
    flagged = 0
    for r in requests:
        ref = lay.oracle_request(q, r)
        check_kmeta(lay, r, ref["bounds"], km)
        check_scores(scores[r], ref["scores"], qh[r], ref["bounds"], lay.w.group)
        flagged += check_request_output(lay, q, r, sel[r], nsel[r], out[r], ref,
                                        f"{lay.w.name} r{r}")
    return flagged


def test_full_layer32k_sampled(gpu_lib):
    """The one-layer Qwen3-30B-A3B-like configuration at full size: batch 8 x
    32768 tokens, budget 2048, one decode step through the fused append +
    scores path; requests 0, 3 and 7 against the oracle."""
    w = WORKLOADS["layer32k"]
    sample = [0, 3, 7]
    lay = Layer(w, DEV, host_requests=sample)
    q, k_new, v_new = lay.step_inputs(0)
    bufs = lay.buffers(extra=1)
    lay.append_score_step(q, k_new, v_new, bufs)
    lay.attend(q, bufs)
    flagged = check_requests(lay, q, bufs, sample)
    log(f"layer32k: ok, flagged {flagged}")


def test_full_ragged_sampled(gpu_lib):
    """32 requests, contexts uniform in [4096, 131072], page 32, budget 10% of
    pages, physical pages permuted in one pool, unwritten slots poisoned: one
    decode step, the shortest, the longest and two more requests checked."""
    w = WORKLOADS["ragged"]
    ctx = workloads.context_lengths(w)
    sample = sorted({int(ctx.argmin()), int(ctx.argmax()), 5, 17})
    log(f"ragged: contexts {int(ctx.min())}..{int(ctx.max())}, sampled requests {sample}")
    lay = Layer(w, DEV, host_requests=sample)
    q, k_new, v_new = lay.step_inputs(0)
    bufs = lay.buffers(extra=1)
    lay.append_score_step(q, k_new, v_new, bufs)
    lay.attend(q, bufs)
    flagged = check_requests(lay, q, bufs, sample)
    log(f"ragged: ok, flagged {flagged}")


def test_full_layers48_sampled(gpu_lib):
    """The full 48-layer decode step (batch 64 x 32768, budget 2048, K outlier
    channels x10), all 48 layers resident (about 219 GB), every layer through
    the sequence bench.py times (quest_append_score, then
    quest_topk_sparse_decode: 256 selection rows, one fused work-group per
    row attending its 128 pages in four rounds and writing the output with
    no merge); layers 0, 23 and 47 checked on requests 0 and 63."""
    w = WORKLOADS["layers48"]
    sampled_layers, sample = (0, 23, 47), [0, 63]
    layers, results = [], {}
    for li in range(w.layers):
        lay = Layer(w, DEV, layer=li, host=li in sampled_layers, host_requests=sample)
        layers.append(lay)
        torch.cuda.empty_cache()     # hand the prompt temporaries back before the next layer
        if li % 8 == 0:
            log(f"layers48: layer {li} cache built, "
                f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")
    log("layers48: decode step over all layers")
    for li, lay in enumerate(layers):
        q, k_new, v_new = lay.step_inputs(0)
        bufs = lay.buffers(extra=1)
        if li == 0:
            plan = quest.quest_topk_sparse_decode_plan(lay.L, w.batch, bufs.max_k)
            assert plan == {"fused": True, "num_splits": 1, "pages_per_split": 128}, plan
        lay.append_score_step(q, k_new, v_new, bufs, topk=False)
        lay.select_attend(q, bufs)
        if li in sampled_layers:
            results[li] = (q, bufs)
    torch.cuda.synchronize()
    for li in sampled_layers:
        q, bufs = results[li]
        flagged = check_requests(layers[li], q, bufs, sample)
        log(f"layers48: layer {li} ok, flagged {flagged}")


def test_full_dense_sampled(gpu_lib):
    """Dense flash-decode on the same pool (the vanilla method): every page of
    every request selected, no scoring and no top-k, at the benchmark's shape
    (batch 8 x 128000 + one appended token); requests 0 and 5 against the
    oracle's dense attention over all their tokens."""
    w = WORKLOADS["bench128k"]
    sample = [0, 5]
    lay = Layer(w, DEV, host_requests=sample)
    q, k_new, v_new = lay.step_inputs(0)
    lay.append_step(k_new, v_new)
    B, H = w.batch, w.num_kv_heads
    max_k = lay.lay.max_pages
    bufs = quest.alloc_decode_buffers(lay.L, B, max_k, DEV)
    bufs.sel_pages.copy_(torch.arange(max_k, dtype=torch.int32, device=DEV).expand(B, H, max_k))
    n = (lay.ctx.to(torch.int64) + w.page_size - 1) // w.page_size
    nsel = n.to(torch.int32).view(B, 1).expand(B, H).contiguous().to(DEV)
    lay.attend(q, bufs, sel=bufs.sel_pages, nsel=nsel)
    torch.cuda.synchronize()
    out = to_f64(bufs.out)
    sm = workloads.default_sm_scale(w)
    for r in sample:
        log(f"dense: oracle request {r} over {int(lay.ctx[r])} tokens")
        qr = np.ascontiguousarray(to_oracle(q[r]))
        ref = oracle.request_dense(lay.shape, qr, lay.host[0], lay.host[1], lay.pt_host[r],
                                   int(lay.ctx[r]), sm)
        check_out(out[r], ref, w.torch_dtype, f"dense r{r}")
    log("dense: ok")


def test_graph_capture_replay(gpu_lib):
    """A decode step (fused append + scores, top-k, decode) captured once in a
    hipGraph and replayed on new inputs matches the same steps run eagerly on
    an identical cache, bit for bit, with eager work between replays."""
    w = scaled(WORKLOADS["layer32k"], batch=4, ctx=3000, budget_tokens=512, steps=4)
    eager = Layer(w, DEV, host=False)
    graphed = Layer(w, DEV, host=False)
    max_k = 32
    bufs_e = eager.buffers(max_k=max_k)
    bufs_g = graphed.buffers(max_k=max_k)
    q_s, k_s, v_s = (x.clone() for x in graphed.step_inputs(0))
    cu = torch.arange(w.batch + 1, dtype=torch.int32, device=DEV)
    ctx_b = graphed.ctx.clone()
    ctx_a = ctx_b + 1
    budget = torch.full_like(ctx_b, 512)
    sm = workloads.default_sm_scale(w)

    def step(q, k, v, cb, ca, lay, bufs):
        quest.decode_step(lay.L, q, k, v, cu, cb, ca, budget, lay.pt, lay.k_cache, lay.v_cache,
                          lay.kmeta, bufs, sm)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up outside the capture
        tmp = Layer(w, DEV, host=False)
        step(q_s, k_s, v_s, ctx_b, ctx_a, tmp, tmp.buffers(max_k=max_k))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del tmp
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(q_s, k_s, v_s, ctx_b, ctx_a, graphed, bufs_g)
    for s in range(w.steps):
        q, k, v = eager.step_inputs(s)
        cb = eager.ctx.clone()
        step(q, k, v, cb, cb + 1, eager, bufs_e)
        eager.ctx = cb + 1
        q_s.copy_(q)
        k_s.copy_(k)
        v_s.copy_(v)
        ctx_b.copy_(cb)
        ctx_a.copy_(cb + 1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs_g.sel_pages, bufs_e.sel_pages), s
        assert torch.equal(bufs_g.out.view(torch.int16), bufs_e.out.view(torch.int16)), s
        assert torch.equal(graphed.kmeta.view(torch.int16), eager.kmeta.view(torch.int16)), s
        _ = (bufs_e.out.float() * 2).sum().item()   # eager work between replays
