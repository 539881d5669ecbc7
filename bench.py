"""Quest sparse-decode benchmark on one MI355X.

Workload (default "bench128k"): one Qwen3-30B-A3B-class attention layer
(32 q / 4 KV heads, head_dim 128, bf16), batch 8, 128000-token contexts in a
paged cache (page 16), token budget 4096 (256 pages per KV head).  A step is
the whole hot path for one new token per request: quest_append_score (KV store
and min/max refresh fused with the page scores) and quest_topk_sparse_decode
(the top-k selection and the split-K attention in one kernel at this shape,
then the merge).  Inputs are seeded synthetic tensors already resident in
HBM.

Timing: the layer's cache is resident in several copies (own K/V pools and
metadata per copy, one shared page table, as a model's layers share one block
table), and the K timed steps rotate over the copies, so a step's metadata
and KV were last touched several layers earlier and are read from HBM, not
from the 256 MB Infinity Cache.  The steps run back to back from one
captured HIP graph (decode steps are replayed from graphs in serving), after
W eager warm-up steps, one eager pass over the sequence and one untimed
replay; a HIP event pair brackets the timed replay.  value = batch * K /
replay time.  Also reported: the same steps launched eagerly one at a time,
the cache evicted before each by an untimed 2 GiB read sweep (each step then
pays its own dispatch latency); the same steps replayed on one copy without
eviction (labelled cache-assisted); the bytes each step moves besides the
headline ones, by item; a per-kernel breakdown; the dominant kernel's
roofline (its average over 128 back-to-back launches cycling through 8
copies of the metadata, and the committed counter record of its HBM
traffic); the dense decode over every page, the
per-q-head selection, the SUM / forced-page / page-size variants and the
prefill-chunk append, each timed like the eager steps; the 48-layer batch-64
step; one step each of the other single-layer workloads (the tiny fp32
request, the 32k-context layer, the ragged batch), each on a cache of its
own and timed like the eager steps; and the CPU oracle on a bounded sample
of the same workload (all host threads and one), its from-scratch metadata
build, and one layer-step of the 48-layer workload.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import platform
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from kv_cache_decode_quest_amd import probe, quest, workloads  # noqa: E402

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
METRIC = "sparse decode tokens/s + achieved HBM GB/s (% peak), batch 8 x 128k ctx"


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


class BenchLayer:
    """The layer's caller-owned buffers (the cache-manager role)."""

    def resident_copy(self):
        """Another layer of the same shape and contents: its own K/V pools and
        metadata, the same page table and context lengths."""
        c = object.__new__(BenchLayer)
        c.__dict__.update(self.__dict__)
        c.k_cache, c.v_cache = self.k_cache.clone(), self.v_cache.clone()
        c.kmeta = self.kmeta.clone()
        c.prefill = None
        return c

    def __init__(self, w: workloads.Workload, capacity: int, device):
        self.w, self.device = w, device
        self.lay = workloads.make_layout(w, device, capacity)
        self.L = quest.make_layout(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                                   w.torch_dtype, self.lay.num_pool_pages, self.lay.max_pages)
        self.k_cache, self.v_cache = workloads.empty_pool(w, self.lay, device)
        self.kmeta = torch.zeros((self.lay.num_pool_pages, w.num_kv_heads, 2, w.head_dim),
                                 dtype=w.torch_dtype, device=device)
        self.pt = self.lay.page_table
        self.ctx0 = self.lay.ctx0.clone()
        k_new, v_new, cu, ctx_before = workloads.prefill_tokens(w, self.lay, device)
        self.prefill = (k_new, v_new, cu)
        quest.quest_append_kv(self.L, k_new, v_new, cu, ctx_before, int(self.ctx0.max()),
                              self.pt, self.k_cache, self.v_cache, self.kmeta)
        self.cu1 = torch.arange(w.batch + 1, dtype=torch.int32, device=device)


def make_steps(w, n, device):
    """Per-step inputs and the context arrays of each step (no host sync in
    the timed loop)."""
    steps = []
    for s in range(n):
        q, k_new, v_new = workloads.step_tokens(w, device, 0, s)
        steps.append((q, k_new, v_new))
    return steps


def run_step(layer, bufs, s, inp, ctx_before, ctx_after, budgets, sm, events=None):
    q, k_new, v_new = inp
    L = layer.L
    if events:
        events[0].record()
    quest.quest_append_score(L, q, k_new, v_new, layer.cu1, ctx_before, 1, layer.pt,
                             layer.k_cache, layer.v_cache, layer.kmeta, bufs.scores)
    if events:
        events[1].record()
    quest.quest_topk_sparse_decode(L, q, layer.k_cache, layer.v_cache, layer.pt, ctx_after,
                                   bufs.scores, budgets, bufs.max_k, sm, bufs.sel_pages,
                                   bufs.num_sel, bufs.out, bufs.workspace)
    if events:
        events[2].record()


def dense_reference(layer, inputs, ctx_b, ctx_a, sm, evict, n_steps, dev):
    """The vanilla decode step on the same pool, timed like the sparse step:
    append one token per request, then the same decode kernel over every page
    of every request (no scoring, no top-k).  Bytes = all valid K/V."""
    w, L = layer.w, layer.L
    B, H = w.batch, w.num_kv_heads
    max_k = layer.lay.max_pages
    bufs = quest.alloc_decode_buffers(L, B, max_k, dev)
    bufs.sel_pages.copy_(torch.arange(max_k, dtype=torch.int32, device=dev).expand(B, H, max_k))
    nsel = [((c.to(torch.int64) + w.page_size - 1) // w.page_size).to(torch.int32)
            .view(B, 1).expand(B, H).contiguous().to(dev) for c in ctx_a[:n_steps]]

    def step(s):
        q, k_new, v_new = inputs[s]
        quest.quest_append_kv(L, k_new, v_new, layer.cu1, ctx_b[s], 1, layer.pt, layer.k_cache,
                              layer.v_cache, layer.kmeta)
        quest.quest_sparse_decode(L, q, layer.k_cache, layer.v_cache, layer.pt, ctx_a[s],
                                  bufs.sel_pages, nsel[s], max_k, sm, bufs.out, bufs.workspace)

    for s in range(min(2, n_steps)):
        step(s)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_steps)]
    torch.cuda.synchronize()
    for s in range(n_steps):
        evict()
        ev[s][0].record()
        step(s)
        ev[s][1].record()
    torch.cuda.synchronize()
    total_s = sum(e[0].elapsed_time(e[1]) for e in ev) / 1e3
    elem = 2 if w.dtype == "bf16" else 4
    kv_bytes = sum(int(c.sum()) for c in ctx_a[:n_steps]) * H * 2 * w.head_dim * elem
    plan = quest.quest_sparse_decode_plan(L, B, max_k)
    return {"what": "the same decode kernel over every page of every request (no scoring, no "
                    "top-k), one token appended per request; cache evicted before each step",
            "tokens_per_s": B * n_steps / total_s, "ms_per_step": total_s / n_steps * 1e3,
            "steps": n_steps, "kv_bytes_per_step": kv_bytes / n_steps,
            "hbm_gbps": kv_bytes / total_s / 1e9,
            "hbm_frac_peak": kv_bytes / total_s / 1e9 / PEAK_HBM_GBPS,
            "plan": plan}


def per_q_head_reference(layer, inputs, ctx_b, ctx_a, budgets, sm, evict, n_steps, dev):
    """The same decode step with per-q-head selection (every q head scores,
    selects and attends its own pages; no sharing across the GQA group),
    timed like the sparse step.  Bytes = metadata + each q head's selected
    valid K/V."""
    w = layer.w
    B, Hq, P = w.batch, w.num_q_heads, w.page_size
    L = quest.make_layout(Hq, w.num_kv_heads, w.head_dim, P, w.torch_dtype,
                          layer.lay.num_pool_pages, layer.lay.max_pages, per_q_head=True)
    max_k = max(1, max(int((b // P).max()) for b in budgets[:n_steps]))
    bufs = quest.alloc_decode_buffers(L, B, max_k, dev)
    sels = torch.empty((n_steps,) + tuple(bufs.sel_pages.shape), dtype=torch.int32, device=dev)
    nsels = torch.empty((n_steps,) + tuple(bufs.num_sel.shape), dtype=torch.int32, device=dev)

    def step(s):
        q, k_new, v_new = inputs[s]
        quest.quest_append_score(L, q, k_new, v_new, layer.cu1, ctx_b[s], 1, layer.pt,
                                 layer.k_cache, layer.v_cache, layer.kmeta, bufs.scores)
        quest.quest_topk_pages(L, bufs.scores, ctx_a[s], budgets[s], max_k, bufs.sel_pages,
                               bufs.num_sel)
        quest.quest_sparse_decode(L, q, layer.k_cache, layer.v_cache, layer.pt, ctx_a[s],
                                  bufs.sel_pages, bufs.num_sel, max_k, sm, bufs.out,
                                  bufs.workspace)

    step(0)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_steps)]
    torch.cuda.synchronize()
    for s in range(n_steps):
        evict()
        ev[s][0].record()
        step(s)
        ev[s][1].record()
        sels[s].copy_(bufs.sel_pages)
        nsels[s].copy_(bufs.num_sel)
    torch.cuda.synchronize()
    total_s = sum(e[0].elapsed_time(e[1]) for e in ev) / 1e3
    meta_b = kv_b = 0
    for s in range(n_steps):
        m, kv = step_bytes(w, ctx_a[s], sels[s], nsels[s])
        meta_b += m
        kv_b += kv
    return {"what": "the same step with every q head scoring, selecting and attending its "
                    "own pages (no sharing across the GQA group); cache evicted before each step",
            "tokens_per_s": B * n_steps / total_s, "ms_per_step": total_s / n_steps * 1e3,
            "steps": n_steps, "selected_kv_bytes_per_step": kv_b / n_steps,
            "hbm_gbps": (meta_b + kv_b) / total_s / 1e9,
            "hbm_frac_peak": (meta_b + kv_b) / total_s / 1e9 / PEAK_HBM_GBPS}


def timed_variant(layer, inputs, ctx_b, ctx_a, budgets, sm, evict, n_steps, dev, reduce="max",
                  n_sink=0, n_recent=0):
    """The step (quest_append_score + quest_topk_sparse_decode) of one
    variant, timed like eager_evicted: one event pair per step, the cache
    evicted before each.  Bytes = metadata + selected valid K/V."""
    w, L = layer.w, layer.L
    B, P = w.batch, w.page_size
    max_k = max(1, max(int((b // P).max()) for b in budgets[:n_steps]))
    bufs = quest.alloc_decode_buffers(L, B, max_k, dev)
    sels = torch.empty((n_steps,) + tuple(bufs.sel_pages.shape), dtype=torch.int32, device=dev)
    nsels = torch.empty((n_steps,) + tuple(bufs.num_sel.shape), dtype=torch.int32, device=dev)

    def step(s):
        q, k_new, v_new = inputs[s]
        quest.quest_append_score(L, q, k_new, v_new, layer.cu1, ctx_b[s], 1, layer.pt,
                                 layer.k_cache, layer.v_cache, layer.kmeta, bufs.scores, reduce)
        quest.quest_topk_sparse_decode(L, q, layer.k_cache, layer.v_cache, layer.pt, ctx_a[s],
                                       bufs.scores, budgets[s], max_k, sm, bufs.sel_pages,
                                       bufs.num_sel, bufs.out, bufs.workspace, n_sink, n_recent)

    step(0)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_steps)]
    torch.cuda.synchronize()
    for s in range(n_steps):
        evict()
        ev[s][0].record()
        step(s)
        ev[s][1].record()
        sels[s].copy_(bufs.sel_pages)
        nsels[s].copy_(bufs.num_sel)
    torch.cuda.synchronize()
    total_s = sum(e[0].elapsed_time(e[1]) for e in ev) / 1e3
    meta_b = kv_b = 0
    for s in range(n_steps):
        m, kv = step_bytes(w, ctx_a[s], sels[s], nsels[s])
        meta_b += m
        kv_b += kv
    return {"page_size": P, "group_reduce": reduce, "n_sink": n_sink, "n_recent": n_recent,
            "tokens_per_s": B * n_steps / total_s, "ms_per_step": total_s / n_steps * 1e3,
            "steps": n_steps, "metadata_bytes_per_step": meta_b / n_steps,
            "selected_kv_bytes_per_step": kv_b / n_steps,
            "hbm_gbps": (meta_b + kv_b) / total_s / 1e9,
            "hbm_frac_peak": (meta_b + kv_b) / total_s / 1e9 / PEAK_HBM_GBPS,
            "one_kernel_topk_decode": quest.quest_topk_sparse_decode_fused(L, B, max_k)}


def variant_legs(layer, inputs, ctx_b, ctx_a, budgets, sm, evict, n_steps, dev, restore):
    """The variants the method leaves open, on the benchmark's shape and token
    budget: the SUM group reduction and forced sink / recent pages on the
    same cache, and page sizes 8, 32 and 64 on caches of their own."""
    out = {}
    restore()
    out["sum_reduce"] = timed_variant(layer, inputs, ctx_b, ctx_a, budgets, sm, evict, n_steps,
                                      dev, reduce="sum")
    restore()
    out["forced_1_sink_2_recent"] = timed_variant(layer, inputs, ctx_b, ctx_a, budgets, sm,
                                                  evict, n_steps, dev, n_sink=1, n_recent=2)
    restore()
    for P in (8, 32, 64):
        wp = workloads.scaled(layer.w, page_size=P)
        lp = BenchLayer(wp, n_steps, dev)
        lp.prefill = None
        cb = [(lp.ctx0 + s).to(torch.int32) for s in range(n_steps)]
        ca = [(lp.ctx0 + s + 1).to(torch.int32) for s in range(n_steps)]
        bp = [workloads.budget_tokens(wp, c).to(dev) for c in ca]
        out[f"page_{P}"] = timed_variant(lp, inputs, cb, ca, bp, sm, evict, n_steps, dev)
        del lp
        torch.cuda.empty_cache()
    return out


def layers48_step(n_steps, n_copies, evict, dev, extra_replays=4):
    """The 48-layer decode step (batch 64 x 32768 tokens, page 16, budget 2048):
    48 layer-steps per model step, layer l on resident copy l mod n_copies
    (every layer has the same shape and cost; n_copies x 537 MB of metadata
    and selected K/V keeps each layer's bytes out of the Infinity Cache),
    n_steps model steps captured in one HIP graph and replayed back to back.
    Bytes = metadata + selected valid K/V of every layer-step."""
    w = workloads.scaled(workloads.WORKLOADS["layers48"], layers=1)
    n_layers = workloads.WORKLOADS["layers48"].layers
    base = BenchLayer(w, n_steps, dev)
    base.prefill = None
    copies = [base] + [base.resident_copy() for _ in range(n_copies - 1)]
    sm = workloads.default_sm_scale(w)
    B, P = w.batch, w.page_size
    inputs = make_steps(w, n_copies, dev)
    ctx_b = [(base.ctx0 + s).to(torch.int32) for s in range(n_steps)]
    ctx_a = [(base.ctx0 + s + 1).to(torch.int32) for s in range(n_steps)]
    budgets = [workloads.budget_tokens(w, c).to(dev) for c in ctx_a]
    max_k = max(1, max(int((b // P).max()) for b in budgets))
    total = n_steps * n_layers
    per_copy = [quest.alloc_decode_buffers(base.L, B, max_k, dev) for _ in range(n_copies)]
    sels = torch.empty((total,) + tuple(per_copy[0].sel_pages.shape), dtype=torch.int32,
                       device=dev)
    nsels = torch.empty((total,) + tuple(per_copy[0].num_sel.shape), dtype=torch.int32,
                        device=dev)
    step_bufs = [dataclasses.replace(per_copy[i % n_copies], sel_pages=sels[i],
                                     num_sel=nsels[i]) for i in range(total)]

    def layer_step(i):
        m, c = i // n_layers, (i % n_layers) % n_copies
        run_step(copies[c], step_bufs[i], i, inputs[c], ctx_b[m], ctx_a[m], budgets[m], sm)

    for i in range(total):
        layer_step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(total):
            layer_step(i)
    graph.replay()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    evict()
    torch.cuda.synchronize()
    ev[0].record()
    graph.replay()
    ev[1].record()
    torch.cuda.synchronize()
    total_s = ev[0].elapsed_time(ev[1]) / 1e3
    # further replays, each queued behind an eviction sweep (the first one,
    # launched after a host synchronisation, also carries the graph's launch)
    replay_ms = [total_s / n_steps * 1e3]
    for _ in range(extra_replays):
        evict()
        ev[0].record()
        graph.replay()
        ev[1].record()
        torch.cuda.synchronize()
        replay_ms.append(ev[0].elapsed_time(ev[1]) / n_steps)
    median_ms = sorted(replay_ms)[len(replay_ms) // 2]
    meta_b = kv_b = 0
    for i in range(total):
        m_, kv = step_bytes(w, ctx_a[i // n_layers], sels[i], nsels[i])
        meta_b += m_
        kv_b += kv
    res = {"what": "48 layer-steps per model step (batch 64 x 32768, page 16, budget 2048), "
                   f"layer l on resident copy l mod {n_copies}, {n_steps} model steps replayed "
                   "from one HIP graph",
           "ms_per_step": total_s / n_steps * 1e3, "tokens_per_s": B * n_steps / total_s,
           "layers": n_layers, "steps": n_steps, "resident_layer_copies": n_copies,
           "bytes_per_step": (meta_b + kv_b) / n_steps,
           "hbm_gbps": (meta_b + kv_b) / total_s / 1e9,
           "hbm_frac_peak": (meta_b + kv_b) / total_s / 1e9 / PEAK_HBM_GBPS,
           "replays_ms_per_step": replay_ms, "ms_per_step_median": median_ms,
           "hbm_frac_peak_median": (meta_b + kv_b) / n_steps / (median_ms * 1e-3) / 1e9
                                   / PEAK_HBM_GBPS,
           "one_kernel_topk_decode": quest.quest_topk_sparse_decode_fused(base.L, B, max_k)}
    del graph, step_bufs, per_copy, copies, base
    torch.cuda.empty_cache()
    return res


def prefill_chunk_append(layer, chunk, n_calls, evict, dev):
    """Bulk on_kv_stored at prefill-chunk granularity: each call stores one
    `chunk`-token chunk of every request's prompt (positions c*chunk ..) with
    quest_append_kv.  The chunks are the prompt's own tokens at their own
    positions and start on a page boundary, so every call rewrites identical
    bytes and leaves the cache as it was.  Bytes = new K/V read + K/V written
    + the chunk pages' metadata written."""
    w, L = layer.w, layer.L
    B, H, D, P = w.batch, w.num_kv_heads, w.head_dim, w.page_size
    k_all, v_all, cu = layer.prefill
    cuh = cu.cpu().tolist()
    lens = [cuh[r + 1] - cuh[r] for r in range(B)]
    n_chunks = min(lens) // chunk
    if n_chunks == 0 or chunk % P:
        return None
    calls = []
    for i in range(min(n_calls, n_chunks)):
        c = i * (n_chunks // min(n_calls, n_chunks))
        idx = torch.cat([torch.arange(cuh[r] + c * chunk, cuh[r] + (c + 1) * chunk)
                         for r in range(B)]).to(dev)
        calls.append((k_all[idx].contiguous(), v_all[idx].contiguous(),
                      torch.full((B,), c * chunk, dtype=torch.int32, device=dev)))
    cu_c = torch.arange(0, B * chunk + 1, chunk, dtype=torch.int32, device=dev)

    def call(i):
        k, v, ctx0 = calls[i]
        quest.quest_append_kv(L, k, v, cu_c, ctx0, chunk, layer.pt, layer.k_cache,
                              layer.v_cache, layer.kmeta)

    call(0)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in calls]
    torch.cuda.synchronize()
    for i in range(len(calls)):
        evict()
        ev[i][0].record()
        call(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    total_s = sum(e[0].elapsed_time(e[1]) for e in ev) / 1e3
    elem = 2 if w.dtype == "bf16" else 4
    tokens = B * chunk * len(calls)
    nbytes = tokens * H * D * elem * 4 + (tokens // P) * H * 2 * D * elem
    # a plain device copy of the call's new K and V (the bytes it reads, and
    # about the bytes it writes), timed the same way: what moving these bytes
    # costs on this chip without any paging or metadata
    src = torch.cat([calls[0][0].reshape(-1), calls[0][1].reshape(-1)])
    dst = torch.empty_like(src)
    dst.copy_(src)
    evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in calls]
    torch.cuda.synchronize()
    for e in evc:
        evict()
        e[0].record()
        dst.copy_(src)
        e[1].record()
    torch.cuda.synchronize()
    copy_s = sum(e[0].elapsed_time(e[1]) for e in evc) / 1e3
    copy_bytes = 2 * src.numel() * src.element_size()
    del src, dst
    return {"what": f"quest_append_kv of one {chunk}-token chunk per request ({B} requests) "
                    "per call, cache evicted before each call",
            "chunk_tokens": chunk, "calls": len(calls), "us_per_call": total_s / len(calls) * 1e6,
            "tokens_per_s": tokens / total_s, "bytes_per_call": nbytes / len(calls),
            "hbm_gbps": nbytes / total_s / 1e9, "hbm_frac_peak": nbytes / total_s / 1e9 / PEAK_HBM_GBPS,
            "copy_probe": {"what": "device copy of one call's new K and V, cache evicted before each",
                           "bytes": copy_bytes, "us": copy_s / len(calls) * 1e6,
                           "gbps": copy_bytes * len(calls) / copy_s / 1e9,
                           "append_rate_of_copy_rate": (nbytes / total_s) /
                                                       (copy_bytes * len(calls) / copy_s)}}


def config_legs(names, n_steps, evict, dev, warm=2):
    """One decode step (append + scores, then the combined top-k + decode
    call) of each named workload on a cache of its own, after `warm`
    untimed steps: the Infinity Cache evicted before each timed step, one
    event pair per step; tokens/s, and HBM rate over metadata + selected
    valid K/V."""
    out = {}
    for name in names:
        w = workloads.WORKLOADS[name]
        layer = BenchLayer(w, warm + n_steps, dev)
        inputs = make_steps(w, warm + n_steps, dev)
        ctx_b = [(layer.ctx0 + s).to(torch.int32) for s in range(warm + n_steps)]
        ctx_a = [(layer.ctx0 + s + 1).to(torch.int32) for s in range(warm + n_steps)]
        budgets = [workloads.budget_tokens(w, c).to(dev) for c in ctx_a]
        max_k = max(1, max(int((b // w.page_size).max()) for b in budgets))
        bufs = quest.alloc_decode_buffers(layer.L, w.batch, max_k, dev)
        sm = workloads.default_sm_scale(w)
        for s in range(warm):
            run_step(layer, bufs, s, inputs[s], ctx_b[s], ctx_a[s], budgets[s], sm)
        total_s, meta_b, kv_b = 0.0, 0, 0
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for s in range(warm, warm + n_steps):
            evict()
            ev[0].record()
            run_step(layer, bufs, s, inputs[s], ctx_b[s], ctx_a[s], budgets[s], sm)
            ev[1].record()
            torch.cuda.synchronize()
            total_s += ev[0].elapsed_time(ev[1]) / 1e3
            m, kv = step_bytes(w, ctx_a[s], bufs.sel_pages, bufs.num_sel)
            meta_b += m
            kv_b += kv
        gbps = (meta_b + kv_b) / total_s / 1e9
        ctx = workloads.context_lengths(w)
        out[name] = {"batch": w.batch, "ctx": [int(ctx.min()), int(ctx.max())],
                     "page_size": w.page_size, "dtype": w.dtype, "max_k": max_k,
                     "steps": n_steps, "us_per_step": total_s / n_steps * 1e6,
                     "tokens_per_s": w.batch * n_steps / total_s,
                     "bytes_per_step": (meta_b + kv_b) / n_steps,
                     "hbm_gbps": gbps, "hbm_frac_peak": gbps / PEAK_HBM_GBPS,
                     "one_kernel_topk_decode": quest.quest_topk_sparse_decode_fused(
                         layer.L, w.batch, max_k)}
        del layer, bufs, inputs
        torch.cuda.empty_cache()
    return out


def step_bytes(w, ctx_after, sel, nsel):
    """Algorithmic HBM bytes of one step: every live page's metadata row plus
    the valid tokens of every selected page (K and V)."""
    P, D, Hkv = w.page_size, w.head_dim, w.num_kv_heads
    es = 2 if w.dtype == "bf16" else 4
    ctx = ctx_after.cpu().to(torch.int64)
    n = (ctx + P - 1) // P
    meta = int(n.sum()) * Hkv * 2 * D * es
    sel = sel.cpu().to(torch.int64)                         # [B][Hkv][max_k]
    live = torch.arange(sel.shape[-1])[None, None, :] < nsel.cpu()[:, :, None]
    valid = torch.clamp(ctx[:, None, None] - sel * P, min=0, max=P)
    kv_tokens = int((valid * live).sum())
    return meta, kv_tokens * 2 * D * es


def full_step_bytes(w, ctx_after, nsel, max_k, n_split, max_pages):
    """Every byte one step moves, the headline ones (metadata rows and the
    selected valid K/V, step_bytes) and the rest: q and out, the new tokens'
    K/V read and stored with their page's metadata row read and written,
    page-table entries (one per live page and KV head for the scoring, one
    per selected page for the decode), the scores written once and read by
    each split of a row (the selection reads the row's register layout, up to
    the table stride), the selection lists, and the split partials written
    and read by the merge."""
    P, D, Hkv, Hq, B = w.page_size, w.head_dim, w.num_kv_heads, w.num_q_heads, w.batch
    G = Hq // Hkv
    es = 2 if w.dtype == "bf16" else 4
    n = (ctx_after.cpu().to(torch.int64) + P - 1) // P
    live_pages = int(n.sum()) * Hkv
    selected = int(nsel.cpu().to(torch.int64).sum())
    parts = {
        "q": B * Hq * D * es,
        "out": B * Hq * D * es,
        "append_kv": B * Hkv * D * es * 4,
        "append_metadata_row": B * Hkv * 2 * D * es * 2,
        "page_table": (live_pages + selected) * 4,
        "scores_write": live_pages * 4,
        "scores_read": n_split * B * Hkv * min(max_pages, 8192) * 4,
        "selection_lists": B * Hkv * (max_k + 1) * 4,
        "split_partials": 2 * B * Hkv * n_split * G * (D + 2) * 4,
    }
    parts["total_besides_headline"] = sum(parts.values())
    return parts


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


SCORE_SOURCES = ["kv_cache_decode_quest_amd/csrc/page_scores.hip",
                 "kv_cache_decode_quest_amd/csrc/append_inline.h",
                 "kv_cache_decode_quest_amd/csrc/quest_device.h"]


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "page_scores_bench128k_traffic.json")
COPY_KERNEL = "copy"    # the runtime's buffer-copy kernel: the known-size calibration


def measured_traffic(workload):
    """HBM traffic of the scoring kernel from the committed rocprofv3 counter
    summary, if it was taken on this workload and on the current kernel
    source (else None)."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    rec = json.load(open(TRAFFIC_JSON))
    if rec.get("workload") != workload or rec.get("source_hash") != source_hash(SCORE_SOURCES):
        return None
    return rec.get("bytes_per_launch")


def traffic_from_pmc(fetch_csv, write_csv, copy_bytes):
    """Per-launch HBM bytes of the scoring kernel from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the
    same counter reads for the calibration copy of copy_bytes (read and
    written once each)."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        for row in csv.DictReader(open(path)):
            if row.get("Counter_Name") != counter:
                continue
            name = row["Kernel_Name"]
            key = "scores" if "page_scores" in name else (
                COPY_KERNEL if "copyBuffer" in name else None)
            if key:
                vals.setdefault(key, []).append(float(row["Counter_Value"]))
        out = {"scores": sum(vals["scores"]) / len(vals["scores"])}
        # the calibration copy is by far the largest buffer copy of the run
        big = sorted(vals[COPY_KERNEL])[-3:]
        out[COPY_KERNEL] = sum(big) / len(big)
        return out

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    wr = per_kernel(write_csv, "WRITE_SIZE")
    f_scale = copy_bytes / (f[COPY_KERNEL] * 1024.0)
    w_scale = copy_bytes / (wr[COPY_KERNEL] * 1024.0)
    fetch_b = f["scores"] * 1024.0 * f_scale
    write_b = wr["scores"] * 1024.0 * w_scale
    return {"kernel": "page_scores_mfma_kernel<128, true>", "workload": "bench128k",
            "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
            "bytes_per_launch": fetch_b + write_b,
            "fetch_scale": f_scale, "write_scale": w_scale,
            "raw_fetch_kib": f["scores"], "raw_write_kib": wr["scores"],
            "copy_fetch_kib": f[COPY_KERNEL], "copy_write_kib": wr[COPY_KERNEL],
            "copy_bytes": copy_bytes, "source_hash": source_hash(SCORE_SOURCES)}


def stream_probe(copies, n_launch):
    """A plain contiguous read of each metadata copy (the bytes the scoring
    kernel scans, plus the unused pool pages), launched back to back over the
    copies between one event pair, like the scoring kernel's roofline loop."""
    sink = torch.zeros(4, dtype=torch.int32, device=copies[0].device)
    R = len(copies)
    nbytes = copies[0].numel() * copies[0].element_size()
    for i in range(R):
        probe.stream_read(copies[i], sink)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(n_launch):
        probe.stream_read(copies[i % R], sink)
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) / n_launch * 1e3
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"what": "contiguous 16-byte-load read of one metadata copy per launch, copies in "
                    "rotation, launches back to back", "bytes": nbytes, "us": us, "gbps": gbps,
            "frac_of_peak": gbps / PEAK_HBM_GBPS}


def gather_probe(w, layers, sels, nsels, n_launch, dev):
    """A plain read of exactly the K and V pages one step selects (one page
    and KV head of K and of V per chunk pair, at scattered offsets): each
    resident copy with its own selection, the copies in rotation, launches
    back to back between one event pair (like the scoring kernel's roofline
    loop; the copies' selected pages together exceed the Infinity Cache)."""
    P, D, Hkv = w.page_size, w.head_dim, w.num_kv_heads
    es = 2 if w.dtype == "bf16" else 4
    chunk = P * D * es
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    pt = layers[0].pt.to(torch.int64)
    runs = []
    for c, lay in enumerate(layers):
        sel, nsel = sels[c].to(torch.int64), nsels[c]
        live = torch.arange(sel.shape[-1], device=dev)[None, None, :] < nsel[:, :, None]
        rr, gg, ii = torch.nonzero(live, as_tuple=True)
        phys = pt[rr, sel[rr, gg, ii]]
        offs = ((phys * Hkv + gg) * (chunk // 16)).contiguous()
        runs.append((lay, offs))
    for lay, offs in runs:
        probe.gather_read(lay.k_cache, lay.v_cache, offs, chunk, sink)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(n_launch):
        lay, offs = runs[i % len(runs)]
        probe.gather_read(lay.k_cache, lay.v_cache, offs, chunk, sink)
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) / n_launch * 1e3
    nbytes = sum(int(offs.numel()) for _, offs in runs) * 2 * chunk / len(runs)
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"what": f"read of the K and V pages of one step's selection ({chunk} B chunks per "
                    "page and KV head), each resident copy with its own selection, launches "
                    "back to back", "bytes": nbytes, "us": us, "gbps": gbps,
            "frac_of_peak": gbps / PEAK_HBM_GBPS, "launches": n_launch}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, layer_inputs, steps_inputs, n_req, n_steps, single_steps):
    """The fp64 oracle doing the same per-request decode work on the host:
    per request and step, store the new token, refresh its page's bounds,
    then scores, top-k and attention.  Timed twice on successive decode
    steps: single-threaded (`single_steps` steps of every request), then with
    one host thread per request (the oracle is plain C with no shared state;
    its ctypes calls release the interpreter lock, and requests own disjoint
    pages) for the next `n_steps` steps."""
    import numpy as np
    import oracle
    from concurrent.futures import ThreadPoolExecutor

    def host(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
            else t.numpy()

    lay, k_new, v_new, cu = layer_inputs
    s = oracle.Shape(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                     lay.num_pool_pages, oracle.BF16 if w.dtype == "bf16" else oracle.F32)
    kh, vh = workloads.empty_pool(w, lay, "cpu")
    kh, vh = host(kh).copy(), host(vh).copy()
    pt = lay.page_table.cpu().numpy()
    cuh = cu.cpu().numpy()
    kn, vn = host(k_new), host(v_new)
    ctx0 = lay.ctx0.cpu().numpy()
    log(f"cpu baseline: storing the prompt KV of {n_req} requests in the oracle's pool")
    bounds = {}
    t_build = 0.0
    for r in range(n_req):
        a, b = int(cuh[r]), int(cuh[r + 1])
        oracle.store_tokens(s, np.ascontiguousarray(kn[a:b]), np.ascontiguousarray(vn[a:b]), 0,
                            pt[r], kh, vh)
        t0 = time.perf_counter()
        bounds[r] = oracle.request_bounds(s, kh, pt[r], int(ctx0[r]))
        t_build += time.perf_counter() - t0
    build_pages = sum(oracle.num_pages(int(ctx0[r]), w.page_size) for r in range(n_req))
    sm = workloads.default_sm_scale(w)
    total = single_steps + n_steps
    step_host = [tuple(host(x) for x in steps_inputs[st]) for st in range(total)]

    def request_steps(r, steps):
        for st in steps:
            q, kn1, vn1 = step_host[st]
            pos = int(ctx0[r]) + st
            oracle.store_tokens(s, np.ascontiguousarray(kn1[r:r + 1]),
                                np.ascontiguousarray(vn1[r:r + 1]), pos, pt[r], kh, vh)
            ctx = pos + 1
            j = pos // w.page_size
            if j == bounds[r].shape[0]:
                bounds[r] = np.concatenate([bounds[r], bounds[r][:1]], axis=0)
            bounds[r][j] = oracle.page_bounds(s, kh, pt[r], ctx, j)
            budget = int(workloads.budget_tokens(w, torch.tensor([ctx], dtype=torch.int32))[0])
            oracle.decode_request(s, np.ascontiguousarray(q[r]), kh, vh, pt[r], ctx, budget, sm,
                                  bounds=np.ascontiguousarray(bounds[r]))
        return len(steps)

    log(f"cpu baseline: single thread, {single_steps} steps x {n_req} requests")
    t0 = time.perf_counter()
    done1 = 0
    for st in range(single_steps):
        for r in range(n_req):
            done1 += request_steps(r, [st])
    dt1 = time.perf_counter() - t0
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max(1, min(avail, n_req))
    log(f"cpu baseline: {threads} threads, {n_steps} steps x {n_req} requests")
    later = list(range(single_steps, total))
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        done = sum(ex.map(lambda r: request_steps(r, later), range(n_req)))
    dt = time.perf_counter() - t0
    cpu = cpu_model()
    return {"value": done / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_steps} decode steps x {n_req} of {w.batch} requests of the same "
                      f"workload (store, page-bounds refresh, scores, top-k, attention per "
                      f"request-step), fp64, one host thread per request ({threads} threads of "
                      f"{avail} available); {dt:.1f} s on {cpu}",
            "seconds": dt, "cpu_model": cpu, "cores_available": avail,
            "single_thread": {"value": done1 / dt1, "unit": "tokens/s", "cores": 1,
                              "steps": single_steps, "seconds": dt1},
            "metadata_build": {"what": "from-scratch page min/max of the prompts (the oracle's "
                                       "request bounds), one thread, timed apart from the steps",
                               "requests": n_req, "pages": build_pages, "seconds": t_build,
                               "pages_per_s": build_pages / t_build if t_build > 0 else None}}


def cpu_layers48_sample(dev, n_threads):
    """The oracle on one layer-step of the 48-layer workload (batch 64 x 32768
    tokens, page 16, budget 2048): per request store the new token, refresh
    its page's bounds, then scores, top-k and attention, requests spread over
    the host threads.  Every layer of the model step has this shape and cost,
    so the model step is 48 of these; the sample is one layer-step."""
    import numpy as np
    import oracle
    from concurrent.futures import ThreadPoolExecutor

    w = workloads.scaled(workloads.WORKLOADS["layers48"], layers=1)
    lay = workloads.make_layout(w, dev)
    k_new, v_new, cu, _ = workloads.prefill_tokens(w, lay, dev)
    s = oracle.Shape(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                     lay.num_pool_pages, oracle.BF16)

    def host(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    fill = 0 if w.poison is None else \
        int(torch.tensor(w.poison, dtype=torch.bfloat16).view(torch.int16).item()) & 0xffff
    kh = np.full((lay.num_pool_pages, w.num_kv_heads, w.page_size, w.head_dim), fill, np.uint16)
    vh = np.full((lay.num_pool_pages, w.num_kv_heads, w.head_dim, w.page_size), fill, np.uint16)
    pt = lay.page_table.cpu().numpy()
    cuh = cu.cpu().numpy()
    kn, vn = host(k_new), host(v_new)
    del k_new, v_new
    ctx0 = lay.ctx0.cpu().numpy()
    bounds = []
    for r in range(w.batch):
        a, b = int(cuh[r]), int(cuh[r + 1])
        oracle.store_tokens(s, np.ascontiguousarray(kn[a:b]), np.ascontiguousarray(vn[a:b]), 0,
                            pt[r], kh, vh)
        bounds.append(oracle.request_bounds(s, kh, pt[r], int(ctx0[r])))
    del kn, vn
    q, k1, v1 = (host(x) for x in workloads.step_tokens(w, dev, 0, 0))
    sm = workloads.default_sm_scale(w)

    def one(r):
        pos = int(ctx0[r])
        oracle.store_tokens(s, np.ascontiguousarray(k1[r:r + 1]), np.ascontiguousarray(v1[r:r + 1]),
                            pos, pt[r], kh, vh)
        j = pos // w.page_size
        bnd = bounds[r]
        if j == bnd.shape[0]:
            bnd = np.concatenate([bnd, bnd[:1]], axis=0)
        bnd[j] = oracle.page_bounds(s, kh, pt[r], pos + 1, j)
        budget = int(workloads.budget_tokens(w, torch.tensor([pos + 1], dtype=torch.int32))[0])
        oracle.decode_request(s, np.ascontiguousarray(q[r]), kh, vh, pt[r], pos + 1, budget, sm,
                              bounds=np.ascontiguousarray(bnd))
        return 1

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=n_threads) as ex:
        done = sum(ex.map(one, range(w.batch)))
    dt = time.perf_counter() - t0
    layers = workloads.WORKLOADS["layers48"].layers
    return {"what": "the oracle on one layer-step of the 48-layer workload (64 requests x "
                    "32768 tokens: store, page-bounds refresh, scores, top-k, attention per "
                    f"request), {n_threads} host threads; a model step is {layers} such "
                    "layer-steps",
            "layer_step_seconds": dt, "requests": done, "cores": n_threads,
            "model_step_seconds": dt * layers,
            "tokens_per_s": w.batch / (dt * layers), "unit": "tokens/s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="bench128k", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--flush-mib", type=int, default=2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip one timed step of each other single-layer workload")
    ap.add_argument("--config-steps", type=int, default=4)
    ap.add_argument("--cpu-requests", type=int, default=8)
    ap.add_argument("--cpu-steps", type=int, default=32,
                    help="decode steps of the threaded CPU-oracle run")
    ap.add_argument("--cpu-single-steps", type=int, default=8,
                    help="decode steps of the single-threaded CPU-oracle run")
    ap.add_argument("--resident-layers", type=int, default=8,
                    help="copies of the layer the timed steps rotate over")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense decode reference (every page, no selection)")
    ap.add_argument("--dense-steps", type=int, default=16)
    ap.add_argument("--no-per-head", action="store_true",
                    help="skip the per-q-head selection reference")
    ap.add_argument("--no-layers48", action="store_true",
                    help="skip the 48-layer batch-64 step")
    ap.add_argument("--layers48-steps", type=int, default=4)
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the SUM-reduction, forced-page and page-size variants")
    ap.add_argument("--prefill-chunk", type=int, default=4096,
                    help="chunk size of the prefill append leg (0 to skip)")
    ap.add_argument("--roofline-copies", type=int, default=8)
    ap.add_argument("--roofline-launches", type=int, default=128,
                    help="back-to-back launches the dominant kernel's average is taken over "
                         "(rounded down to a multiple of the copies); independent of --steps, "
                         "so a short run does not weigh the first launch from an idle GPU more")
    ap.add_argument("--extra-replays", type=int, default=4,
                    help="timed replays after the first, for the median per-step time")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run a plain copy of this size (counter calibration)")
    ap.add_argument("--traffic-from-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_MIB"),
                    help="no GPU: turn two rocprofv3 --pmc runs into the committed traffic record")
    args = ap.parse_args()
    if args.traffic_from_pmc:
        fcsv, wcsv, mib = args.traffic_from_pmc
        rec = traffic_from_pmc(fcsv, wcsv, int(mib) * (1 << 20))
        json.dump(rec, open(TRAFFIC_JSON, "w"), indent=1)
        print(json.dumps(rec))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the Quest decode path here is built and timed "
              "on a single MI355X (requests and KV heads are independent, so it would shard "
              "by request or by KV head with no exchange); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    dev = torch.device("cuda:0")
    quest.load()
    w = workloads.WORKLOADS[args.workload]
    if w.layers != 1:
        print("bench.py times single-layer workloads", file=sys.stderr)
        sys.exit(2)
    K, W = args.steps, args.warmup
    # the CPU-oracle baseline runs its own successive decode steps on a host
    # copy of the same cache: the page table has room for them too
    cpu_total = 0 if args.no_cpu_baseline else args.cpu_single_steps + args.cpu_steps
    cap = max(K, W, cpu_total, 1)
    log(f"workload {w.name}: batch {w.batch}, ctx {workloads.context_lengths(w).tolist()[:4]}..,"
        f" building the cache")
    layer = BenchLayer(w, cap, dev)
    torch.cuda.synchronize()
    log("cache built; drawing step inputs")
    inputs = make_steps(w, cap, dev)
    ctx_b = [(layer.ctx0 + s).to(torch.int32) for s in range(cap)]
    ctx_a = [(layer.ctx0 + s + 1).to(torch.int32) for s in range(cap)]
    budgets = [workloads.budget_tokens(w, c).to(dev) for c in ctx_a]
    max_k = max(1, max(int((b // w.page_size).max()) for b in budgets))
    bufs = quest.alloc_decode_buffers(layer.L, w.batch, max_k, dev)
    sm = workloads.default_sm_scale(w)
    plan = quest.quest_sparse_decode_plan(layer.L, w.batch, max_k)
    flush = torch.ones(args.flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)

    def evict():
        torch.sum(flush)

    # snapshot the metadata rows the warm-up touches, restore them afterwards
    P = w.page_size
    touched = []
    for r in range(w.batch):
        c0 = int(layer.ctx0[r])
        for j in range(c0 // P, (c0 + cap - 1) // P + 1):
            touched.append(int(layer.pt[r, j]))
    touched = torch.tensor(sorted(set(touched)), dtype=torch.int64, device=dev)
    saved = layer.kmeta[touched].clone()

    def restore():
        layer.kmeta[touched] = saved

    # 1. the timed steps: step s runs on copy s % NL at decode position s // NL
    NL = max(1, args.resident_layers)
    log(f"resident copies of the layer: {NL}")
    layers = [layer] + [layer.resident_copy() for _ in range(NL - 1)]
    sels = torch.empty((K,) + tuple(bufs.sel_pages.shape), dtype=torch.int32, device=dev)
    nsels = torch.empty((K,) + tuple(bufs.num_sel.shape), dtype=torch.int32, device=dev)
    per_copy = [quest.alloc_decode_buffers(layer.L, w.batch, max_k, dev) for _ in range(NL)]
    step_bufs = [dataclasses.replace(per_copy[s % NL], sel_pages=sels[s], num_sel=nsels[s])
                 for s in range(K)]

    def rot_step(s):
        m = s // NL
        run_step(layers[s % NL], step_bufs[s], s, inputs[s], ctx_b[m], ctx_a[m], budgets[m], sm)

    def restore_all():
        # Every copy's touched metadata rows back to their state before the
        # first step.  Re-storing a token at its position rewrites the same
        # K/V, but a page's min/max only restarts at slot 0: a pass that
        # starts mid-page would otherwise see bounds that already hold the
        # later steps' tokens, and score that page differently.  With this,
        # every pass over the K steps (the eager one and each replay) sees
        # the same state step by step.
        for c in layers:
            c.kmeta[touched] = saved

    log(f"warm-up: {W} steps, then one eager pass over the {K} steps")
    for s in range(W):
        rot_step(s % K)
    restore_all()
    for s in range(K):
        rot_step(s)
    torch.cuda.synchronize()
    eager_sel, eager_nsel = sels.clone(), nsels.clone()
    eager_out = [b.out.clone() for b in per_copy]        # each copy's last step
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(K):
            rot_step(s)
    restore_all()
    graph.replay()
    torch.cuda.synchronize()
    def same_as_eager():
        return (torch.equal(sels, eager_sel) and torch.equal(nsels, eager_nsel) and
                all(torch.equal(b.out, o) for b, o in zip(per_copy, eager_out)))

    same = [same_as_eager()]
    log(f"timed: {K} steps replayed")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    restore_all()
    evict()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev[0].record()
    graph.replay()
    ev[1].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_s = ev[0].elapsed_time(ev[1]) / 1e3
    same.append(same_as_eager())
    value = w.batch * K / total_s
    # the same replay a few more times (cache evicted before each), for the
    # spread of the per-step time; `value` is the first timed replay alone
    replay_ms = [total_s / K * 1e3]
    for _ in range(args.extra_replays):
        restore_all()
        evict()
        ev[0].record()
        graph.replay()
        ev[1].record()
        torch.cuda.synchronize()
        replay_ms.append(ev[0].elapsed_time(ev[1]) / K)
    same.append(same_as_eager())

    meta_b, kv_b = 0, 0
    for s in range(K):
        m, kv = step_bytes(w, ctx_a[s // NL], sels[s], nsels[s])
        meta_b += m
        kv_b += kv
    gbps = (meta_b + kv_b) / total_s / 1e9
    n_g = min(NL, K)
    gather = gather_probe(w, layers[:n_g], sels[:n_g], nsels[:n_g], max(16, n_g), dev)
    del graph, step_bufs, per_copy, layers
    torch.cuda.empty_cache()

    # 1b. the same steps on one copy, launched eagerly one at a time, the
    #     cache evicted before each (one event pair per step)
    restore()
    torch.cuda.synchronize()
    ev_step = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for s in range(K):
        evict()
        ev_step[s][0].record()
        run_step(layer, bufs, s, inputs[s], ctx_b[s], ctx_a[s], budgets[s], sm)
        ev_step[s][1].record()
    torch.cuda.synchronize()
    eager_each = sorted(e[0].elapsed_time(e[1]) for e in ev_step)
    eager_ms = sum(eager_each) / K
    eager = {"tokens_per_s": w.batch / (eager_ms / 1e3), "ms_per_step": eager_ms,
             "ms_per_step_median": eager_each[K // 2],
             "note": "one copy of the layer, steps launched one at a time from Python, "
                     "a 2 GiB read sweep before each step, one event pair per step"}
    # 1c. cache-assisted: the same steps on one copy from one HIP graph, back
    #     to back with no eviction, so consecutive steps find part of their
    #     bytes in the 256 MB Infinity Cache (labelled as such; not `value`)
    restore()
    g1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        for s in range(K):
            run_step(layer, bufs, s, inputs[s], ctx_b[s], ctx_a[s], budgets[s], sm)
    restore()
    g1.replay()
    restore()
    ev_w = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev_w[0].record()
    g1.replay()
    ev_w[1].record()
    torch.cuda.synchronize()
    warm_ms = ev_w[0].elapsed_time(ev_w[1]) / K
    del g1
    cache_assisted = {"ms_per_step": warm_ms, "tokens_per_s": w.batch / (warm_ms / 1e3),
                      "note": "cache-assisted: one copy of the layer, the K steps replayed back "
                              "to back from one HIP graph without eviction, so consecutive steps "
                              "reuse what the 256 MB Infinity Cache still holds"}
    # 2. per-kernel breakdown: the same steps again, an event between kernels
    #    (each event adds a few microseconds of dispatch gap to its interval)
    restore()
    ev_k = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for s in range(K):
        evict()
        run_step(layer, bufs, s, inputs[s], ctx_b[s], ctx_a[s], budgets[s], sm, ev_k[s])
    torch.cuda.synchronize()
    phase_ms = {name: [e[i].elapsed_time(e[i + 1]) for e in ev_k]
                for i, name in [(0, "append_score"), (1, "topk_decode")]}
    decode_us = sum(phase_ms["topk_decode"]) / K * 1e3
    decode_gbps = (kv_b / K) / (decode_us * 1e-6) / 1e9

    # 3. the dominant kernel alone: the fused append + page-scoring kernel over
    #    R copies of the metadata (R * 131 MB >> the 256 MB Infinity Cache, so
    #    every launch reads HBM), launched back to back between one event pair.
    #    Re-appending the same token is idempotent, so every launch does the
    #    same work as the first step's.
    R = args.roofline_copies
    restore()
    copies = [layer.kmeta.clone() for _ in range(R)]
    q0, k0, v0 = inputs[0]
    n_launch = max(R, (args.roofline_launches // R) * R)

    def fused(i):
        quest.quest_append_score(layer.L, q0, k0, v0, layer.cu1, ctx_b[0], 1, layer.pt,
                                 layer.k_cache, layer.v_cache, copies[i % R], bufs.scores)

    for i in range(R):
        fused(i)
    ev_r = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev_r[0].record()
    for i in range(n_launch):
        fused(i)
    ev_r[1].record()
    torch.cuda.synchronize()
    score_us = ev_r[0].elapsed_time(ev_r[1]) / n_launch * 1e3
    n_last = (ctx_a[0].cpu().to(torch.int64) + w.page_size - 1) // w.page_size
    score_bytes = int(n_last.sum()) * w.num_kv_heads * 2 * w.head_dim * \
        (2 if w.dtype == "bf16" else 4)
    score_gbps = score_bytes / (score_us * 1e-6) / 1e9
    stream = stream_probe(copies, n_launch)
    traffic = measured_traffic(w.name)
    if args.calibrate_copy_mib:
        src = torch.ones(args.calibrate_copy_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    del copies

    dense = None
    if not args.no_dense:
        log(f"dense reference: {min(args.dense_steps, K)} steps over every page")
        dense = dense_reference(layer, inputs, ctx_b, ctx_a, sm, evict,
                                max(1, min(args.dense_steps, K)), dev)
        # both timed the same way: eager launches, cache evicted before each step
        dense["sparse_speedup"] = eager["tokens_per_s"] / dense["tokens_per_s"]
        restore()

    per_head = None
    if not args.no_per_head:
        log(f"per-q-head selection: {min(args.dense_steps, K)} steps")
        per_head = per_q_head_reference(layer, inputs, ctx_b, ctx_a, budgets, sm, evict,
                                        max(1, min(args.dense_steps, K)), dev)
        per_head["shared_speedup"] = eager["tokens_per_s"] / per_head["tokens_per_s"]
        restore()

    variants = None
    if not args.no_variants:
        log(f"variants: SUM reduction, forced pages, page sizes 8/32/64, "
            f"{min(args.dense_steps, K)} steps each")
        variants = variant_legs(layer, inputs, ctx_b, ctx_a, budgets, sm, evict,
                                max(1, min(args.dense_steps, K)), dev, restore)
        for v in variants.values():
            v["vs_eager_evicted_page16"] = v["tokens_per_s"] / eager["tokens_per_s"]
        restore()

    prefill = None
    if args.prefill_chunk > 0:
        log(f"prefill append: {args.prefill_chunk}-token chunks")
        prefill = prefill_chunk_append(layer, args.prefill_chunk, 16, evict, dev)
        restore()

    layers48 = None
    if not args.no_layers48 and w.name == "bench128k":
        log("48-layer step: batch 64 x 32768 over 8 resident layers")
        layers48 = layers48_step(args.layers48_steps, 8, evict, dev, args.extra_replays)

    configs = None
    if not args.no_configs and w.name == "bench128k":
        names = ["tiny", "layer32k", "ragged"]
        log(f"other workloads: {', '.join(names)}, {args.config_steps} timed steps each")
        configs = config_legs(names, args.config_steps, evict, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, (layer.lay,) + layer.prefill, inputs,
                           min(args.cpu_requests, w.batch), args.cpu_steps, args.cpu_single_steps)
        if not args.no_layers48 and w.name == "bench128k":
            log("cpu baseline: one layer-step of the 48-layer workload")
            cpu["layers48_layer_step"] = cpu_layers48_sample(dev, cpu["cores"])

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": total_s / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch,
                   "ctx": workloads.context_lengths(w).tolist()[0] if w.ctx_range is None
                   else list(w.ctx_range),
                   "page_size": w.page_size, "budget_tokens": w.budget_tokens,
                   "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "decode_steps": K, "layers": 1},
        "hbm_gbps": gbps,
        "hbm_frac_peak": gbps / PEAK_HBM_GBPS,
        "bytes_per_step": {"metadata": meta_b / K, "selected_kv": kv_b / K},
        "full_bytes_per_step": full_step_bytes(
            w, ctx_a[0], nsels[0], max_k,
            quest.quest_topk_sparse_decode_plan(layer.L, w.batch, max_k)["num_splits"],
            layer.lay.max_pages),
        "roofline": {"kernel": "page_scores_mfma_kernel<128, true> (append + scores)",
                     "bound": "hbm",
                     "achieved": score_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": score_gbps / PEAK_HBM_GBPS,
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": score_bytes,
                     "avg_launch_us": score_us, "launches": n_launch,
                     "metadata_copies": R,
                     "frac_of_stream_probe": score_gbps / stream["gbps"]},
        "ms_per_step_median": sorted(replay_ms)[len(replay_ms) // 2],
        "replays_ms_per_step": replay_ms,
        "hbm_probe": {"stream_read": stream, "gather_read": gather},
        "kernels_us_event_bracketed": {k: sum(v) / K * 1e3 for k, v in phase_ms.items()},
        "topk_decode": {"selected_kv_gbps": decode_gbps, "plan": plan,
                        "combined_plan": quest.quest_topk_sparse_decode_plan(layer.L, w.batch,
                                                                             max_k),
                        "one_kernel": quest.quest_topk_sparse_decode_fused(layer.L, w.batch,
                                                                           max_k)},
        "launch": {"hip_graph": True, "resident_layer_copies": NL,
                   "steps_per_replay": K, "selections_and_outputs_equal_eager": all(same)},
        "wall_s_timed_replay": t_wall,
        "eager_evicted": eager,
        "cache_assisted_replay": cache_assisted,
        "dense_reference": dense,
        "per_q_head_reference": per_head,
        "variants": variants,
        "layers48_step": layers48,
        "other_workloads": configs,
        "prefill_append": prefill,
        "cpu_baseline": cpu,
        "host": platform.node(),
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
