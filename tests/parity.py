"""GPU-vs-oracle parity plumbing: builds one layer's paged cache on the GPU
through the library and the same cache on the host through the oracle, runs
decode steps on both, and compares.

Tolerances (floating point; integers and page ids are compared exactly):
  page metadata   exact (min/max involve no rounding)
  page scores     |S_gpu - S_ref| <= 2 (D + 2) 2^-24 max_h sum_d |q_hd| max(|min_d|, |max_d|)
                  (fp32 summation bound gamma_n, doubled for any rounding mode)
  selections      bit-exact per row; a row whose differing pages all pair up
                  with scores within 1e-5 relative is only flagged
  outputs         max-abs <= 2e-2 and mean-abs <= 2e-3, and elementwise
                  |err| <= 2^-8 |o| + 5e-4 (bf16) or 1e-5 (1 + |o|) (fp32)
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
from helpers import elem_of, to_f64, to_oracle
from kv_cache_decode_quest_amd import quest, workloads
from kv_cache_decode_quest_amd.workloads import WORKLOADS, scaled

U32 = 2.0 ** -24


def log(msg):
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


class Layer:
    """One attention layer's paged cache on the GPU (filled by quest_append_kv)
    and, optionally, its host mirror for the oracle (filled by oracle.store)."""

    def __init__(self, w: workloads.Workload, device, layer=0, capacity=None, host=True,
                 kmeta_junk=7.0, host_requests=None):
        self.w, self.device, self.layer = w, device, layer
        self.lay = workloads.make_layout(w, device, capacity)
        self.L = quest.make_layout(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                                   w.torch_dtype, self.lay.num_pool_pages, self.lay.max_pages)
        self.k_cache, self.v_cache = workloads.empty_pool(w, self.lay, device)
        self.kmeta = torch.full((self.lay.num_pool_pages, w.num_kv_heads, 2, w.head_dim),
                                kmeta_junk, dtype=w.torch_dtype, device=device)
        self.ctx = self.lay.ctx0.clone()
        self.pt = self.lay.page_table
        self.pt_host = self.pt.cpu().numpy()
        k_new, v_new, cu, ctx_before = workloads.prefill_tokens(w, self.lay, device, layer)
        max_new = int(self.ctx.max()) if self.ctx.numel() else 0
        quest.quest_append_kv(self.L, k_new, v_new, cu, ctx_before, max_new, self.pt,
                              self.k_cache, self.v_cache, self.kmeta)
        self.shape = oracle.Shape(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                                  self.lay.num_pool_pages, elem_of(w.torch_dtype))
        self.host = None
        if host:
            kh, vh = workloads.empty_pool(w, self.lay, "cpu")
            self.host = [to_oracle(kh).copy(), to_oracle(vh).copy()]
            # the host mirror holds every request, or only the sampled ones
            # (then only those requests may be compared)
            self.host_requests = list(range(w.batch)) if host_requests is None \
                else list(host_requests)
            cuh = cu.cpu().numpy()
            for r in self.host_requests:
                a, b = int(cuh[r]), int(cuh[r + 1])
                if b > a:
                    oracle.store_tokens(self.shape, np.ascontiguousarray(to_oracle(k_new[a:b])),
                                        np.ascontiguousarray(to_oracle(v_new[a:b])), 0,
                                        self.pt_host[r], self.host[0], self.host[1])
        del k_new, v_new
        torch.cuda.synchronize()

    # ----- one decode step ---------------------------------------------------
    def step_inputs(self, step):
        return workloads.step_tokens(self.w, self.device, self.layer, step)

    def host_append(self, k_new, v_new):
        """The oracle's store of one new token per request into the host
        mirror, at each request's current length (the GPU side is the
        caller's); the lengths then grow by one."""
        if self.host is not None:
            kn, vn = to_oracle(k_new), to_oracle(v_new)
            ctx = self.ctx.cpu().numpy()
            for r in self.host_requests:
                oracle.store_tokens(self.shape, np.ascontiguousarray(kn[r:r + 1]),
                                    np.ascontiguousarray(vn[r:r + 1]), int(ctx[r]),
                                    self.pt_host[r], self.host[0], self.host[1])
        self.ctx = self.ctx + 1

    def append_step(self, k_new, v_new):
        B = self.w.batch
        cu = torch.arange(B + 1, dtype=torch.int32, device=self.device)
        quest.quest_append_kv(self.L, k_new, v_new, cu, self.ctx, 1, self.pt, self.k_cache,
                              self.v_cache, self.kmeta)
        self.host_append(k_new, v_new)

    def append_score_step(self, q, k_new, v_new, bufs, reduce="max", topk=True):
        """One token per request through the fused quest_append_score (and the
        same store on the host), then (topk) the top-k."""
        B = self.w.batch
        cu = torch.arange(B + 1, dtype=torch.int32, device=self.device)
        quest.quest_append_score(self.L, q, k_new, v_new, cu, self.ctx, 1, self.pt, self.k_cache,
                                 self.v_cache, self.kmeta, bufs.scores, reduce)
        self.host_append(k_new, v_new)
        if topk:
            quest.quest_topk_pages(self.L, bufs.scores, self.ctx, self.budgets(), bufs.max_k,
                                   bufs.sel_pages, bufs.num_sel)

    def select_attend(self, q, bufs, sm_scale=None):
        """The top-k and the attention through quest_topk_sparse_decode."""
        sm = workloads.default_sm_scale(self.w) if sm_scale is None else sm_scale
        quest.quest_topk_sparse_decode(self.L, q, self.k_cache, self.v_cache, self.pt, self.ctx,
                                       bufs.scores, self.budgets(), bufs.max_k, sm,
                                       bufs.sel_pages, bufs.num_sel, bufs.out, bufs.workspace)

    def budgets(self):
        return workloads.budget_tokens(self.w, self.ctx).to(self.device)

    def max_k(self):
        b = self.budgets().cpu()
        return max(1, int((b // self.w.page_size).max()))

    def view(self, q, bufs, reduce="max"):
        quest.quest_page_scores(self.L, q, self.kmeta, self.pt, self.ctx, bufs.scores, reduce)
        quest.quest_topk_pages(self.L, bufs.scores, self.ctx, self.budgets(), bufs.max_k,
                               bufs.sel_pages, bufs.num_sel)

    def attend(self, q, bufs, sel=None, nsel=None, sm_scale=None):
        sm = workloads.default_sm_scale(self.w) if sm_scale is None else sm_scale
        quest.quest_sparse_decode(self.L, q, self.k_cache, self.v_cache, self.pt, self.ctx,
                                  bufs.sel_pages if sel is None else sel,
                                  bufs.num_sel if nsel is None else nsel, bufs.max_k, sm,
                                  bufs.out, bufs.workspace)

    def buffers(self, max_k=None, extra=0):
        if max_k is None:
            b = workloads.budget_tokens(self.w, self.ctx + extra).cpu()
            max_k = max(1, int((b // self.w.page_size).max()))
        return quest.alloc_decode_buffers(self.L, self.w.batch, max_k, self.device)

    # ----- oracle side -------------------------------------------------------
    def oracle_request(self, q, r, reduce="max", sm_scale=None, per_q_head=False, n_sink=0,
                       n_recent=0):
        sm = workloads.default_sm_scale(self.w) if sm_scale is None else sm_scale
        qr = np.ascontiguousarray(to_oracle(q[r]))
        ctx = int(self.ctx[r])
        budget = int(self.budgets()[r])
        return oracle.decode_request(self.shape, qr, self.host[0], self.host[1],
                                     self.pt_host[r], ctx, budget, sm, reduce,
                                     n_sink=n_sink, n_recent=n_recent, per_q_head=per_q_head)


# ----- comparisons -----------------------------------------------------------

def check_pool_bytes(layer: Layer):
    kg = to_oracle(layer.k_cache)
    vg = to_oracle(layer.v_cache)
    assert kg.tobytes() == layer.host[0].tobytes(), "K pool differs from the oracle's store"
    assert vg.tobytes() == layer.host[1].tobytes(), "V pool differs from the oracle's store"


def check_kmeta(layer: Layer, r, bounds, kmeta_host=None):
    """GPU metadata of request r's live pages equals the oracle's from-scratch
    min/max exactly (values; +0 and -0 compare equal)."""
    km = to_f64(layer.kmeta) if kmeta_host is None else kmeta_host
    n = bounds.shape[0]
    phys = layer.pt_host[r][:n]
    got = km[phys]                                  # [n][Hkv][2][D]
    bad = np.argwhere(got != bounds)
    assert bad.size == 0, f"request {r}: metadata differs at {bad[:5].tolist()}"


def score_bound(q_r, bounds, G):
    """Per (g, j) fp32 summation error bound of the page score."""
    qa = np.abs(q_r)                                # [Hq][D]
    mag = np.maximum(np.abs(bounds[:, :, 0, :]), np.abs(bounds[:, :, 1, :]))   # [n][Hkv][D]
    Hq, D = q_r.shape
    Hkv = Hq // G
    per_head = np.einsum("hd,jhd->hj", qa, np.repeat(mag, G, axis=1))   # [Hq][n]
    grp = per_head.reshape(Hkv, G, -1).max(axis=1)                      # [Hkv][n]
    return 2.0 * (D + 2) * U32 * grp + 1e-30


def check_scores(gpu_scores_r, ref_scores, q_r, bounds, G):
    n = ref_scores.shape[1]
    got = gpu_scores_r[:, :n]
    err = np.abs(got - ref_scores)
    tol = score_bound(q_r, bounds, G)
    worst = (err / tol).max() if n else 0.0
    assert np.all(err <= tol), f"scores outside the fp32 bound (worst ratio {worst:.3g})"
    return worst


def compare_selection(gpu_sel_row, gpu_nsel, ref_sel, ref_scores_row, rel=1e-5):
    """Returns 'exact' or 'flagged'; raises on a real mismatch."""
    k = len(ref_sel)
    assert gpu_nsel == k, f"num_sel {gpu_nsel} != {k}"
    assert np.all(gpu_sel_row[k:] == -1), "tail of the selection row is not -1"
    g = gpu_sel_row[:k]
    assert np.all(np.diff(g) > 0), "selection not strictly ascending"
    if np.array_equal(g, ref_sel):
        return "exact"
    A = sorted(set(ref_sel.tolist()) - set(g.tolist()))
    B = sorted(set(g.tolist()) - set(ref_sel.tolist()))
    assert len(A) == len(B)
    for a in A:
        for b in B:
            sa, sb = ref_scores_row[a], ref_scores_row[b]
            assert abs(sa - sb) <= rel * max(abs(sa), abs(sb)), \
                f"page {b} selected instead of {a}: scores {sb!r} vs {sa!r} are not a near-tie"
    return "flagged"


# Rows whose selection differed from the oracle's only by near-tied pages,
# over the test session; each such request's output is checked against the
# oracle's attention over the GPU's own selection (check_request_output).
FLAGGED = {"rows": 0, "requests": 0, "requests_checked": 0}


def check_request_output(lay: "Layer", q, r, sel_r, nsel_r, out_r, ref, what, n_sink=0,
                         n_recent=0, per_q_head=False, sm_scale=None):
    """Selections of request r against the oracle's (exact, or only near-tie
    differences), then its output: against the oracle's decode when every row
    matched, else against the oracle's attention over the GPU's own
    selection.  Returns the number of flagged rows."""
    rows = len(ref["sel"])
    flags = [compare_selection(sel_r[x], int(nsel_r[x]), ref["sel"][x], ref["scores"][x])
             for x in range(rows)]
    n_flag = flags.count("flagged")
    FLAGGED["requests_checked"] += 1
    if n_flag == 0:
        check_out(out_r, ref["out"], lay.w.torch_dtype, what)
        return 0
    FLAGGED["rows"] += n_flag
    FLAGGED["requests"] += 1
    sm = workloads.default_sm_scale(lay.w) if sm_scale is None else sm_scale
    qr = np.ascontiguousarray(to_oracle(q[r]))
    gpu_sel = [np.asarray(sel_r[x][:int(nsel_r[x])], np.int32) for x in range(rows)]
    ctx = int(lay.ctx[r])
    if per_q_head:
        want = oracle.request_attend_heads(lay.shape, qr, lay.host[0], lay.host[1],
                                           lay.pt_host[r], ctx, gpu_sel, sm)
    else:
        want = oracle.request_attend(lay.shape, qr, lay.host[0], lay.host[1], lay.pt_host[r],
                                     ctx, gpu_sel, sm)
    check_out(out_r, want, lay.w.torch_dtype, f"{what} (flagged rows {n_flag}: the oracle's "
              f"attention over the GPU selection)")
    log(f"{what}: {n_flag} flagged row(s), output checked over the GPU selection")
    return n_flag


def check_out(got, ref, dtype, what="output"):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    if err.size == 0:
        return 0.0
    assert err.max() <= 2e-2, f"{what}: max-abs {err.max():.3g} > 2e-2"
    assert err.mean() <= 2e-3, f"{what}: mean-abs {err.mean():.3g} > 2e-3"
    if dtype == torch.bfloat16:
        tol = 2.0 ** -8 * np.abs(ref) + 5e-4
    else:
        tol = 1e-5 * (1 + np.abs(ref))
    bad = err > tol
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond the internal bar, max {err.max():.3g}"
    return float(err.max())


# Reduced copies of the workloads (the oracle finishes them in seconds; they
# still span several tiles and a ragged tail), and edge workloads.
SMALL = {
    "tiny": WORKLOADS["tiny"],
    "layer32k_small": scaled(WORKLOADS["layer32k"], batch=3, ctx=4000, budget_tokens=512,
                             steps=3),
    "bench128k_small": scaled(WORKLOADS["bench128k"], batch=2, ctx=6000, budget_tokens=1024,
                              steps=3),
    "ragged_small": scaled(WORKLOADS["ragged"], batch=6, ctx_range=(40, 3000), steps=3),
    "layers48_small": scaled(WORKLOADS["layers48"], batch=3, ctx=2048, budget_tokens=256,
                             layers=2, steps=2),
    "edges": workloads.Workload("edges", 7, 16, 2, 128, 16, "bf16",
                                ctx_list=(0, 1, 15, 16, 17, 33, 700), budget_tokens=40,
                                poison=float("nan"), steps=2, seed=77),
    "edges_d64_p32": workloads.Workload("edges_d64_p32", 5, 12, 4, 64, 32, "bf16",
                                        ctx_list=(1, 31, 32, 65, 1000), budget_tokens=100,
                                        poison=float("nan"), steps=2, seed=78),
    "f32_g1": workloads.Workload("f32_g1", 2, 2, 2, 128, 32, "f32", ctx=2100,
                                 budget_tokens=300, steps=2, seed=79, permute_pages=True,
                                 poison=1e4),
    # groups wider than 8 q heads (every head column of the matrix-core tiles in use)
    "g16_p32": workloads.Workload("g16_p32", 3, 32, 2, 128, 32, "bf16", ctx=3000,
                                  budget_tokens=600, steps=2, seed=80, poison=float("nan")),
    "g12_d64": workloads.Workload("g12_d64", 2, 24, 2, 64, 16, "bf16", ctx_list=(500, 2000),
                                  budget_tokens=256, steps=2, seed=81, permute_pages=True),
    # 64-token pages (one page per wave and round in the decode)
    "p64_d128": workloads.Workload("p64_d128", 4, 32, 4, 128, 64, "bf16",
                                   ctx_list=(1, 64, 1000, 6001), budget_tokens=640, steps=2,
                                   seed=82, poison=float("nan"), permute_pages=True),
    "p64_d64_f32": workloads.Workload("p64_d64_f32", 2, 8, 2, 64, 64, "f32", ctx=2100,
                                      budget_tokens=500, steps=2, seed=83),
    # 8-token pages (two to a 16-token matrix-core tile in the decode); odd
    # page budgets leave the second half of a tile empty
    "p8_d128": workloads.Workload("p8_d128", 4, 32, 4, 128, 8, "bf16",
                                  ctx_list=(1, 9, 1001, 5003), budget_tokens=200, steps=2,
                                  seed=84, poison=float("nan"), permute_pages=True),
    "p8_d64": workloads.Workload("p8_d64", 3, 12, 4, 64, 8, "bf16", ctx_list=(7, 800, 3000),
                                 budget_tokens=88, steps=2, seed=85),
    "p8_f32": workloads.Workload("p8_f32", 2, 8, 2, 128, 8, "f32", ctx=700, budget_tokens=136,
                                 steps=2, seed=86),
}


def topk_rows(n_max, gen):
    """Score rows that reach every branch of the row selection."""
    rows = []
    rows.append(torch.randn(n_max, generator=gen))                           # distinct
    rows.append(torch.randint(0, 5, (n_max,), generator=gen).float())        # heavy ties
    rows.append(torch.full((n_max,), 3.25))                                  # all equal
    z = torch.zeros(n_max)
    z[::2] = -0.0
    z[::7] = -1.0
    rows.append(z)                                                           # signed zeros
    base = torch.ones(n_max)
    rows.append(torch.nextafter(base, base + 1) + (torch.arange(n_max) % 13) * 2 ** -23)
    thr = torch.full((n_max,), 5.0)                                          # > 64 tied keys
    thr[: n_max // 10] = 9.0 + torch.rand(n_max // 10, generator=gen)
    thr[n_max // 2:] = -torch.rand(n_max - n_max // 2, generator=gen)
    rows.append(thr[torch.randperm(n_max, generator=gen)])
    rows.append(torch.randn(n_max, generator=gen) * 1e30)                    # wide range
    rows.append(torch.randn(n_max, generator=gen) * 1e-3 + 100.0)            # narrow range
    low = torch.randn(n_max, generator=gen) + 30.0                          # low outliers
    low[torch.randperm(n_max, generator=gen)[: max(1, n_max // 500)]] = float("-inf")
    low[torch.randint(0, n_max, (2,), generator=gen)] = -1e30
    rows.append(low)
    top = torch.full((n_max,), 2.0)                      # most keys tied at the maximum
    top[torch.randperm(n_max, generator=gen)[: n_max // 8]] = \
        torch.randn(n_max // 8, generator=gen) - 4.0
    rows.append(top)
    return rows
