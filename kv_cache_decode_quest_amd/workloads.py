"""Seeded synthetic workloads for Quest sparse decode.

This module only draws inputs and lays out the page pool: random q/K/V, page
tables, context lengths and token budgets.  It holds none of the method's
arithmetic (no bounds, scores, selection or attention), so both the HIP path
and the CPU oracle can take their inputs from it.

The five workloads follow the serving shapes the pages benchmark: the
Sparse-vLLM skill page's Validation section runs 128000-token contexts at
batch 8 with 128 output tokens on one GPU, and the SparseEngine digest's key
results use Qwen3-30B-A3B-class attention (32 q heads, 4 KV heads, head dim
128).  Values are N(0, 1) drawn in fp32 from a seeded torch generator on the
requested device and rounded to bf16 (round to nearest even) where the
workload is bf16.  No dataset or trained weight is involved: the synthetic
tensors stand in for the long-context serving traces the pages measure.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str                      # "f32" or "bf16"
    ctx: int = 0                    # fixed context per request (if ctx_range is None)
    ctx_range: tuple | None = None  # inclusive uniform range for ragged batches
    ctx_list: tuple | None = None   # explicit per-request lengths (edge cases)
    budget_tokens: int = 0          # fixed token budget per request ...
    budget_page_div: int = 0        # ... or max(1, n_pages // div) whole pages
    steps: int = 1                  # decode steps, one appended token per request each
    layers: int = 1                 # independent attention layers (own pool each)
    permute_pages: bool = False     # physical pages randomly permuted in a shared pool
    outlier_channels: int = 0       # K channels per (layer, KV head) scaled up
    outlier_scale: float = 1.0
    poison: float | None = None     # fill for never-written slots (None: zeros)
    seed: int = 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads


WORKLOADS = {
    # 1 request, 4 q / 1 KV head, D 64, P 16, 1024 tokens (64 pages), budget 256, fp32.
    "tiny": Workload("tiny", 1, 4, 1, 64, 16, "f32", ctx=1024, budget_tokens=256,
                     seed=1001),
    # One Qwen3-30B-A3B-like attention layer: 32 q / 4 KV heads, D 128, P 16,
    # batch 8 at 32768 tokens, budget 2048, one decode step.
    "layer32k": Workload("layer32k", 8, 32, 4, 128, 16, "bf16", ctx=32768,
                         budget_tokens=2048, seed=1002),
    # The benchmark shape: batch 8 at 128000 tokens, budget 4096, 128 steps.
    "bench128k": Workload("bench128k", 8, 32, 4, 128, 16, "bf16", ctx=128000,
                          budget_tokens=4096, steps=128, seed=1003),
    # Ragged batch: 32 requests with contexts uniform in [4096, 131072], P 32,
    # budget 10% of each request's pages, partial last pages, pages permuted.
    "ragged": Workload("ragged", 32, 32, 4, 128, 32, "bf16", ctx_range=(4096, 131072),
                       budget_page_div=10, permute_pages=True, poison=1.0e4,
                       seed=1004),
    # Full 48-layer decode step at batch 64 x 32k, budget 2048, with 4 K
    # outlier channels per (layer, KV head) scaled x10.
    "layers48": Workload("layers48", 64, 32, 4, 128, 16, "bf16", ctx=32768,
                         budget_tokens=2048, layers=48, outlier_channels=4,
                         outlier_scale=10.0, seed=1005),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (smaller test sizes)."""
    return dataclasses.replace(w, **changes)


def generator(w: Workload, device, layer: int, stream: int) -> torch.Generator:
    """Independent generator for one (layer, purpose) of a workload."""
    g = torch.Generator(device=device)
    g.manual_seed(w.seed + 1000 * layer + 1_000_003 * stream)
    return g


# purpose ids for generator streams
_LAYOUT, _PREFILL_K, _PREFILL_V, _OUTLIERS = 0, 1, 2, 3


def _step_stream(step: int, which: int) -> int:
    return 16 + 3 * step + which


def normal(shape, w: Workload, gen: torch.Generator, device) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(w.torch_dtype)


def pages_of(ctx, page_size):
    return (ctx + page_size - 1) // page_size


@dataclass
class Layout:
    """Request lengths and the paged pool's page table for one layer."""
    ctx0: torch.Tensor          # int32 [B], context before the first decode step
    page_table: torch.Tensor    # int32 [B][max_pages]
    num_pool_pages: int
    max_pages: int


def context_lengths(w: Workload) -> torch.Tensor:
    """int32 [B] on the CPU: prompt lengths (seeded for ragged workloads)."""
    if w.ctx_list is not None:
        assert len(w.ctx_list) == w.batch
        return torch.tensor(w.ctx_list, dtype=torch.int32)
    if w.ctx_range is None:
        return torch.full((w.batch,), w.ctx, dtype=torch.int32)
    lo, hi = w.ctx_range
    g = generator(w, "cpu", 0, _LAYOUT)
    return torch.randint(lo, hi + 1, (w.batch,), generator=g, dtype=torch.int64).to(torch.int32)


def make_layout(w: Workload, device, capacity_tokens: int | None = None) -> Layout:
    """Page table with room for ``capacity_tokens`` extra tokens per request
    (default: the workload's decode steps).  Pages are contiguous per request,
    or a seeded random permutation of one shared pool."""
    extra = w.steps if capacity_tokens is None else capacity_tokens
    ctx0 = context_lengths(w)
    need = [pages_of(int(c) + extra, w.page_size) for c in ctx0.tolist()]
    max_pages = max(need) if need else 1
    pool = sum(need)
    if w.permute_pages:
        g = generator(w, "cpu", 0, _LAYOUT)
        order = torch.randperm(max(pool, 1), generator=g)[:pool].to(torch.int32)
    else:
        order = torch.arange(pool, dtype=torch.int32)
    table = torch.zeros((w.batch, max_pages), dtype=torch.int32)
    start = 0
    for r, n in enumerate(need):
        table[r, :n] = order[start:start + n]
        start += n
    return Layout(ctx0.to(device), table.to(device), max(pool, 1), max_pages)


def budget_tokens(w: Workload, ctx_lens: torch.Tensor) -> torch.Tensor:
    """int32 [B] token budgets for the given context lengths."""
    if w.budget_page_div > 0:
        n = pages_of(ctx_lens.to(torch.int64), w.page_size)
        k = torch.clamp(n // w.budget_page_div, min=1)
        return (k * w.page_size).to(torch.int32)
    return torch.full_like(ctx_lens, w.budget_tokens, dtype=torch.int32)


def empty_pool(w: Workload, layout: Layout, device):
    """K pool [pool][Hkv][P][D] and V pool [pool][Hkv][D][P], filled with the
    workload's poison value (or zeros) so unwritten slots hold junk."""
    kshape = (layout.num_pool_pages, w.num_kv_heads, w.page_size, w.head_dim)
    vshape = (layout.num_pool_pages, w.num_kv_heads, w.head_dim, w.page_size)
    fill = 0.0 if w.poison is None else w.poison
    k = torch.full(kshape, fill, dtype=w.torch_dtype, device=device)
    v = torch.full(vshape, fill, dtype=w.torch_dtype, device=device)
    return k, v


def outlier_scale(w: Workload, layer: int, device) -> torch.Tensor | None:
    """fp32 [Hkv][D] per-channel multipliers for K (None when unused)."""
    if w.outlier_channels <= 0:
        return None
    g = generator(w, "cpu", layer, _OUTLIERS)
    s = torch.ones((w.num_kv_heads, w.head_dim), dtype=torch.float32)
    for h in range(w.num_kv_heads):
        ch = torch.randperm(w.head_dim, generator=g)[:w.outlier_channels]
        s[h, ch] = w.outlier_scale
    return s.to(device)


def _keys(shape, w, gen, device, scale):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if scale is not None:
        x = x * scale
    return x.to(w.torch_dtype)


def prefill_tokens(w: Workload, layout: Layout, device, layer: int = 0):
    """The prompt KV of every request as new tokens for one bulk append:
    k_new, v_new [T][Hkv][D], cu_new int32 [B+1], ctx_before int32 [B] (zeros)."""
    ctx = layout.ctx0.to("cpu").to(torch.int64)
    cu = torch.zeros(w.batch + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(ctx, 0)
    T = int(cu[-1])
    scale = outlier_scale(w, layer, device)
    k = _keys((T, w.num_kv_heads, w.head_dim), w, generator(w, device, layer, _PREFILL_K),
              device, scale)
    v = normal((T, w.num_kv_heads, w.head_dim), w, generator(w, device, layer, _PREFILL_V),
               device)
    zeros = torch.zeros(w.batch, dtype=torch.int32, device=device)
    return k, v, cu.to(torch.int32).to(device), zeros


def step_tokens(w: Workload, device, layer: int, step: int):
    """Decode step inputs: q [B][Hq][D], k_new, v_new [B][Hkv][D]."""
    q = normal((w.batch, w.num_q_heads, w.head_dim), w,
               generator(w, device, layer, _step_stream(step, 0)), device)
    k = _keys((w.batch, w.num_kv_heads, w.head_dim), w,
              generator(w, device, layer, _step_stream(step, 1)), device,
              outlier_scale(w, layer, device))
    v = normal((w.batch, w.num_kv_heads, w.head_dim), w,
               generator(w, device, layer, _step_stream(step, 2)), device)
    return q, k, v


def default_sm_scale(w: Workload) -> float:
    return 1.0 / math.sqrt(w.head_dim)
