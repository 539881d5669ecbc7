"""A seeded sweep over the options the library takes, each configuration
checked end to end against the oracle on the GPU.

Every configuration is one decode step (the fused append + scores, then the
top-k and the decode, through the two calls or the combined one) on a small
random pool: head dim 64 / 128, page sizes 8 to 64, GQA groups 1 to 16,
bf16 and fp32, selection per KV head or per q head, MAX or SUM group
reduction, forced sink / recent pages, permuted physical pages, NaN-poisoned
unwritten slots, and request lengths from 0 up.  The bar is the one of
tests/parity.py: metadata exact, selections bit-exact (rows differing only
by near-tied pages are flagged), outputs within tolerance.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from helpers import to_f64, to_oracle
from kv_cache_decode_quest_amd import quest, workloads
from parity import Layer, check_kmeta, check_request_output, log

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

SHAPES = [(64, 8), (64, 16), (64, 32), (64, 64), (128, 8), (128, 16), (128, 32), (128, 64)]
GROUPS = [(4, 4), (8, 1), (16, 2), (24, 2), (32, 4), (12, 1), (16, 16)]      # (Hq, Hkv)
FORCED = [(0, 0), (1, 0), (0, 2), (1, 2)]


def sweep_configs(n=32, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D, P = SHAPES[i % len(SHAPES)]
        Hq, Hkv = GROUPS[int(rng.integers(len(GROUPS)))]
        dtype = "f32" if i % 6 == 5 else "bf16"
        if dtype == "f32" and P == 64:
            D = 64                                  # fp32 64-token pages need D = 64
        B = int(rng.integers(1, 4))
        ctx = [int(x) for x in rng.integers(0, 2600, size=B)]
        if i % 5 == 0:
            ctx[0] = 0                              # an empty request
        if i % 7 == 1:
            ctx[-1] = 1
        budget = int(rng.choice([P, 3 * P, 128, 300, 1000]))
        cfg = dict(i=i, D=D, P=P, Hq=Hq, Hkv=Hkv, dtype=dtype, B=B, ctx=tuple(ctx),
                   budget=budget, per_q_head=i % 4 == 3,
                   forced=FORCED[i % 4] if i % 3 == 0 else (0, 0),
                   reduce="sum" if i % 5 == 4 else "max", combined=i % 2 == 1,
                   permute=i % 3 == 1, poison=float("nan") if i % 4 == 2 else None,
                   seed=9000 + i)
        cfg["name"] = (f"c{i}_d{D}_p{P}_g{Hq}x{Hkv}_{dtype}_b{B}"
                       f"{'_qh' if cfg['per_q_head'] else ''}"
                       f"{'_f%d%d' % cfg['forced'] if any(cfg['forced']) else ''}"
                       f"_{cfg['reduce']}{'_one' if cfg['combined'] else '_two'}")
        out.append(cfg)
    return out


CONFIGS = sweep_configs()


@pytest.mark.parametrize("cfg", CONFIGS, ids=[c["name"] for c in CONFIGS])
def test_sweep_matches_oracle(cfg, gpu_lib):
    w = workloads.Workload(cfg["name"], cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["P"],
                           cfg["dtype"], ctx_list=cfg["ctx"], budget_tokens=cfg["budget"],
                           steps=1, seed=cfg["seed"], permute_pages=cfg["permute"],
                           poison=cfg["poison"])
    log(f"{cfg['name']}: ctx {cfg['ctx']}, budget {cfg['budget']}")
    lay = Layer(w, DEV)
    if cfg["per_q_head"]:
        lay.L = quest.make_layout(w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                                  w.torch_dtype, lay.lay.num_pool_pages, lay.lay.max_pages,
                                  per_q_head=True)
    ns, nr = cfg["forced"]
    sm = workloads.default_sm_scale(w)
    q, k_new, v_new = lay.step_inputs(0)
    bufs = lay.buffers(extra=1)
    lay.append_score_step(q, k_new, v_new, bufs, cfg["reduce"], topk=False)
    if cfg["combined"]:
        quest.quest_topk_sparse_decode(lay.L, q, lay.k_cache, lay.v_cache, lay.pt, lay.ctx,
                                       bufs.scores, lay.budgets(), bufs.max_k, sm,
                                       bufs.sel_pages, bufs.num_sel, bufs.out, bufs.workspace,
                                       ns, nr)
    else:
        quest.quest_topk_pages_forced(lay.L, bufs.scores, lay.ctx, lay.budgets(), bufs.max_k,
                                      ns, nr, bufs.sel_pages, bufs.num_sel)
        lay.attend(q, bufs)
    torch.cuda.synchronize()
    km = to_f64(lay.kmeta)
    sel, nsel = bufs.sel_pages.cpu().numpy(), bufs.num_sel.cpu().numpy()
    out = to_f64(bufs.out)
    flagged = 0
    for r in range(w.batch):
        ctx = int(lay.ctx[r])
        ref = oracle.decode_request(lay.shape, np.ascontiguousarray(to_oracle(q[r])),
                                    lay.host[0], lay.host[1], lay.pt_host[r], ctx,
                                    int(lay.budgets()[r]), sm, cfg["reduce"], n_sink=ns,
                                    n_recent=nr, per_q_head=cfg["per_q_head"])
        if ctx:
            check_kmeta(lay, r, ref["bounds"], km)
        flagged += check_request_output(lay, q, r, sel[r], nsel[r], out[r], ref,
                                        f"{cfg['name']} r{r}", per_q_head=cfg["per_q_head"])
        if ctx == 0:
            assert np.all(nsel[r] == 0) and np.all(out[r] == 0.0)
    log(f"{cfg['name']}: ok, flagged rows {flagged}")
