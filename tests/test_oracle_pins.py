"""Pins of the fp64 CPU oracle to facts other than itself.

Each pin checks the oracle against something it does not contain: a
hand-worked example (tests/golden/hand_example.json), brute force over tiny
inputs, closed forms, invariants that define min/max and the Quest bound, and
torch's own scaled_dot_product_attention in fp64 as the textbook attention.
``test_planted_mistakes_are_caught`` plants plausible mistakes into copies of
the oracle's C source (on the CPU) and shows every one of them fails a pin.
"""
from __future__ import annotations

import itertools
import json
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle
from helpers import pool_arrays, random_tokens, shape_of, store_request, to_f64, to_oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_example.json")
DTYPES = [torch.float32, torch.bfloat16]


def _npages(ctx, P):
    return -(-ctx // P)


def _request(gen, Hq, Hkv, D, P, ctx, dtype, permute=True, fill=1.0e4, extra_pool=3,
             k_scale=1.0):
    """One request in a pool: logical tokens, page table, pools, q."""
    n = _npages(ctx, P)
    pool = n + extra_pool
    s = shape_of(Hq, Hkv, D, P, pool, dtype)
    if permute:
        pt = torch.randperm(pool, generator=gen)[:max(n, 1)].to(torch.int32).numpy()
    else:
        pt = np.arange(max(n, 1), dtype=np.int32)
    k_tok = to_oracle(random_tokens(gen, ctx, Hkv, D, dtype, k_scale))
    v_tok = to_oracle(random_tokens(gen, ctx, Hkv, D, dtype))
    k_pool, v_pool = pool_arrays(s, fill)
    store_request(s, k_tok, v_tok, pt, k_pool, v_pool)
    q = to_oracle(torch.randn((Hq, D), generator=gen).to(dtype))
    return s, pt, k_tok, v_tok, k_pool, v_pool, q


# --------------------------------------------------------------------------
# hand-worked example
# --------------------------------------------------------------------------

def pin_hand_example(dtype):
    ex = json.load(open(GOLDEN))
    sh, exp = ex["shape"], ex["expected"]
    Hq, Hkv, D, P, ctx = (sh[k] for k in ("num_q_heads", "num_kv_heads", "head_dim",
                                          "page_size", "ctx"))
    s = shape_of(Hq, Hkv, D, P, 5, dtype)
    pt = np.array([3, 0, 4], np.int32)             # logical page j -> physical page
    k_tok = to_oracle(torch.tensor(ex["k_tokens"]).reshape(ctx, 1, D).to(dtype))
    v_tok = to_oracle(torch.tensor(ex["v_tokens"]).reshape(ctx, 1, D).to(dtype))
    q = to_oracle(torch.tensor(ex["q"]).to(dtype))
    k_pool, v_pool = pool_arrays(s, 1.0e4)
    store_request(s, k_tok, v_tok, pt, k_pool, v_pool)

    b = oracle.request_bounds(s, k_pool, pt, ctx)
    assert b[:, 0, 0, :].tolist() == exp["bounds_min"]
    assert b[:, 0, 1, :].tolist() == exp["bounds_max"]
    assert oracle.request_scores(s, q, b, "max")[0].tolist() == exp["scores_max"]
    assert oracle.request_scores(s, q, b, "sum")[0].tolist() == exp["scores_sum"]
    for h in range(Hq):     # each head alone: a one-head group
        s1 = shape_of(1, 1, D, P, 5, dtype)
        q1 = np.ascontiguousarray(q[h:h + 1])
        assert oracle.request_scores(s1, q1, b, "max")[0].tolist() == exp["head_scores"][h]
    smax = np.array(exp["scores_max"])
    for budget, want in exp["selection_by_budget"].items():
        k = oracle.pages_for_budget(int(budget), ctx, P)
        assert oracle.select(smax, k).tolist() == want, budget

    out = oracle.request_attend(s, q, k_pool, v_pool, pt, ctx, [np.array([0, 1])], 1.0)
    v = np.array(ex["v_tokens"])[exp["tokens_view_0_1"]]
    for h in range(Hq):
        logits = exp["logits_view_0_1"][h]
        w = [math.exp(x - max(logits)) for x in logits]
        want = sum(wi * vi for wi, vi in zip(w, v)) / sum(w)
        assert np.allclose(out[h], want, rtol=0, atol=1e-14), (h, out[h], want)


# --------------------------------------------------------------------------
# the KV store and the page bounds
# --------------------------------------------------------------------------

def pin_store_layout(dtype):
    gen = torch.Generator().manual_seed(11)
    P, D, Hkv, ctx = 4, 6, 2, 11
    s, pt, k_tok, v_tok, k_pool, v_pool, _ = _request(gen, 2, Hkv, D, P, ctx, dtype)
    written = np.zeros((s.pool, P), bool)
    for t in range(ctx):       # documented offsets: K [pool][Hkv][P][D], V [pool][Hkv][D][P]
        phys, slot = pt[t // P], t % P
        assert np.array_equal(k_pool[phys, :, slot, :], k_tok[t])
        assert np.array_equal(v_pool[phys, :, :, slot], v_tok[t])
        written[phys, slot] = True
    fill = to_oracle(torch.tensor([1.0e4]).to(dtype))[0]
    assert np.all(k_pool.transpose(0, 2, 1, 3)[~written] == fill)
    assert np.all(v_pool.transpose(0, 3, 1, 2)[~written] == fill)


def pin_store_incremental_equals_bulk(dtype):
    gen = torch.Generator().manual_seed(12)
    s, pt, k_tok, v_tok, k_bulk, v_bulk, _ = _request(gen, 4, 2, 8, 4, 19, dtype)
    k_inc, v_inc = pool_arrays(s, 1.0e4)
    for t in range(19):
        store_request(s, k_tok[t:t + 1], v_tok[t:t + 1], pt, k_inc, v_inc, pos0=t)
    assert k_inc.tobytes() == k_bulk.tobytes() and v_inc.tobytes() == v_bulk.tobytes()


def pin_bounds_contain_and_attain(dtype):
    """min/max are the unique values that bound every valid key and are each
    reached by one of them; never-written slots (poison) take no part."""
    gen = torch.Generator().manual_seed(13)
    for ctx in (1, 4, 5, 13, 16):
        P = 4
        s, pt, k_tok, _, k_pool, _, _ = _request(gen, 2, 2, 8, P, ctx, dtype)
        b = oracle.request_bounds(s, k_pool, pt, ctx)
        kf = to_f64(k_tok)
        assert b.shape[0] == _npages(ctx, P)
        for j in range(b.shape[0]):
            keys = kf[j * P:min((j + 1) * P, ctx)]            # [t][Hkv][D]
            lo, hi = b[j, :, 0, :], b[j, :, 1, :]
            assert np.all(keys >= lo) and np.all(keys <= hi)
            assert np.all(np.any(keys == lo, axis=0)) and np.all(np.any(keys == hi, axis=0))
        for j in range(b.shape[0]):
            assert np.array_equal(oracle.page_bounds(s, k_pool, pt, ctx, j), b[j])


def pin_bounds_keep_first_seen(dtype):
    """Among equal key values the bound keeps the one met first in position
    order (strict comparisons), which only shows in the sign of a zero: on
    one page, a channel whose keys are +0, -0, +0, -0 has bounds (+0, +0),
    one whose keys are -0, +0, -0, +0 has (-0, -0), and one with +0, -0, 1,
    -1 has min -1 and max 1."""
    P, D, Hkv = 4, 8, 1
    s = shape_of(Hkv, Hkv, D, P, 2, dtype)
    pt = np.array([1], dtype=np.int32)
    k = torch.ones((P, Hkv, D))
    k[:, 0, 0] = torch.tensor([0.0, -0.0, 0.0, -0.0])
    k[:, 0, 1] = torch.tensor([-0.0, 0.0, -0.0, 0.0])
    k[:, 0, 2] = torch.tensor([0.0, -0.0, 1.0, -1.0])
    k_tok = to_oracle(k.to(dtype))
    v_tok = to_oracle(torch.zeros((P, Hkv, D)).to(dtype))
    k_pool, v_pool = pool_arrays(s, 7.0)
    store_request(s, k_tok, v_tok, pt, k_pool, v_pool)
    b = oracle.request_bounds(s, k_pool, pt, P)[0, 0]           # [2][D]
    assert b[0, 0] == 0 and not np.signbit(b[0, 0]) and b[1, 0] == 0 and not np.signbit(b[1, 0])
    assert b[0, 1] == 0 and np.signbit(b[0, 1]) and b[1, 1] == 0 and np.signbit(b[1, 1])
    assert b[0, 2] == -1.0 and b[1, 2] == 1.0
    assert np.all(b[:, 3:] == 1.0)


# --------------------------------------------------------------------------
# page scores
# --------------------------------------------------------------------------

def pin_score_is_box_maximum(dtype):
    """With one q head per KV head, a page's score is the largest q.x over the
    box [min, max] -- brute force over its 2^D corners."""
    gen = torch.Generator().manual_seed(21)
    D, P, ctx, H = 5, 4, 14, 3
    s, pt, _, _, k_pool, _, q = _request(gen, H, H, D, P, ctx, dtype)
    b = oracle.request_bounds(s, k_pool, pt, ctx)
    sc = oracle.request_scores(s, q, b, "max")
    qf = to_f64(q)
    for g in range(H):
        for j in range(b.shape[0]):
            best = -math.inf
            for corner in itertools.product((0, 1), repeat=D):
                x = [b[j, g, c, d] for d, c in enumerate(corner)]
                best = max(best, sum(qf[g, d] * x[d] for d in range(D)))
            assert abs(sc[g, j] - best) <= 1e-12 * (1 + abs(best)), (g, j)


def pin_score_bounds_every_key(dtype):
    """The group score is at least q_h.k_t for every q head h of the group and
    every valid key t of the page; single-token pages reach it exactly."""
    gen = torch.Generator().manual_seed(22)
    Hq, Hkv, D, P = 8, 2, 16, 4
    for ctx in (17, 20):                                    # last page: 1 token, then full
        s, pt, k_tok, _, k_pool, _, q = _request(gen, Hq, Hkv, D, P, ctx, dtype,
                                                 k_scale=3.0)
        b = oracle.request_bounds(s, k_pool, pt, ctx)
        sc = oracle.request_scores(s, q, b, "max")
        kf, qf = to_f64(k_tok), to_f64(q)
        G = Hq // Hkv
        for g in range(Hkv):
            heads = qf[g * G:(g + 1) * G]                   # q heads h with h // G == g
            for j in range(b.shape[0]):
                keys = kf[j * P:min((j + 1) * P, ctx), g]    # [t][D]
                dots = heads @ keys.T                        # [G][t]
                slack = 1e-12 * (np.abs(heads) @ np.abs(keys).T).max()
                assert sc[g, j] >= dots.max() - slack
                if keys.shape[0] == 1:
                    assert abs(sc[g, j] - dots.max()) <= slack


def pin_score_closed_forms(dtype):
    gen = torch.Generator().manual_seed(23)
    D, P, ctx, H = 16, 4, 12, 2
    s, pt, _, _, k_pool, _, q = _request(gen, H, H, D, P, ctx, dtype)
    b = oracle.request_bounds(s, k_pool, pt, ctx)
    qpos = np.ascontiguousarray(to_oracle(torch.from_numpy(np.abs(to_f64(q))).to(
        torch.float32 if dtype == torch.float32 else torch.bfloat16)))
    sc = oracle.request_scores(s, qpos, b, "max")
    want = np.einsum("gd,jgd->gj", to_f64(qpos), b[:, :, 1, :])   # q >= 0: q . max
    assert np.allclose(sc, want, rtol=1e-13, atol=1e-13)
    qneg = np.ascontiguousarray(to_oracle(torch.from_numpy(-np.abs(to_f64(q))).to(
        torch.float32 if dtype == torch.float32 else torch.bfloat16)))
    sc = oracle.request_scores(s, qneg, b, "max")
    want = np.einsum("gd,jgd->gj", to_f64(qneg), b[:, :, 0, :])   # q <= 0: q . min
    assert np.allclose(sc, want, rtol=1e-13, atol=1e-13)
    zero = np.zeros_like(q)
    assert np.all(oracle.request_scores(s, zero, b, "max") == 0.0)


def pin_group_reduce(dtype):
    """A group's score is the max (or sum) of its q heads' own scores, where q
    head h reads KV head h // G.  Each head's own score comes from a pool with
    one KV head per q head (KV head h // G copied to slot h)."""
    gen = torch.Generator().manual_seed(24)
    Hq, Hkv, D, P, ctx = 8, 2, 8, 4, 15
    G = Hq // Hkv
    s, pt, _, _, k_pool, v_pool, q = _request(gen, Hq, Hkv, D, P, ctx, dtype)
    b = oracle.request_bounds(s, k_pool, pt, ctx)
    s1 = shape_of(Hq, Hq, D, P, s.pool, dtype)
    k1 = np.ascontiguousarray(np.repeat(k_pool, G, axis=1))
    per_head = oracle.request_scores(s1, q, oracle.request_bounds(s1, k1, pt, ctx), "max")
    grouped = per_head.reshape(Hkv, G, -1)
    assert np.array_equal(oracle.request_scores(s, q, b, "max"), grouped.max(axis=1))
    assert np.allclose(oracle.request_scores(s, q, b, "sum"), grouped.sum(axis=1),
                       rtol=1e-13, atol=1e-12)


def pin_per_head_selection(dtype):
    """Per-q-head selection reduces to the pinned grouped path on a pool with
    one KV head per q head (KV head h // G copied to slot h, G = 1 there):
    each head's own scores are that pool's group scores, and attention with
    one page list per q head is that pool's attention with the same lists."""
    gen = torch.Generator().manual_seed(25)
    Hq, Hkv, D, P, ctx = 8, 2, 8, 4, 37
    G = Hq // Hkv
    s, pt, _, _, k_pool, v_pool, q = _request(gen, Hq, Hkv, D, P, ctx, dtype)
    b = oracle.request_bounds(s, k_pool, pt, ctx)
    s1 = shape_of(Hq, Hq, D, P, s.pool, dtype)
    k1 = np.ascontiguousarray(np.repeat(k_pool, G, axis=1))
    v1 = np.ascontiguousarray(np.repeat(v_pool, G, axis=1))
    b1 = oracle.request_bounds(s1, k1, pt, ctx)
    heads = oracle.request_head_scores(s, q, b)
    assert np.array_equal(heads, oracle.request_scores(s1, q, b1, "max"))
    for budget in (4, 13, 40):
        r = oracle.decode_request(s, q, k_pool, v_pool, pt, ctx, budget, 0.3, per_q_head=True)
        k = oracle.pages_for_budget(budget, ctx, P)
        assert len(r["sel"]) == Hq
        assert all(np.array_equal(r["sel"][h], oracle.select(heads[h], k)) for h in range(Hq))
        want = oracle.request_attend(s1, q, k1, v1, pt, ctx, r["sel"], 0.3)
        assert np.array_equal(r["out"], want)
    # with every page selected, per-head and shared selection are both dense
    full = oracle.decode_request(s, q, k_pool, v_pool, pt, ctx, 10 ** 6, 0.3, per_q_head=True)
    assert np.array_equal(full["out"],
                          oracle.request_dense(s, q, k_pool, v_pool, pt, ctx, 0.3))


# --------------------------------------------------------------------------
# budget and selection
# --------------------------------------------------------------------------

def pin_budget_table():
    # (budget tokens, ctx, page size) -> pages
    table = [((256, 1024, 16), 16), ((4096, 128001, 16), 256), ((0, 100, 16), 1),
             ((15, 100, 16), 1), ((16, 100, 16), 1), ((32, 100, 16), 2),
             ((47, 100, 16), 2), ((10000, 100, 16), 7), ((5, 0, 16), 0),
             ((17, 1, 16), 1), ((64, 33, 32), 2), ((96, 33, 32), 2)]
    for args, want in table:
        assert oracle.pages_for_budget(*args) == want, args


def pin_select_bruteforce():
    rng = np.random.default_rng(31)
    for n in (1, 2, 5, 17, 64, 200):
        for levels in (3, 1000):                     # many ties, few ties
            scores = rng.integers(0, levels, n).astype(np.float64) - levels / 2
            for k in sorted({0, 1, n // 3, n // 2, n - 1, n} - {-1}):
                if k < 0:
                    continue
                want = sorted(sorted(range(n), key=lambda j: (-scores[j], j))[:k])
                assert oracle.select(scores, k).tolist() == want, (n, levels, k)
    assert oracle.select(np.zeros(9), 4).tolist() == [0, 1, 2, 3]      # all equal
    assert oracle.select(np.array([0.0, -0.0, 0.0, -1.0]), 2).tolist() == [0, 1]
    assert oracle.select(np.array([-0.0, 0.0, 5.0]), 2).tolist() == [0, 2]


def pin_select_forced():
    """Forced sink / recent pages reduce to the pinned plain selection: with
    none forced it is the plain selection; when k covers the forced set F, the
    result is F plus the plain selection of k - |F| pages among the others;
    otherwise the k lowest pages of F."""
    rng = np.random.default_rng(37)
    for n in (1, 3, 10, 64, 200):
        for levels in (3, 1000):
            scores = rng.integers(0, levels, n).astype(np.float64) - levels / 2
            for ns, nr in ((0, 0), (1, 0), (0, 1), (1, 1), (2, 3), (n, 0), (0, n + 2), (5, 5)):
                forced = [j for j in range(n) if j < ns or j >= n - nr]
                rest = [j for j in range(n) if not (j < ns or j >= n - nr)]
                for k in sorted({0, 1, len(forced) - 1, len(forced), len(forced) + 1,
                                 n // 2, n}):
                    if not 0 <= k <= n:
                        continue
                    got = oracle.select(scores, k, ns, nr).tolist()
                    if k <= len(forced):
                        want = forced[:k]
                    else:
                        sub = oracle.select(scores[rest], k - len(forced)).tolist()
                        want = sorted(forced + [rest[i] for i in sub])
                    assert got == want, (n, levels, ns, nr, k)
            if n > 2:
                # a forced page outranks even the best scored page
                best = int(np.argmax(scores[1:])) + 1
                assert oracle.select(scores, 1, 1, 0).tolist() == [0], best


# --------------------------------------------------------------------------
# attention over the selected view
# --------------------------------------------------------------------------

def _sdpa(qf, kf, vf, allowed, scale):
    """torch's fp64 scaled_dot_product_attention of one request.
    qf [Hq][D], kf/vf [ctx][Hkv][D], allowed bool [Hkv][ctx]."""
    Hq, Hkv = qf.shape[0], kf.shape[1]
    G = Hq // Hkv
    qt = torch.from_numpy(qf)[None, :, None, :]
    kt = torch.from_numpy(kf).permute(1, 0, 2)[None].repeat_interleave(G, dim=1).contiguous()
    vt = torch.from_numpy(vf).permute(1, 0, 2)[None].repeat_interleave(G, dim=1).contiguous()
    mask = torch.from_numpy(allowed).repeat_interleave(G, dim=0)[None, :, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                           scale=scale)
    return out[0, :, 0, :].numpy()


def pin_dense_equals_sdpa(dtype):
    gen = torch.Generator().manual_seed(41)
    Hq, Hkv, D, P, ctx = 8, 2, 16, 4, 23
    s, pt, k_tok, v_tok, k_pool, v_pool, q = _request(gen, Hq, Hkv, D, P, ctx, dtype)
    scale = 1 / math.sqrt(D)
    out = oracle.request_dense(s, q, k_pool, v_pool, pt, ctx, scale)
    want = _sdpa(to_f64(q), to_f64(k_tok), to_f64(v_tok), np.ones((Hkv, ctx), bool), scale)
    assert np.allclose(out, want, rtol=0, atol=1e-13)


def pin_sparse_equals_masked_sdpa(dtype):
    gen = torch.Generator().manual_seed(42)
    rng = np.random.default_rng(42)
    Hq, Hkv, D, P, ctx = 8, 2, 16, 4, 23
    s, pt, k_tok, v_tok, k_pool, v_pool, q = _request(gen, Hq, Hkv, D, P, ctx, dtype)
    n = _npages(ctx, P)
    sel = [np.sort(rng.choice(n, size=k, replace=False)) for k in (2, 5)]
    sel[1][-1] = n - 1                                  # include the partial page
    sel[1] = np.unique(sel[1])
    allowed = np.zeros((Hkv, ctx), bool)
    for g in range(Hkv):
        for j in sel[g]:
            allowed[g, j * P:min((j + 1) * P, ctx)] = True
    scale = 0.3
    out = oracle.request_attend(s, q, k_pool, v_pool, pt, ctx, sel, scale)
    want = _sdpa(to_f64(q), to_f64(k_tok), to_f64(v_tok), allowed, scale)
    assert np.allclose(out, want, rtol=0, atol=1e-13)


def pin_attention_closed_forms(dtype):
    gen = torch.Generator().manual_seed(43)
    Hq, Hkv, D, P, ctx = 4, 2, 8, 4, 9                  # last page holds token 8 only
    s, pt, k_tok, v_tok, k_pool, v_pool, q = _request(gen, Hq, Hkv, D, P, ctx, dtype)
    vf = to_f64(v_tok)
    zero = np.zeros_like(q)
    sel = [np.array([0, 2]), np.array([1])]
    out = oracle.request_attend(s, zero, k_pool, v_pool, pt, ctx, sel, 0.5)
    assert np.allclose(out[0], vf[[0, 1, 2, 3, 8], 0].mean(0), atol=1e-15)   # q = 0: mean of v
    assert np.allclose(out[3], vf[4:8, 1].mean(0), atol=1e-15)
    out = oracle.request_attend(s, q, k_pool, v_pool, pt, ctx, [np.array([2]), np.array([2])],
                                0.5)
    assert np.array_equal(out[0], vf[8, 0]) and np.array_equal(out[3], vf[8, 1])  # one token
    # identical keys: uniform weights whatever q is
    same = np.repeat(k_tok[:1], ctx, axis=0)
    k_same, v_same = pool_arrays(s, 1.0e4)
    store_request(s, same, v_tok, pt, k_same, v_same)
    out = oracle.request_attend(s, q, k_same, v_same, pt, ctx, sel, 0.7)
    assert np.allclose(out[1], vf[[0, 1, 2, 3, 8], 0].mean(0), atol=1e-14)
    # a head whose view is empty outputs zeros
    out = oracle.request_attend(s, q, k_pool, v_pool, pt, ctx, [np.array([], np.int32),
                                                                np.array([1])], 0.5)
    assert np.all(out[:2] == 0.0)


def pin_permutation_invariance(dtype):
    """Moving physical pages (and the page table with them) changes nothing."""
    gen = torch.Generator().manual_seed(44)
    Hq, Hkv, D, P, ctx = 8, 2, 16, 4, 30
    s, pt, k_tok, v_tok, k_pool, v_pool, q = _request(gen, Hq, Hkv, D, P, ctx, dtype,
                                                      permute=False)
    pt2 = torch.randperm(s.pool, generator=gen)[:pt.size].to(torch.int32).numpy()
    k2, v2 = pool_arrays(s, -7.0)
    store_request(s, k_tok, v_tok, pt2, k2, v2)
    a = oracle.decode_request(s, q, k_pool, v_pool, pt, ctx, 12, 0.25)
    b = oracle.decode_request(s, q, k2, v2, pt2, ctx, 12, 0.25)
    assert np.array_equal(a["scores"], b["scores"])
    assert all(np.array_equal(x, y) for x, y in zip(a["sel"], b["sel"]))
    assert np.array_equal(a["out"], b["out"])


def pin_budget_covering_all_is_dense(dtype):
    gen = torch.Generator().manual_seed(45)
    Hq, Hkv, D, P, ctx = 8, 2, 16, 4, 21
    s, pt, _, _, k_pool, v_pool, q = _request(gen, Hq, Hkv, D, P, ctx, dtype)
    scale = 1 / math.sqrt(D)
    dense = oracle.request_dense(s, q, k_pool, v_pool, pt, ctx, scale)
    for budget in (ctx, 4 * P * ctx):
        r = oracle.decode_request(s, q, k_pool, v_pool, pt, ctx, budget + P, scale)
        assert r["k"] == _npages(ctx, P)
        assert np.allclose(r["out"], dense, rtol=0, atol=1e-15)


PINS = [
    pin_hand_example, pin_store_layout, pin_store_incremental_equals_bulk,
    pin_bounds_contain_and_attain, pin_bounds_keep_first_seen, pin_score_is_box_maximum,
    pin_score_bounds_every_key,
    pin_score_closed_forms, pin_group_reduce, pin_per_head_selection, pin_budget_table,
    pin_select_bruteforce, pin_select_forced,
    pin_dense_equals_sdpa, pin_sparse_equals_masked_sdpa, pin_attention_closed_forms,
    pin_permutation_invariance, pin_budget_covering_all_is_dense,
]


def _run(pin, dtype):
    import inspect
    if "dtype" in inspect.signature(pin).parameters:
        pin(dtype)
    else:
        pin()


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "bf16"])
@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin, dtype):
    _run(pin, dtype)


# --------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin
# --------------------------------------------------------------------------

MUTANTS = {
    "bound drops the max (always q*max)": ("u += (a > b ? a : b);", "u += b;"),
    "bound takes the min": ("u += (a > b ? a : b);", "u += (a < b ? a : b);"),
    "strided GQA groups": ("for (int32_t h = g * G; h < (g + 1) * G; ++h) {",
                           "for (int32_t h = g; h < Hq; h += H) {"),
    "group max keeps the last head": ("score = (u > score ? u : score);", "score = u;"),
    "ties to the higher page": ("return (a->page > b->page) - (a->page < b->page);",
                                "return (a->page < b->page) - (a->page > b->page);"),
    "selection left in score order": (
        "qsort(sel, (size_t)k, sizeof(int32_t), ascending_int);", ""),
    "bounds read stale slots": ("const int32_t last = (first + P < ctx ? first + P : ctx);",
                                "const int32_t last = first + P;"),
    "bounds keep the last-seen of equal values": ("if (x < lo) lo = x;", "if (x <= lo) lo = x;"),
    "min and max swapped": ("bounds_j[((int64_t)g * 2 + 0) * D + d] = lo;",
                            "bounds_j[((int64_t)g * 2 + 0) * D + d] = hi; (void)lo;"),
    "budget rounds up": ("int32_t k = budget_tokens / page_size;",
                         "int32_t k = (budget_tokens + page_size - 1) / page_size;"),
    "attention reads stale slots": ("if (j * P + slot >= ctx) break;", ""),
    "V read token-major": ("return ((phys * s->num_kv_heads + g) * s->head_dim + d) *\n"
                           "             (int64_t)s->page_size + slot;",
                           "return ((phys * s->num_kv_heads + g) * s->page_size + slot) *\n"
                           "             (int64_t)s->head_dim + d;"),
    "attention uses KV head h mod Hkv": ("const int32_t g = h / (s->num_q_heads / H);",
                                         "const int32_t g = h % H;"),
    "softmax denominator without the max shift": ("denom += exp(logit[t] - m);",
                                                  "denom += exp(logit[t]);"),
    "store drops the page table": ("const int64_t phys = pt_row[pos / P];",
                                   "const int64_t phys = pos / P;"),
    "recent pages counted from the front": ("return j < n_sink || j >= n - n_recent;",
                                            "return j < n_sink || j < n_recent;"),
    "forced pages not ranked first": ("if (a->forced != b->forced) return a->forced ? -1 : 1;",
                                      ""),
    "head scores read KV head h mod Hkv": ("const int32_t kvh = h / G;",
                                           "const int32_t kvh = h % H;"),
    "per-head attention uses the group's first list": (
        "sel + (int64_t)h * sel_stride,",
        "sel + (int64_t)(h - h % (s->num_q_heads / s->num_kv_heads)) * sel_stride,"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistakes_are_caught(name, mutant_dir):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    tag = "m%02d" % list(MUTANTS).index(name)
    c_path = mutant_dir / f"{tag}.c"
    so_path = mutant_dir / f"{tag}.so"
    c_path.write_text(src.replace(old, new))
    shutil.copy(os.path.join(os.path.dirname(oracle.SOURCE), "quest_oracle.h"),
                mutant_dir / "quest_oracle.h")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", str(c_path), "-o",
                    str(so_path), "-lm"], check=True)
    saved = oracle._lib
    oracle._lib = oracle.load(str(so_path))
    caught = []
    try:
        for pin in PINS:
            for dtype in DTYPES:
                try:
                    _run(pin, dtype)
                except (AssertionError, ValueError) as e:  # noqa: PERF203
                    caught.append(f"{pin.__name__}[{dtype}]: {type(e).__name__}")
                    break
    finally:
        oracle._lib = saved
    assert caught, f"planted mistake '{name}' passed every pin"
