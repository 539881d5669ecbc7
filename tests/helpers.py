"""Shared test plumbing: tensor conversion and pool construction.

Holds no Quest arithmetic; expected values always come from the oracle (or,
for the oracle's own pins, from closed forms, brute force and library
routines written in the tests themselves).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def elem_of(dtype) -> int:
    return oracle.F32 if dtype == torch.float32 else oracle.BF16


def to_oracle(t: torch.Tensor) -> np.ndarray:
    """Host numpy view in oracle storage: float32, or uint16 bf16 patterns."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.int32:
        return t.numpy()
    raise TypeError(t.dtype)


def to_f64(t) -> np.ndarray:
    """Exact fp64 values of a bf16/fp32 tensor or oracle-storage array."""
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    if t.dtype == np.uint16:
        return oracle.bf16_to_f64(t)
    return t.astype(np.float64)


def from_f64(a, dtype) -> torch.Tensor:
    return torch.from_numpy(np.asarray(a, np.float64)).to(dtype)


def shape_of(Hq, Hkv, D, P, pool, dtype) -> oracle.Shape:
    return oracle.Shape(Hq, Hkv, D, P, pool, elem_of(dtype))


def store_request(s: oracle.Shape, k_tok, v_tok, pt_row, k_pool, v_pool, pos0=0):
    """Write one request's tokens ([T][Hkv][D] oracle storage) into the pool."""
    if k_tok.shape[0]:
        oracle.store_tokens(s, np.ascontiguousarray(k_tok), np.ascontiguousarray(v_tok),
                            pos0, np.ascontiguousarray(pt_row, dtype=np.int32), k_pool, v_pool)


def random_tokens(gen: torch.Generator, n, Hkv, D, dtype, scale=1.0):
    x = torch.randn((n, Hkv, D), generator=gen, dtype=torch.float32) * scale
    return x.to(dtype)


def pool_arrays(s: oracle.Shape, fill=0.0):
    """Empty K pool [pool][Hkv][P][D] and V pool [pool][Hkv][D][P]."""
    dt = torch.float32 if s.elem == oracle.F32 else torch.bfloat16
    k = torch.full((s.pool, s.Hkv, s.P, s.D), fill, dtype=dt)
    v = torch.full((s.pool, s.Hkv, s.D, s.P), fill, dtype=dt)
    return to_oracle(k).copy(), to_oracle(v).copy()
