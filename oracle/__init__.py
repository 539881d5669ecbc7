"""fp64 CPU oracle for Quest query-aware sparse decode over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
library (``kv_cache_decode_quest_amd``) never imports, loads or calls it, and
the two share no code: this package wraps ``quest_oracle.c`` (plain C, built
with gcc) through ctypes and adds only argument marshalling.

Arrays are numpy.  Element storage: ``float32`` arrays are fp32 data,
``uint16`` arrays are raw bfloat16 bit patterns.  Every result is fp64 (or
int32 for page ids).  What each function computes, and the readings taken
where the pages are silent, is documented in ``quest_oracle.c``.

Parity status: page bounds, scores, budget, selection, attention and the KV
store are pinned by ``tests/test_oracle_pins.py``; the choice of MAX as the
GQA reduction and the absence of forced pages are readings, not pins
("parity unpinned" as to which variant the pages mean).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "quest_oracle.c")
LIB_PATH = os.path.join(_HERE, "libquest_oracle.so")

F32, BF16 = 0, 1
REDUCE = {"max": 0, "sum": 1}


def build() -> str:
    """Compile the oracle with gcc (no HIP, no OpenMP: single-threaded)."""
    tmp = LIB_PATH + ".tmp"
    subprocess.run(
        ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
         SOURCE, "-o", tmp, "-lm"],
        check=True, cwd=_HERE)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Shape(ctypes.Structure):
    _fields_ = [
        ("elem", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pool_pages", ctypes.c_int64),
    ]


_lib = None


def lib():
    """Load the built oracle; build it first only if nothing is built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = load(LIB_PATH)
    return _lib


def load(path):
    """A ctypes handle on an oracle shared object with its signatures set."""
    L = ctypes.CDLL(path)
    vp, i32, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double
    sp = ctypes.POINTER(_Shape)
    L.qo_store_tokens.argtypes = [sp, i32, vp, vp, i32, vp, vp, vp]
    L.qo_request_bounds.argtypes = [sp, vp, vp, i32, vp]
    L.qo_page_bounds.argtypes = [sp, vp, vp, i32, i32, vp]
    L.qo_request_scores.argtypes = [sp, vp, vp, i32, i32, vp]
    L.qo_pages_for_budget.argtypes = [i32, i32, i32]
    L.qo_pages_for_budget.restype = i32
    L.qo_request_head_scores.argtypes = [sp, vp, vp, i32, vp]
    L.qo_request_attend_heads.argtypes = [sp, vp, vp, vp, vp, i32, vp, vp, i32, f64, vp]
    L.qo_select.argtypes = [vp, i32, i32, vp]
    L.qo_select_forced.argtypes = [vp, i32, i32, i32, i32, vp]
    L.qo_request_attend.argtypes = [sp, vp, vp, vp, vp, i32, vp, vp, i32, f64, vp]
    L.qo_request_dense.argtypes = [sp, vp, vp, vp, vp, i32, f64, vp]
    for fn in (L.qo_store_tokens, L.qo_request_bounds, L.qo_page_bounds,
               L.qo_request_scores, L.qo_request_head_scores, L.qo_request_attend_heads,
               L.qo_select, L.qo_select_forced, L.qo_request_attend,
               L.qo_request_dense):
        fn.restype = None
    return L


class Shape:
    """Head counts, head dim, page size, pool size and element type."""

    def __init__(self, num_q_heads, num_kv_heads, head_dim, page_size,
                 num_pool_pages, elem):
        if num_q_heads % num_kv_heads:
            raise ValueError("num_q_heads must be a multiple of num_kv_heads")
        self.Hq, self.Hkv, self.D, self.P = num_q_heads, num_kv_heads, head_dim, page_size
        self.pool, self.elem = int(num_pool_pages), int(elem)
        self.G = num_q_heads // num_kv_heads
        self._c = _Shape(self.elem, self.Hq, self.Hkv, self.D, self.P, self.pool)

    @property
    def c(self):
        return ctypes.byref(self._c)

    def storage_dtype(self):
        return np.float32 if self.elem == F32 else np.uint16


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(a: np.ndarray, dtype, shape=None, name="array"):
    if not isinstance(a, np.ndarray) or a.dtype != np.dtype(dtype):
        raise TypeError(f"{name}: expected numpy {np.dtype(dtype)}, got {getattr(a, 'dtype', type(a))}")
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError(f"{name}: must be C-contiguous")
    if shape is not None and tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {a.shape}")


def num_pages(ctx: int, page_size: int) -> int:
    return 0 if ctx <= 0 else -(-ctx // page_size)


def _check_pool(s: Shape, k_cache, v_cache):
    e = s.storage_dtype()
    _check(k_cache, e, (s.pool, s.Hkv, s.P, s.D), "k_cache")
    if v_cache is not None:
        _check(v_cache, e, (s.pool, s.Hkv, s.D, s.P), "v_cache")


def _check_row(s: Shape, pt_row, ctx):
    _check(pt_row, np.int32, None, "page_table row")
    n = num_pages(ctx, s.P)
    if pt_row.ndim != 1 or pt_row.shape[0] < n:
        raise ValueError("page_table row shorter than the request's pages")
    if n and (pt_row[:n].min() < 0 or pt_row[:n].max() >= s.pool):
        raise ValueError("page id out of the pool")
    return n


def store_tokens(s: Shape, k_new, v_new, pos0, pt_row, k_cache, v_cache):
    """Write k_new/v_new ([n_new][Hkv][D]) at positions pos0.. in place."""
    _check_pool(s, k_cache, v_cache)
    e = s.storage_dtype()
    n_new = k_new.shape[0]
    _check(k_new, e, (n_new, s.Hkv, s.D), "k_new")
    _check(v_new, e, (n_new, s.Hkv, s.D), "v_new")
    _check_row(s, pt_row, pos0 + n_new)
    lib().qo_store_tokens(s.c, n_new, _ptr(k_new), _ptr(v_new), int(pos0),
                          _ptr(pt_row), _ptr(k_cache), _ptr(v_cache))


def request_bounds(s: Shape, k_cache, pt_row, ctx) -> np.ndarray:
    """fp64 [n_pages][Hkv][2][D]: per-page key min (index 0) and max (1)."""
    _check_pool(s, k_cache, None)
    n = _check_row(s, pt_row, ctx)
    out = np.empty((n, s.Hkv, 2, s.D), np.float64)
    lib().qo_request_bounds(s.c, _ptr(k_cache), _ptr(pt_row), int(ctx), _ptr(out))
    return out


def page_bounds(s: Shape, k_cache, pt_row, ctx, j) -> np.ndarray:
    """fp64 [Hkv][2][D] for logical page j only."""
    _check_pool(s, k_cache, None)
    n = _check_row(s, pt_row, ctx)
    if not 0 <= j < n:
        raise ValueError("page index outside the request")
    out = np.empty((s.Hkv, 2, s.D), np.float64)
    lib().qo_page_bounds(s.c, _ptr(k_cache), _ptr(pt_row), int(ctx), int(j), _ptr(out))
    return out


def request_scores(s: Shape, q_r, bounds, reduce="max") -> np.ndarray:
    """fp64 [Hkv][n_pages] page scores of one request."""
    _check(q_r, s.storage_dtype(), (s.Hq, s.D), "q")
    n = bounds.shape[0]
    _check(bounds, np.float64, (n, s.Hkv, 2, s.D), "bounds")
    out = np.empty((s.Hkv, n), np.float64)
    lib().qo_request_scores(s.c, _ptr(q_r), _ptr(bounds), n, REDUCE[reduce], _ptr(out))
    return out


def request_head_scores(s: Shape, q_r, bounds) -> np.ndarray:
    """fp64 [Hq][n_pages]: every q head's own page bound (no group reduction)."""
    _check(q_r, s.storage_dtype(), (s.Hq, s.D), "q")
    n = bounds.shape[0]
    _check(bounds, np.float64, (n, s.Hkv, 2, s.D), "bounds")
    out = np.empty((s.Hq, n), np.float64)
    lib().qo_request_head_scores(s.c, _ptr(q_r), _ptr(bounds), n, _ptr(out))
    return out


def pages_for_budget(budget_tokens, ctx, page_size) -> int:
    return int(lib().qo_pages_for_budget(int(budget_tokens), int(ctx), int(page_size)))


def select(scores_row, k, n_sink=0, n_recent=0) -> np.ndarray:
    """Ascending logical ids of the k best pages of one score row; with
    n_sink / n_recent, the first / last pages of the row are kept first."""
    scores_row = np.ascontiguousarray(scores_row, dtype=np.float64)
    n = scores_row.shape[0]
    if not 0 <= k <= n:
        raise ValueError("k outside [0, n]")
    out = np.empty(max(k, 1), np.int32)
    if n_sink or n_recent:
        lib().qo_select_forced(_ptr(scores_row), n, int(k), int(n_sink), int(n_recent),
                               _ptr(out))
    else:
        lib().qo_select(_ptr(scores_row), n, int(k), _ptr(out))
    return out[:k].copy()


def _page_table(sel, rows, n):
    stride = max([len(x) for x in sel] + [1])
    table = np.full((rows, stride), -1, np.int32)
    nsel = np.zeros(rows, np.int32)
    for g, pages in enumerate(sel):
        pages = np.asarray(pages, np.int32)
        if pages.size and (pages.min() < 0 or pages.max() >= n):
            raise ValueError("selected page outside the request")
        table[g, :pages.size] = pages
        nsel[g] = pages.size
    return table, nsel, stride


def request_attend(s: Shape, q_r, k_cache, v_cache, pt_row, ctx, sel, sm_scale) -> np.ndarray:
    """fp64 [Hq][D]: attention of one request over the pages in ``sel``.

    ``sel`` is a list of Hkv integer arrays (logical page ids per KV head)."""
    _check_pool(s, k_cache, v_cache)
    _check(q_r, s.storage_dtype(), (s.Hq, s.D), "q")
    n = _check_row(s, pt_row, ctx)
    if len(sel) != s.Hkv:
        raise ValueError("need one page list per KV head")
    table, nsel, stride = _page_table(sel, s.Hkv, n)
    out = np.empty((s.Hq, s.D), np.float64)
    lib().qo_request_attend(s.c, _ptr(q_r), _ptr(k_cache), _ptr(v_cache), _ptr(pt_row),
                            int(ctx), _ptr(table), _ptr(nsel), stride, float(sm_scale),
                            _ptr(out))
    return out


def request_attend_heads(s: Shape, q_r, k_cache, v_cache, pt_row, ctx, sel,
                         sm_scale) -> np.ndarray:
    """fp64 [Hq][D]: attention with one page list per q head (``sel`` has Hq
    integer arrays of logical ids)."""
    _check_pool(s, k_cache, v_cache)
    _check(q_r, s.storage_dtype(), (s.Hq, s.D), "q")
    n = _check_row(s, pt_row, ctx)
    if len(sel) != s.Hq:
        raise ValueError("need one page list per q head")
    table, nsel, stride = _page_table(sel, s.Hq, n)
    out = np.empty((s.Hq, s.D), np.float64)
    lib().qo_request_attend_heads(s.c, _ptr(q_r), _ptr(k_cache), _ptr(v_cache), _ptr(pt_row),
                                  int(ctx), _ptr(table), _ptr(nsel), stride, float(sm_scale),
                                  _ptr(out))
    return out


def request_dense(s: Shape, q_r, k_cache, v_cache, pt_row, ctx, sm_scale) -> np.ndarray:
    """fp64 [Hq][D]: attention of one request over all of its valid tokens."""
    _check_pool(s, k_cache, v_cache)
    _check(q_r, s.storage_dtype(), (s.Hq, s.D), "q")
    _check_row(s, pt_row, ctx)
    out = np.empty((s.Hq, s.D), np.float64)
    lib().qo_request_dense(s.c, _ptr(q_r), _ptr(k_cache), _ptr(v_cache), _ptr(pt_row),
                           int(ctx), float(sm_scale), _ptr(out))
    return out


def decode_request(s: Shape, q_r, k_cache, v_cache, pt_row, ctx, budget_tokens,
                   sm_scale, reduce="max", bounds=None, n_sink=0, n_recent=0,
                   per_q_head=False) -> dict:
    """One request's decode view and output: bounds, scores, k, selection, out.

    ``bounds`` may be passed when already computed for the same pool state.
    per_q_head: every q head scores and selects its own pages (``reduce`` is
    not used); scores and sel then have one row per q head."""
    if bounds is None:
        bounds = request_bounds(s, k_cache, pt_row, ctx)
    k = pages_for_budget(budget_tokens, ctx, s.P)
    if per_q_head:
        scores = request_head_scores(s, q_r, bounds)
        sel = [select(scores[h], k, n_sink, n_recent) for h in range(s.Hq)]
        out = request_attend_heads(s, q_r, k_cache, v_cache, pt_row, ctx, sel, sm_scale)
        return {"bounds": bounds, "scores": scores, "k": k, "sel": sel, "out": out}
    scores = request_scores(s, q_r, bounds, reduce)
    sel = [select(scores[g], k, n_sink, n_recent) for g in range(s.Hkv)]
    out = request_attend(s, q_r, k_cache, v_cache, pt_row, ctx, sel, sm_scale)
    return {"bounds": bounds, "scores": scores, "k": k, "sel": sel, "out": out}


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """View a uint16 array of bf16 patterns; identity helper for clarity."""
    _check(a, np.uint16, None, "bf16 array")
    return a


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact fp64 values of an array of bf16 bit patterns."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
