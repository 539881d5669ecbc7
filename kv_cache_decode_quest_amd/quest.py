"""Python binding of libquest.so (include/quest.h) over ctypes.

Argument marshalling only: every function checks device, dtype, shape and
contiguity of torch tensors, then passes raw device pointers, sizes and the
current HIP stream to the C entry point of the same name.  All computation
happens in the library's HIP kernels.  There is no fallback: if the library
is not built, or the HIP runtime rejects a launch, these functions raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libquest.so")

ABI_VERSION = 1
QUEST_F32, QUEST_BF16 = 0, 1
REDUCE = {"max": 0, "sum": 1}
QUEST_SELECT_PER_KV_HEAD, QUEST_SELECT_PER_Q_HEAD = 0, 1
QUEST_ERR_SCRATCH = -7
STATIC_SCRATCH_BYTES = 16 << 20     # QUEST_STATIC_SCRATCH_BYTES

# exported symbols declared in include/quest.h
EXPORTS = ("quest_abi_version", "quest_status_string", "quest_append_kv", "quest_page_scores",
           "quest_append_score", "quest_topk_pages", "quest_topk_pages_forced",
           "quest_sparse_decode_workspace_bytes", "quest_sparse_decode", "quest_sparse_decode_plan",
           "quest_topk_sparse_decode", "quest_topk_sparse_decode_fused",
           "quest_topk_sparse_decode_plan", "quest_decode_step", "quest_decode_step_noalloc")


class QuestError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")


class QuestLayout(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("num_pool_pages", ctypes.c_int64),
        ("max_pages_per_seq", ctypes.c_int32),
        ("selection", ctypes.c_int32),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Loads libquest.so (once) and declares the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m kv_cache_decode_quest_amd.build`"
                           " (or __graft_entry__.build())")
    L = ctypes.CDLL(path)
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    lp = ctypes.POINTER(QuestLayout)
    ip = ctypes.POINTER(ctypes.c_int32)
    L.quest_abi_version.argtypes, L.quest_abi_version.restype = [], ctypes.c_int
    L.quest_status_string.argtypes, L.quest_status_string.restype = [ctypes.c_int], ctypes.c_char_p
    L.quest_append_kv.argtypes = [lp, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp]
    L.quest_page_scores.argtypes = [lp, i32, vp, vp, vp, vp, i32, vp, vp]
    L.quest_append_score.argtypes = [lp, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, i32, vp,
                                     vp]
    L.quest_topk_pages.argtypes = [lp, i32, vp, vp, vp, i32, vp, vp, vp]
    L.quest_topk_pages_forced.argtypes = [lp, i32, vp, vp, vp, i32, i32, i32, vp, vp, vp]
    L.quest_sparse_decode_workspace_bytes.argtypes = [lp, i32, i32]
    L.quest_sparse_decode_workspace_bytes.restype = sz
    L.quest_sparse_decode.argtypes = [lp, i32, vp, vp, vp, vp, vp, vp, vp, i32, f32, vp, vp,
                                      sz, vp]
    L.quest_sparse_decode_plan.argtypes = [lp, i32, i32, ip, ip]
    L.quest_topk_sparse_decode.argtypes = [lp, i32, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                           f32, vp, vp, vp, vp, sz, vp]
    L.quest_topk_sparse_decode_fused.argtypes = [lp, i32, i32]
    L.quest_topk_sparse_decode_plan.argtypes = [lp, i32, i32, ip, ip, ip]
    L.quest_decode_step.argtypes = [lp, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, i32, vp, vp,
                                    i32, i32, i32, f32, vp, vp, vp, vp, vp, sz, vp]
    L.quest_decode_step_noalloc.argtypes = [lp, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, i32,
                                            vp, vp, i32, i32, i32, f32, vp, vp, vp, vp, vp]
    for name in ("quest_append_kv", "quest_page_scores", "quest_append_score", "quest_topk_pages",
                 "quest_topk_pages_forced", "quest_sparse_decode", "quest_sparse_decode_plan",
                 "quest_topk_sparse_decode", "quest_topk_sparse_decode_fused",
                 "quest_topk_sparse_decode_plan", "quest_decode_step", "quest_decode_step_noalloc"):
        getattr(L, name).restype = ctypes.c_int
    if L.quest_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libquest ABI {L.quest_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().quest_status_string(int(status)).decode()


def quest_abi_version() -> int:
    return int(load().quest_abi_version())


def quest_status_string(status: int) -> str:
    return status_string(status)


def _dtype_code(dtype) -> int:
    if dtype == torch.float32:
        return QUEST_F32
    if dtype == torch.bfloat16:
        return QUEST_BF16
    raise TypeError(f"unsupported element type {dtype}")


def make_layout(num_q_heads, num_kv_heads, head_dim, page_size, dtype, num_pool_pages,
                max_pages_per_seq, abi_version=ABI_VERSION, per_q_head=False) -> QuestLayout:
    """per_q_head: every q head selects its own pages (no GQA sharing)."""
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    sel = QUEST_SELECT_PER_Q_HEAD if per_q_head else QUEST_SELECT_PER_KV_HEAD
    return QuestLayout(abi_version, num_q_heads, num_kv_heads, head_dim, page_size, code,
                       int(num_pool_pages), int(max_pages_per_seq), sel)


def selection_rows(L: QuestLayout) -> int:
    """Rows of scores / selections per request: KV heads, or q heads when
    every q head selects its own pages."""
    return L.num_q_heads if L.selection == QUEST_SELECT_PER_Q_HEAD else L.num_kv_heads


def _layout_dtype(L: QuestLayout):
    return torch.float32 if L.dtype == QUEST_F32 else torch.bfloat16


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t: torch.Tensor, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be on a GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _raise(fn, st):
    if st != 0:
        raise QuestError(fn, st)


def _pool_shapes(L: QuestLayout):
    return ((L.num_pool_pages, L.num_kv_heads, L.page_size, L.head_dim),
            (L.num_pool_pages, L.num_kv_heads, L.head_dim, L.page_size),
            (L.num_pool_pages, L.num_kv_heads, 2, L.head_dim))


def quest_append_kv(L: QuestLayout, k_new, v_new, cu_new, ctx_before, max_new_per_seq,
                    page_table, k_cache, v_cache, kmeta):
    """on_kv_stored: store k_new/v_new [T][Hkv][D] and refresh kmeta."""
    dt, dev = _layout_dtype(L), k_cache.device
    batch = ctx_before.shape[0]
    kshape, vshape, mshape = _pool_shapes(L)
    _check(k_cache, "k_cache", dt, kshape, dev)
    _check(v_cache, "v_cache", dt, vshape, dev)
    _check(kmeta, "kmeta", dt, mshape, dev)
    T = k_new.shape[0]
    _check(k_new, "k_new", dt, (T, L.num_kv_heads, L.head_dim), dev)
    _check(v_new, "v_new", dt, (T, L.num_kv_heads, L.head_dim), dev)
    _check(cu_new, "cu_new", torch.int32, (batch + 1,), dev)
    _check(ctx_before, "ctx_before", torch.int32, (batch,), dev)
    _check(page_table, "page_table", torch.int32, (batch, L.max_pages_per_seq), dev)
    if T == 0:
        return                       # no token to store
    st = load().quest_append_kv(ctypes.byref(L), batch, _ptr(k_new), _ptr(v_new), _ptr(cu_new),
                                _ptr(ctx_before), int(max_new_per_seq), _ptr(page_table),
                                _ptr(k_cache), _ptr(v_cache), _ptr(kmeta), _stream(dev))
    _raise("quest_append_kv", st)


def quest_page_scores(L: QuestLayout, q, kmeta, page_table, ctx_lens, scores, group_reduce="max"):
    """build_decode_view part 1: fp32 page scores [B][Hkv][max_pages]."""
    dt, dev = _layout_dtype(L), q.device
    batch = ctx_lens.shape[0]
    _check(q, "q", dt, (batch, L.num_q_heads, L.head_dim), dev)
    _check(kmeta, "kmeta", dt, _pool_shapes(L)[2], dev)
    _check(page_table, "page_table", torch.int32, (batch, L.max_pages_per_seq), dev)
    _check(ctx_lens, "ctx_lens", torch.int32, (batch,), dev)
    _check(scores, "scores", torch.float32, (batch, selection_rows(L), L.max_pages_per_seq), dev)
    st = load().quest_page_scores(ctypes.byref(L), batch, _ptr(q), _ptr(kmeta), _ptr(page_table),
                                  _ptr(ctx_lens), REDUCE[group_reduce], _ptr(scores), _stream(dev))
    _raise("quest_page_scores", st)


def quest_append_score(L: QuestLayout, q, k_new, v_new, cu_new, ctx_before, max_new_per_seq,
                       page_table, k_cache, v_cache, kmeta, scores, group_reduce="max"):
    """on_kv_stored + build_decode_view part 1 in one pass (request lengths
    after the append are ctx_before + new tokens)."""
    dt, dev = _layout_dtype(L), q.device
    batch = ctx_before.shape[0]
    kshape, vshape, mshape = _pool_shapes(L)
    _check(q, "q", dt, (batch, L.num_q_heads, L.head_dim), dev)
    _check(k_cache, "k_cache", dt, kshape, dev)
    _check(v_cache, "v_cache", dt, vshape, dev)
    _check(kmeta, "kmeta", dt, mshape, dev)
    T = k_new.shape[0]
    _check(k_new, "k_new", dt, (T, L.num_kv_heads, L.head_dim), dev)
    _check(v_new, "v_new", dt, (T, L.num_kv_heads, L.head_dim), dev)
    _check(cu_new, "cu_new", torch.int32, (batch + 1,), dev)
    _check(ctx_before, "ctx_before", torch.int32, (batch,), dev)
    _check(page_table, "page_table", torch.int32, (batch, L.max_pages_per_seq), dev)
    _check(scores, "scores", torch.float32, (batch, selection_rows(L), L.max_pages_per_seq), dev)
    if T == 0:                       # nothing to store: a plain scoring pass
        k_new = v_new = torch.empty((1, L.num_kv_heads, L.head_dim), dtype=dt, device=dev)
    st = load().quest_append_score(ctypes.byref(L), batch, _ptr(q), _ptr(k_new), _ptr(v_new),
                                   _ptr(cu_new), _ptr(ctx_before), int(max_new_per_seq),
                                   _ptr(page_table), _ptr(k_cache), _ptr(v_cache), _ptr(kmeta),
                                   REDUCE[group_reduce], _ptr(scores), _stream(dev))
    _raise("quest_append_score", st)


def quest_topk_pages(L: QuestLayout, scores, ctx_lens, budget_tokens, max_k, sel_pages, num_sel):
    """build_decode_view part 2: ascending top-k logical pages per (r, KV head)."""
    _topk(L, scores, ctx_lens, budget_tokens, max_k, sel_pages, num_sel)


def quest_topk_pages_forced(L: QuestLayout, scores, ctx_lens, budget_tokens, max_k, n_sink,
                            n_recent, sel_pages, num_sel):
    """quest_topk_pages with the first n_sink and last n_recent pages of each
    request kept ahead of the scored ones."""
    _topk(L, scores, ctx_lens, budget_tokens, max_k, sel_pages, num_sel, n_sink, n_recent)


def _topk(L, scores, ctx_lens, budget_tokens, max_k, sel_pages, num_sel, n_sink=None,
          n_recent=None):
    dev = scores.device
    batch = ctx_lens.shape[0]
    _check(scores, "scores", torch.float32, (batch, selection_rows(L), L.max_pages_per_seq), dev)
    _check(ctx_lens, "ctx_lens", torch.int32, (batch,), dev)
    _check(budget_tokens, "budget_tokens", torch.int32, (batch,), dev)
    _check(sel_pages, "sel_pages", torch.int32, (batch, selection_rows(L), max_k), dev)
    _check(num_sel, "num_sel", torch.int32, (batch, selection_rows(L)), dev)
    if n_sink is None:
        st = load().quest_topk_pages(ctypes.byref(L), batch, _ptr(scores), _ptr(ctx_lens),
                                     _ptr(budget_tokens), int(max_k), _ptr(sel_pages),
                                     _ptr(num_sel), _stream(dev))
        _raise("quest_topk_pages", st)
    else:
        st = load().quest_topk_pages_forced(ctypes.byref(L), batch, _ptr(scores),
                                            _ptr(ctx_lens), _ptr(budget_tokens), int(max_k),
                                            int(n_sink), int(n_recent), _ptr(sel_pages),
                                            _ptr(num_sel), _stream(dev))
        _raise("quest_topk_pages_forced", st)


def quest_sparse_decode_workspace_bytes(L: QuestLayout, batch: int, max_k: int) -> int:
    return int(load().quest_sparse_decode_workspace_bytes(ctypes.byref(L), int(batch), int(max_k)))


def quest_sparse_decode_plan(L: QuestLayout, batch: int, max_k: int):
    ns, pps = ctypes.c_int32(), ctypes.c_int32()
    st = load().quest_sparse_decode_plan(ctypes.byref(L), int(batch), int(max_k),
                                         ctypes.byref(ns), ctypes.byref(pps))
    _raise("quest_sparse_decode_plan", st)
    return {"num_splits": ns.value, "pages_per_split": pps.value}


def quest_sparse_decode(L: QuestLayout, q, k_cache, v_cache, page_table, ctx_lens, sel_pages,
                        num_sel, max_k, sm_scale, out, workspace):
    """Attention over the selected pages; out [B][Hq][D] in the layout dtype."""
    dt, dev = _layout_dtype(L), q.device
    batch = ctx_lens.shape[0]
    kshape, vshape, _ = _pool_shapes(L)
    _check(q, "q", dt, (batch, L.num_q_heads, L.head_dim), dev)
    _check(k_cache, "k_cache", dt, kshape, dev)
    _check(v_cache, "v_cache", dt, vshape, dev)
    _check(page_table, "page_table", torch.int32, (batch, L.max_pages_per_seq), dev)
    _check(ctx_lens, "ctx_lens", torch.int32, (batch,), dev)
    _check(sel_pages, "sel_pages", torch.int32, (batch, selection_rows(L), max_k), dev)
    _check(num_sel, "num_sel", torch.int32, (batch, selection_rows(L)), dev)
    _check(out, "out", dt, (batch, L.num_q_heads, L.head_dim), dev)
    _check(workspace, "workspace", None, None, dev)
    nbytes = workspace.numel() * workspace.element_size()
    st = load().quest_sparse_decode(ctypes.byref(L), batch, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(page_table), _ptr(ctx_lens), _ptr(sel_pages),
                                    _ptr(num_sel), int(max_k), float(sm_scale), _ptr(out),
                                    _ptr(workspace), nbytes, _stream(dev))
    _raise("quest_sparse_decode", st)


def quest_topk_sparse_decode(L: QuestLayout, q, k_cache, v_cache, page_table, ctx_lens, scores,
                             budget_tokens, max_k, sm_scale, sel_pages, num_sel, out, workspace,
                             n_sink=0, n_recent=0):
    """quest_topk_pages_forced then quest_sparse_decode on its selection, in
    one kernel (plus the merge) where the shape allows."""
    dt, dev = _layout_dtype(L), q.device
    batch = ctx_lens.shape[0]
    kshape, vshape, _ = _pool_shapes(L)
    rows = selection_rows(L)
    _check(q, "q", dt, (batch, L.num_q_heads, L.head_dim), dev)
    _check(k_cache, "k_cache", dt, kshape, dev)
    _check(v_cache, "v_cache", dt, vshape, dev)
    _check(page_table, "page_table", torch.int32, (batch, L.max_pages_per_seq), dev)
    _check(ctx_lens, "ctx_lens", torch.int32, (batch,), dev)
    _check(scores, "scores", torch.float32, (batch, rows, L.max_pages_per_seq), dev)
    _check(budget_tokens, "budget_tokens", torch.int32, (batch,), dev)
    _check(sel_pages, "sel_pages", torch.int32, (batch, rows, max_k), dev)
    _check(num_sel, "num_sel", torch.int32, (batch, rows), dev)
    _check(out, "out", dt, (batch, L.num_q_heads, L.head_dim), dev)
    _check(workspace, "workspace", None, None, dev)
    nbytes = workspace.numel() * workspace.element_size()
    st = load().quest_topk_sparse_decode(ctypes.byref(L), batch, _ptr(q), _ptr(k_cache),
                                         _ptr(v_cache), _ptr(page_table), _ptr(ctx_lens),
                                         _ptr(scores), _ptr(budget_tokens), int(max_k),
                                         int(n_sink), int(n_recent), float(sm_scale),
                                         _ptr(sel_pages), _ptr(num_sel), _ptr(out),
                                         _ptr(workspace), nbytes, _stream(dev))
    _raise("quest_topk_sparse_decode", st)


def quest_topk_sparse_decode_fused(L: QuestLayout, batch: int, max_k: int) -> bool:
    """Whether quest_topk_sparse_decode runs as one fused kernel here."""
    st = load().quest_topk_sparse_decode_fused(ctypes.byref(L), int(batch), int(max_k))
    if st < 0:
        _raise("quest_topk_sparse_decode_fused", st)
    return st == 1


def quest_topk_sparse_decode_plan(L: QuestLayout, batch: int, max_k: int):
    """The plan of quest_topk_sparse_decode: whether it runs the fused kernel,
    and its splits per selection row and pages per split."""
    fu, ns, pps = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    st = load().quest_topk_sparse_decode_plan(ctypes.byref(L), int(batch), int(max_k),
                                              ctypes.byref(fu), ctypes.byref(ns),
                                              ctypes.byref(pps))
    _raise("quest_topk_sparse_decode_plan", st)
    return {"fused": bool(fu.value), "num_splits": ns.value, "pages_per_split": pps.value}


def quest_decode_step(L: QuestLayout, q, k_new, v_new, cu_new, ctx_before, max_new_per_seq,
                      page_table, k_cache, v_cache, kmeta, ctx_lens, budget_tokens, max_k,
                      sm_scale, scores, sel_pages, num_sel, out, workspace, group_reduce="max",
                      n_sink=0, n_recent=0):
    """The whole decode step of one layer in one call: quest_append_score,
    then quest_topk_sparse_decode on its scores."""
    dt, dev = _layout_dtype(L), q.device
    batch = ctx_before.shape[0]
    kshape, vshape, mshape = _pool_shapes(L)
    rows = selection_rows(L)
    _check(q, "q", dt, (batch, L.num_q_heads, L.head_dim), dev)
    _check(k_cache, "k_cache", dt, kshape, dev)
    _check(v_cache, "v_cache", dt, vshape, dev)
    _check(kmeta, "kmeta", dt, mshape, dev)
    T = k_new.shape[0]
    _check(k_new, "k_new", dt, (T, L.num_kv_heads, L.head_dim), dev)
    _check(v_new, "v_new", dt, (T, L.num_kv_heads, L.head_dim), dev)
    _check(cu_new, "cu_new", torch.int32, (batch + 1,), dev)
    _check(ctx_before, "ctx_before", torch.int32, (batch,), dev)
    _check(ctx_lens, "ctx_lens", torch.int32, (batch,), dev)
    _check(page_table, "page_table", torch.int32, (batch, L.max_pages_per_seq), dev)
    _check(budget_tokens, "budget_tokens", torch.int32, (batch,), dev)
    _check(scores, "scores", torch.float32, (batch, rows, L.max_pages_per_seq), dev)
    _check(sel_pages, "sel_pages", torch.int32, (batch, rows, max_k), dev)
    _check(num_sel, "num_sel", torch.int32, (batch, rows), dev)
    _check(out, "out", dt, (batch, L.num_q_heads, L.head_dim), dev)
    _check(workspace, "workspace", None, None, dev)
    if T == 0:                       # nothing to store
        k_new = v_new = torch.empty((1, L.num_kv_heads, L.head_dim), dtype=dt, device=dev)
    nbytes = workspace.numel() * workspace.element_size()
    st = load().quest_decode_step(ctypes.byref(L), batch, _ptr(q), _ptr(k_new), _ptr(v_new),
                                  _ptr(cu_new), _ptr(ctx_before), int(max_new_per_seq),
                                  _ptr(page_table), _ptr(k_cache), _ptr(v_cache), _ptr(kmeta),
                                  REDUCE[group_reduce], _ptr(ctx_lens), _ptr(budget_tokens),
                                  int(max_k), int(n_sink), int(n_recent), float(sm_scale),
                                  _ptr(scores), _ptr(sel_pages), _ptr(num_sel), _ptr(out),
                                  _ptr(workspace), nbytes, _stream(dev))
    _raise("quest_decode_step", st)


def quest_decode_step_noalloc(L: QuestLayout, q, k_new, v_new, cu_new, ctx_before,
                              max_new_per_seq, page_table, k_cache, v_cache, kmeta, ctx_lens,
                              budget_tokens, max_k, sm_scale, scores, sel_pages, num_sel, out,
                              group_reduce="max", n_sink=0, n_recent=0):
    """quest_decode_step with the split partials in the library's static
    device scratch (QUEST_STATIC_SCRATCH_BYTES per GPU) instead of a caller
    workspace: for callers that cannot allocate.  Calls that may overlap on
    one GPU race on that scratch."""
    dt, dev = _layout_dtype(L), q.device
    batch = ctx_before.shape[0]
    kshape, vshape, mshape = _pool_shapes(L)
    rows = selection_rows(L)
    _check(q, "q", dt, (batch, L.num_q_heads, L.head_dim), dev)
    _check(k_cache, "k_cache", dt, kshape, dev)
    _check(v_cache, "v_cache", dt, vshape, dev)
    _check(kmeta, "kmeta", dt, mshape, dev)
    T = k_new.shape[0]
    _check(k_new, "k_new", dt, (T, L.num_kv_heads, L.head_dim), dev)
    _check(v_new, "v_new", dt, (T, L.num_kv_heads, L.head_dim), dev)
    _check(cu_new, "cu_new", torch.int32, (batch + 1,), dev)
    _check(ctx_before, "ctx_before", torch.int32, (batch,), dev)
    _check(ctx_lens, "ctx_lens", torch.int32, (batch,), dev)
    _check(page_table, "page_table", torch.int32, (batch, L.max_pages_per_seq), dev)
    _check(budget_tokens, "budget_tokens", torch.int32, (batch,), dev)
    _check(scores, "scores", torch.float32, (batch, rows, L.max_pages_per_seq), dev)
    _check(sel_pages, "sel_pages", torch.int32, (batch, rows, max_k), dev)
    _check(num_sel, "num_sel", torch.int32, (batch, rows), dev)
    _check(out, "out", dt, (batch, L.num_q_heads, L.head_dim), dev)
    if T == 0:                       # nothing to store: the append reads at most row 0 of
        k_new = v_new = q            # k_new / v_new (clamped loads), which q's storage covers
    with torch.cuda.device(dev):     # the scratch copy of the stream's device
        st = load().quest_decode_step_noalloc(
            ctypes.byref(L), batch, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(cu_new),
            _ptr(ctx_before), int(max_new_per_seq), _ptr(page_table), _ptr(k_cache),
            _ptr(v_cache), _ptr(kmeta), REDUCE[group_reduce], _ptr(ctx_lens),
            _ptr(budget_tokens), int(max_k), int(n_sink), int(n_recent), float(sm_scale),
            _ptr(scores), _ptr(sel_pages), _ptr(num_sel), _ptr(out), _stream(dev))
    _raise("quest_decode_step_noalloc", st)


@dataclass
class DecodeBuffers:
    """Caller-owned per-step buffers for one layer (scores, selection, output)."""
    scores: torch.Tensor
    sel_pages: torch.Tensor
    num_sel: torch.Tensor
    out: torch.Tensor
    workspace: torch.Tensor
    max_k: int


def alloc_decode_buffers(L: QuestLayout, batch: int, max_k: int, device) -> DecodeBuffers:
    dt = _layout_dtype(L)
    ws = max(quest_sparse_decode_workspace_bytes(L, batch, max_k), 16)
    return DecodeBuffers(
        scores=torch.empty((batch, selection_rows(L), L.max_pages_per_seq), dtype=torch.float32,
                           device=device),
        sel_pages=torch.empty((batch, selection_rows(L), max_k), dtype=torch.int32,
                              device=device),
        num_sel=torch.empty((batch, selection_rows(L)), dtype=torch.int32, device=device),
        out=torch.empty((batch, L.num_q_heads, L.head_dim), dtype=dt, device=device),
        workspace=torch.empty((ws + 3) // 4, dtype=torch.float32, device=device),
        max_k=max_k)


def decode_step(L: QuestLayout, q, k_new, v_new, cu_new, ctx_before, ctx_lens, budget_tokens,
                page_table, k_cache, v_cache, kmeta, bufs: DecodeBuffers, sm_scale,
                group_reduce="max", max_new_per_seq=1):
    """One Quest decode step of one layer: on_kv_stored fused with the page
    scores, then the top-k (the rest of build_decode_view) and attention over
    the view, through quest_decode_step (asynchronous on the current stream);
    ctx_lens must equal ctx_before + the new tokens."""
    quest_decode_step(L, q, k_new, v_new, cu_new, ctx_before, max_new_per_seq, page_table,
                      k_cache, v_cache, kmeta, ctx_lens, budget_tokens, bufs.max_k, sm_scale,
                      bufs.scores, bufs.sel_pages, bufs.num_sel, bufs.out, bufs.workspace,
                      group_reduce)
    return bufs.out
