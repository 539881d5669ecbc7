"""Host-side checks of libquest.so: it loads, exports every entry point the
header declares, and rejects bad arguments before any HIP call.  Nothing here
launches a kernel (the validation failures return before any launch, and
batch-0 calls launch nothing)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from kv_cache_decode_quest_amd import quest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "quest.h")
PROBE_HEADER = os.path.join(ROOT, "include", "quest_probe.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_ABI = 0, -1, -2, -3, -4, -5
FAKE = ctypes.c_void_p(0x100000)          # aligned, never dereferenced on the host


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(quest_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return quest.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(lib, name), f"{name} declared in quest.h but not exported"
    assert sorted(quest.EXPORTS) == names


def test_version_and_status_strings(lib):
    assert quest.quest_abi_version() == 1
    for st in (OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_ABI, -6):
        assert quest.status_string(st) != "unknown status"
    assert quest.status_string(-99) == "unknown status"


def layout(**kw):
    base = dict(num_q_heads=32, num_kv_heads=4, head_dim=128, page_size=16, dtype=1,
                num_pool_pages=1000, max_pages_per_seq=100)
    base.update(kw)
    abi = base.pop("abi_version", 1)
    L = quest.make_layout(base["num_q_heads"], base["num_kv_heads"], base["head_dim"],
                          base["page_size"], base["dtype"], base["num_pool_pages"],
                          base["max_pages_per_seq"], abi_version=abi)
    L.selection = base.get("selection", 0)
    return L


def scores_call(lib, L, batch=1, reduce=0, q=FAKE, kmeta=FAKE, out=FAKE):
    return lib.quest_page_scores(ctypes.byref(L) if L is not None else None, batch, q, kmeta,
                                 FAKE, FAKE, reduce, out, None)


def decode_call(lib, L, batch=1, max_k=16, ws=FAKE, ws_bytes=1 << 30, q=FAKE, scale=0.1):
    return lib.quest_sparse_decode(ctypes.byref(L), batch, q, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, max_k, scale, FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,want", [
    (dict(abi_version=2), ERR_ABI),
    (dict(num_q_heads=30), ERR_SHAPE),                 # 30 % 4 != 0
    (dict(num_q_heads=0), ERR_SHAPE),
    (dict(num_pool_pages=0), ERR_SHAPE),
    (dict(max_pages_per_seq=0), ERR_SHAPE),
    (dict(head_dim=96), ERR_UNSUPPORTED),
    (dict(page_size=12), ERR_UNSUPPORTED),
    (dict(page_size=128), ERR_UNSUPPORTED),
    (dict(page_size=64, dtype=0), ERR_UNSUPPORTED),
    (dict(dtype=7), ERR_UNSUPPORTED),
    (dict(num_q_heads=68), ERR_UNSUPPORTED),           # G = 17 > 16
    (dict(selection=2), ERR_UNSUPPORTED),
    (dict(selection=-1), ERR_UNSUPPORTED),
])
def test_layout_rejections(lib, kw, want):
    L = layout(**kw)
    assert scores_call(lib, L) == want
    assert lib.quest_topk_pages(ctypes.byref(L), 1, FAKE, FAKE, FAKE, 8, FAKE, FAKE, None) == want
    assert decode_call(lib, L) == want
    assert lib.quest_append_kv(ctypes.byref(L), 1, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE,
                               FAKE, None) == want
    assert fused_call(lib, L) == want


def fused_call(lib, L, batch=1, reduce=0, q=FAKE, kmeta=FAKE, max_new=1, k_new=FAKE):
    return lib.quest_append_score(ctypes.byref(L), batch, q, k_new, FAKE, FAKE, FAKE, max_new,
                                  FAKE, FAKE, FAKE, kmeta, reduce, FAKE, None)


def test_fused_append_score_rejections(lib):
    L = layout()
    assert fused_call(lib, L, q=None) == ERR_NULL
    assert fused_call(lib, L, k_new=None) == ERR_NULL
    assert fused_call(lib, L, reduce=3) == ERR_UNSUPPORTED
    assert fused_call(lib, L, max_new=-1) == ERR_SHAPE
    assert fused_call(lib, L, kmeta=ctypes.c_void_p(0x100002)) == ERR_SHAPE
    assert fused_call(lib, L, batch=-1) == ERR_SHAPE
    assert lib.quest_append_score(ctypes.byref(L), 0, None, None, None, None, None, 0, None,
                                  None, None, None, 0, None, None) == OK


def test_forced_topk_rejections(lib):
    L = layout()

    def call(n_sink, n_recent, batch=1, scores=FAKE):
        return lib.quest_topk_pages_forced(ctypes.byref(L), batch, scores, FAKE, FAKE, 8,
                                           n_sink, n_recent, FAKE, FAKE, None)
    assert call(-1, 0) == ERR_SHAPE
    assert call(0, -2) == ERR_SHAPE
    assert call(1, 1, scores=None) == ERR_NULL
    assert call(1, 1, batch=0, scores=None) == OK


def test_null_layout(lib):
    assert lib.quest_page_scores(None, 1, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None) == ERR_NULL


def test_batch_bounds_and_empty_batch(lib):
    L = layout()
    assert scores_call(lib, L, batch=-1) == ERR_SHAPE
    assert scores_call(lib, L, batch=70000) == ERR_SHAPE
    # batch * Hq <= 2^19 keeps the decode and merge grids within 2^32 work-items
    wide = layout(num_q_heads=1024, num_kv_heads=64)
    assert decode_call(lib, wide, batch=513) == ERR_SHAPE
    assert lib.quest_sparse_decode_workspace_bytes(ctypes.byref(wide), 513, 8) == 0
    assert lib.quest_sparse_decode_workspace_bytes(ctypes.byref(wide), 512, 8) > 0
    # max_pages_per_seq * Hkv < 2^30 keeps the scoring grid within 2^32 work-items
    assert scores_call(lib, layout(max_pages_per_seq=1 << 28, num_pool_pages=1 << 28)) == ERR_SHAPE
    # batch 0: nothing to do, no pointer needed, nothing launched
    assert lib.quest_page_scores(ctypes.byref(L), 0, None, None, None, None, 0, None, None) == OK
    assert lib.quest_topk_pages(ctypes.byref(L), 0, None, None, None, 4, None, None, None) == OK
    assert lib.quest_sparse_decode(ctypes.byref(L), 0, None, None, None, None, None, None, None,
                                   4, 0.1, None, None, 0, None) == OK
    assert lib.quest_append_kv(ctypes.byref(L), 0, None, None, None, None, 0, None, None, None,
                               None, None) == OK
    assert lib.quest_sparse_decode_workspace_bytes(ctypes.byref(L), 0, 4) == 0


def test_null_pointers(lib):
    L = layout()
    assert scores_call(lib, L, q=None) == ERR_NULL
    assert scores_call(lib, L, out=None) == ERR_NULL
    assert lib.quest_topk_pages(ctypes.byref(L), 1, FAKE, None, FAKE, 8, FAKE, FAKE, None) == ERR_NULL
    assert decode_call(lib, L, q=None) == ERR_NULL
    assert lib.quest_append_kv(ctypes.byref(L), 1, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE,
                               None, None) == ERR_NULL


def test_argument_rejections(lib):
    L = layout()
    assert scores_call(lib, L, reduce=2) == ERR_UNSUPPORTED
    assert lib.quest_topk_pages(ctypes.byref(L), 1, FAKE, FAKE, FAKE, 0, FAKE, FAKE, None) == ERR_SHAPE
    assert decode_call(lib, L, max_k=0) == ERR_SHAPE
    assert decode_call(lib, L, scale=float("nan")) == ERR_SHAPE
    assert decode_call(lib, L, scale=float("inf")) == ERR_SHAPE
    assert lib.quest_append_kv(ctypes.byref(L), 1, FAKE, FAKE, FAKE, FAKE, -1, FAKE, FAKE, FAKE,
                               FAKE, None) == ERR_SHAPE
    # bf16 vector loads need 16-byte alignment
    assert scores_call(lib, L, q=ctypes.c_void_p(0x100002)) == ERR_SHAPE
    assert decode_call(lib, L, q=ctypes.c_void_p(0x100008)) == ERR_SHAPE


def test_per_q_head_rows(lib):
    """Per-q-head selection: one selection row per q head, each a single head,
    in the plan's rows and the workspace size."""
    shared, per_head = layout(), layout(selection=1)
    assert quest.selection_rows(shared) == 4 and quest.selection_rows(per_head) == 32
    p = quest.quest_sparse_decode_plan(per_head, 8, 256)
    need = lib.quest_sparse_decode_workspace_bytes(ctypes.byref(per_head), 8, 256)
    assert need == 8 * 32 * p["num_splits"] * 1 * (128 + 2) * 4
    q = quest.make_layout(32, 4, 128, 16, 1, 1000, 100, per_q_head=True)
    assert q.selection == quest.QUEST_SELECT_PER_Q_HEAD


def test_workspace_contract(lib):
    L = layout()
    need = lib.quest_sparse_decode_workspace_bytes(ctypes.byref(L), 8, 256)
    plan = quest.quest_sparse_decode_plan(L, 8, 256)
    assert need == 8 * 4 * plan["num_splits"] * 8 * (128 + 2) * 4
    assert plan["num_splits"] * plan["pages_per_split"] >= 256
    assert decode_call(lib, L, batch=8, max_k=256, ws_bytes=need - 1) == ERR_WORKSPACE
    assert decode_call(lib, L, batch=8, max_k=256, ws=None) == ERR_WORKSPACE
    assert decode_call(lib, L, batch=8, max_k=256, ws=ctypes.c_void_p(0x100004)) == ERR_WORKSPACE
    assert lib.quest_sparse_decode_workspace_bytes(ctypes.byref(layout(head_dim=96)), 8, 256) == 0


def test_plan_covers_every_page():
    """Splits cover max_k pages with no empty split, and never exceed the 256
    splits a plan may use (bf16 at every page size; fp32, whose splits start
    at one page)."""
    for batch, hkv, max_k in [(1, 1, 1), (1, 1, 16), (8, 4, 256), (8, 4, 128), (32, 4, 409),
                              (64, 4, 128), (3, 2, 1000), (1, 1, 60000), (2, 4, 4097)]:
        for page_size, dtype in ((8, 1), (16, 1), (32, 1), (64, 1), (16, 0), (32, 0)):
            L = layout(num_kv_heads=hkv, num_q_heads=hkv * 8, page_size=page_size,
                       dtype=dtype)
            p = quest.quest_sparse_decode_plan(L, batch, max_k)
            assert p["pages_per_split"] >= 1
            assert 1 <= p["num_splits"] <= 256
            assert (p["num_splits"] - 1) * p["pages_per_split"] < max_k
            assert p["num_splits"] * p["pages_per_split"] >= max_k


def test_plan_shapes_of_the_workloads():
    """The plan at the measured shapes: one round per split (8 waves x 4 pages
    at page 16, x 2 at page 32), or as many rounds as keep a bf16 row within
    8 splits, or within as many as give each of 256 CUs a split when the
    batch has fewer than 32 rows."""
    def plan(batch, hkv, max_k, page_size):
        L = layout(num_kv_heads=hkv, num_q_heads=hkv * 8, page_size=page_size, dtype=1)
        p = quest.quest_sparse_decode_plan(L, batch, max_k)
        return p["num_splits"], p["pages_per_split"]
    assert plan(8, 4, 256, 16) == (8, 32)        # batch 8 x 128000, budget 4096: one round each
    assert plan(8, 4, 8008, 16) == (8, 1024)     # every page (the dense reference): 32 rounds
    assert plan(32, 4, 383, 32) == (8, 48)       # the ragged batch: 3 rounds of 16 pages
    assert plan(64, 4, 128, 16) == (4, 32)       # 256 rows of 128 pages
    for batch, max_k in [(1, 60000), (2, 9000), (8, 8008)]:
        assert plan(batch, 4, max_k, 16)[0] <= max(8, -(-256 // (batch * 4)))
    assert plan(1, 4, 60000, 16) == (63, 960)     # 4 rows: 63 splits each, so 252 in all
    assert plan(1, 1, 8000, 16) == (250, 32)      # one row: one round per split


def test_missing_library_fails_loudly(tmp_path):
    saved = quest._lib
    quest._lib = None
    try:
        with pytest.raises(RuntimeError, match="not built"):
            quest.load(str(tmp_path / "libquest.so"))
    finally:
        quest._lib = saved


def test_product_never_touches_the_oracle():
    """The library package and its kernels name no oracle module or file."""
    pkg = os.path.join(ROOT, "kv_cache_decode_quest_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "quest_oracle" not in text and "libquest_oracle" not in text, f


def topk_decode_call(lib, L, batch=1, max_k=16, ws=FAKE, ws_bytes=1 << 30, q=FAKE, scores=FAKE,
               scale=0.1, n_sink=0, n_recent=0):
    return lib.quest_topk_sparse_decode(ctypes.byref(L), batch, q, FAKE, FAKE, FAKE, FAKE,
                                        scores, FAKE, max_k, n_sink, n_recent, scale, FAKE, FAKE,
                                        FAKE, ws, ws_bytes, None)


def test_topk_sparse_decode_rejections(lib):
    """The combined call validates like quest_topk_pages_forced and
    quest_sparse_decode together, before any launch."""
    L = layout()
    assert topk_decode_call(lib, L, scores=None) == ERR_NULL
    assert topk_decode_call(lib, L, q=None) == ERR_NULL
    assert topk_decode_call(lib, L, n_sink=-1) == ERR_SHAPE
    assert topk_decode_call(lib, L, n_recent=-1) == ERR_SHAPE
    assert topk_decode_call(lib, L, max_k=0) == ERR_SHAPE
    assert topk_decode_call(lib, L, scale=float("nan")) == ERR_SHAPE
    assert topk_decode_call(lib, L, q=ctypes.c_void_p(0x100002)) == ERR_SHAPE
    need = lib.quest_sparse_decode_workspace_bytes(ctypes.byref(L), 1, 16)
    assert topk_decode_call(lib, L, ws_bytes=need - 1) == ERR_WORKSPACE
    assert topk_decode_call(lib, L, ws=None) == ERR_WORKSPACE
    assert topk_decode_call(lib, layout(head_dim=96)) == ERR_UNSUPPORTED
    assert lib.quest_topk_sparse_decode(ctypes.byref(L), 0, None, None, None, None, None, None,
                                        None, 4, 0, 0, 0.1, None, None, None, None, 0,
                                        None) == OK


def test_topk_sparse_decode_fused_rule(lib):
    """One kernel for bf16 rows of at most 8192 pages, D 64 or (D 128, P 16),
    each row split into at most min(256 / rows, the decode plan's splits)
    parts (whole rounds of 32 pages at P 16, D 128) of at most 256 pages; two
    kernels otherwise."""
    bench = layout(num_pool_pages=8 * 8009, max_pages_per_seq=8009)
    assert quest.quest_topk_sparse_decode_fused(bench, 8, 256)          # 32 rows x 8 splits
    assert quest.quest_topk_sparse_decode_fused(bench, 9, 256)          # 36 rows x 4 splits of 64
    assert quest.quest_topk_sparse_decode_fused(bench, 64, 128)         # 256 rows, whole rows
    assert not quest.quest_topk_sparse_decode_fused(bench, 65, 128)     # 260 rows
    assert quest.quest_topk_sparse_decode_fused(layout(selection=1), 8, 256)   # 256 q-head rows
    assert not quest.quest_topk_sparse_decode_fused(layout(selection=1), 8, 257)  # 288 pages
    # a split past INT32_MAX pages (256 rows, max_k near INT32_MAX) is not fused
    assert not quest.quest_topk_sparse_decode_fused(layout(selection=1), 8, 2 ** 31 - 1)
    assert not quest.quest_topk_sparse_decode_fused(layout(page_size=32), 1, 16)
    assert not quest.quest_topk_sparse_decode_fused(layout(page_size=8), 1, 16)
    assert quest.quest_topk_sparse_decode_fused(layout(head_dim=64, page_size=64), 1, 16)
    assert not quest.quest_topk_sparse_decode_fused(layout(dtype=0, head_dim=64), 1, 16)
    assert not quest.quest_topk_sparse_decode_fused(layout(max_pages_per_seq=8193), 1, 16)
    assert quest.quest_topk_sparse_decode_fused(layout(max_pages_per_seq=8192), 1, 16)
    assert not quest.quest_topk_sparse_decode_fused(layout(), 0, 16)
    big = layout(num_kv_heads=1, num_q_heads=8, num_pool_pages=9000, max_pages_per_seq=8000)
    assert quest.quest_topk_sparse_decode_fused(big, 1, 8000)           # 250 splits of 32
    assert quest.quest_topk_sparse_decode_plan(big, 1, 8000) == {
        "fused": True, "num_splits": 250, "pages_per_split": 32}
    assert quest.quest_topk_sparse_decode_plan(big, 1, 8193) == {       # 129 splits of 64
        "fused": True, "num_splits": 129, "pages_per_split": 64}
    assert not quest.quest_topk_sparse_decode_fused(big, 1, 100000)     # 241 splits of 416
    assert lib.quest_topk_sparse_decode_fused(ctypes.byref(layout()), 1, 0) == ERR_SHAPE
    # one request of 4 KV heads with 2048 pages kept: 64 splits each (the
    # decode plan's, whose partials the workspace holds), one round each
    one = layout(num_pool_pages=4000, max_pages_per_seq=4000)
    assert quest.quest_topk_sparse_decode_plan(one, 1, 2048) == {
        "fused": True, "num_splits": 64, "pages_per_split": 32}
    p = quest.quest_topk_sparse_decode_plan(bench, 8, 256)
    assert p == {"fused": True, "num_splits": 8, "pages_per_split": 32}
    assert quest.quest_topk_sparse_decode_plan(bench, 64, 128) == {
        "fused": True, "num_splits": 1, "pages_per_split": 128}
    two = quest.quest_topk_sparse_decode_plan(layout(page_size=32), 1, 16)
    assert not two["fused"]
    assert two == dict(fused=False, **quest.quest_sparse_decode_plan(layout(page_size=32), 1, 16))
    assert lib.quest_topk_sparse_decode_plan(ctypes.byref(layout()), 1, 16, None, None,
                                             None) == ERR_NULL


def test_fused_plan_fits_the_workspace():
    """Over every row count the fused kernel takes (1..256) and selection
    sizes up to 8192 pages, the fused plan never has more splits than the
    decode plan the workspace is sized for, covers max_k with no empty split,
    and uses whole rounds; so its partials always fit
    quest_sparse_decode_workspace_bytes."""
    per_round = {(16, 128): 32, (8, 64): 64, (16, 64): 32, (32, 64): 16, (64, 64): 8}
    ks = sorted(set(list(range(1, 600)) + list(range(600, 8193, 37)) +
                [2 ** e + d for e in range(5, 14) for d in (-1, 0, 1)]))
    ks = [k for k in ks if 1 <= k <= 8192]
    checked = 0
    for (P, D), rnd in per_round.items():
        for hkv in (1, 4):
            for batch in sorted(set([1, 2, 3, 5, 7, 8, 9, 16, 31, 32, 33, 63, 64] +
                                    [256 // hkv])):
                L = layout(num_kv_heads=hkv, num_q_heads=hkv * 8, head_dim=D, page_size=P,
                           num_pool_pages=9000, max_pages_per_seq=8192)
                for k in ks:
                    f = quest.quest_topk_sparse_decode_plan(L, batch, k)
                    if not f["fused"]:
                        continue
                    d = quest.quest_sparse_decode_plan(L, batch, k)
                    assert f["num_splits"] <= d["num_splits"], (P, D, hkv, batch, k, f, d)
                    assert batch * hkv * f["num_splits"] <= 256
                    assert f["pages_per_split"] % rnd == 0 and f["pages_per_split"] <= 256
                    assert (f["num_splits"] - 1) * f["pages_per_split"] < k
                    assert f["num_splits"] * f["pages_per_split"] >= k
                    checked += 1
    assert checked > 10000


def step_call(lib, L, batch=1, max_k=16, ws=FAKE, ws_bytes=1 << 30, q=FAKE, k_new=FAKE,
              ctx_lens=FAKE, reduce=0, max_new=1, scale=0.1, n_sink=0):
    return lib.quest_decode_step(ctypes.byref(L), batch, q, k_new, FAKE, FAKE, FAKE, max_new,
                                 FAKE, FAKE, FAKE, FAKE, reduce, ctx_lens, FAKE, max_k, n_sink,
                                 0, scale, FAKE, FAKE, FAKE, FAKE, ws, ws_bytes, None)


def test_decode_step_rejections(lib):
    """The one-call step validates like quest_append_score and
    quest_topk_sparse_decode together, before any launch."""
    L = layout()
    assert step_call(lib, L, q=None) == ERR_NULL
    assert step_call(lib, L, k_new=None) == ERR_NULL
    assert step_call(lib, L, ctx_lens=None) == ERR_NULL
    assert step_call(lib, L, reduce=2) == ERR_UNSUPPORTED
    assert step_call(lib, L, max_new=-1) == ERR_SHAPE
    assert step_call(lib, L, max_k=0) == ERR_SHAPE
    assert step_call(lib, L, n_sink=-1) == ERR_SHAPE
    assert step_call(lib, L, scale=float("inf")) == ERR_SHAPE
    assert step_call(lib, L, q=ctypes.c_void_p(0x100002)) == ERR_SHAPE
    need = lib.quest_sparse_decode_workspace_bytes(ctypes.byref(L), 1, 16)
    assert step_call(lib, L, ws_bytes=need - 1) == ERR_WORKSPACE
    assert step_call(lib, L, ws=None) == ERR_WORKSPACE
    assert step_call(lib, layout(page_size=48)) == ERR_UNSUPPORTED
    assert step_call(lib, layout(abi_version=2)) == ERR_ABI
    assert step_call(lib, L, batch=0, q=None, k_new=None, ctx_lens=None, ws=None) == OK


def noalloc_call(lib, L, batch=1, max_k=16, q=FAKE, scale=0.1, reduce=0):
    return lib.quest_decode_step_noalloc(ctypes.byref(L), batch, q, FAKE, FAKE, FAKE, FAKE, 1,
                                         FAKE, FAKE, FAKE, FAKE, reduce, FAKE, FAKE, max_k, 0, 0,
                                         scale, FAKE, FAKE, FAKE, FAKE, None)


def test_decode_step_noalloc_rejections(lib):
    """The no-allocation step validates like quest_decode_step and refuses,
    before any HIP call, a step whose split partials exceed the library's
    static scratch (QUEST_ERR_SCRATCH); batch 0 is a no-op."""
    ERR_SCRATCH = quest.QUEST_ERR_SCRATCH
    L = layout()
    assert noalloc_call(lib, L, q=None) == ERR_NULL
    assert noalloc_call(lib, L, max_k=0) == ERR_SHAPE
    assert noalloc_call(lib, L, scale=float("nan")) == ERR_SHAPE
    assert noalloc_call(lib, L, reduce=5) == ERR_UNSUPPORTED
    assert noalloc_call(lib, L, q=ctypes.c_void_p(0x100002)) == ERR_SHAPE
    assert noalloc_call(lib, layout(abi_version=3)) == ERR_ABI
    assert noalloc_call(lib, L, batch=0, q=None) == OK
    assert quest.status_string(ERR_SCRATCH) != "unknown status"
    # 1100 requests x 4 KV heads: 4400 rows of one split, 8 heads x 130
    # floats each = 18.3 MB of partials, beyond 16 MiB
    need = lib.quest_sparse_decode_workspace_bytes(ctypes.byref(L), 1100, 16)
    assert need > quest.STATIC_SCRATCH_BYTES
    assert noalloc_call(lib, L, batch=1100) == ERR_SCRATCH
    # fp32 at G 16, D 128: 32 rows x 64 one-page splits x 16 heads x 130 floats
    Lf = layout(dtype=0, num_q_heads=64)
    assert lib.quest_sparse_decode_workspace_bytes(ctypes.byref(Lf), 8, 64) > \
        quest.STATIC_SCRATCH_BYTES
    assert noalloc_call(lib, Lf, batch=8, max_k=64) == ERR_SCRATCH
    # the measured shapes fit: batch 8 x 128000 (budget 4096), the 48-layer
    # step's layer, the ragged batch, every page of batch 8 x 128000
    for batch, max_k, P in [(8, 256, 16), (64, 128, 16), (32, 409, 32), (8, 8008, 16)]:
        Lm = layout(page_size=P, num_pool_pages=70000, max_pages_per_seq=8192)
        assert lib.quest_sparse_decode_workspace_bytes(ctypes.byref(Lm), batch, max_k) <= \
            quest.STATIC_SCRATCH_BYTES, (batch, max_k, P)


def test_probe_library_exports_and_rejections():
    """The measurement library (HBM read probes, include/quest_probe.h) loads,
    exports what its header declares, and rejects bad arguments before any
    launch."""
    from kv_cache_decode_quest_amd import probe
    L = probe.load()
    names = declared_functions(PROBE_HEADER)
    assert sorted(probe.EXPORTS) == names
    for name in names:
        assert hasattr(L, name)
    sink = ctypes.c_void_p(0x200000)
    assert L.quest_probe_stream_read(None, 1024, 4, 0, sink, None) == -1
    assert L.quest_probe_stream_read(FAKE, 1000, 4, 0, sink, None) == -2
    assert L.quest_probe_stream_read(ctypes.c_void_p(0x100008), 1024, 4, 0, sink, None) == -2
    assert L.quest_probe_stream_read(FAKE, 1024, 0, 0, sink, None) == -2
    assert L.quest_probe_stream_read(FAKE, 0, 4, 0, sink, None) == 0
    assert L.quest_probe_gather_read(FAKE, FAKE, None, 4, 4096, 4, 0, sink, None) == -1
    assert L.quest_probe_gather_read(FAKE, FAKE, FAKE, 4, 1000, 4, 0, sink, None) == -3
    assert L.quest_probe_gather_read(FAKE, FAKE, FAKE, -1, 4096, 4, 0, sink, None) == -2
    assert L.quest_probe_gather_read(FAKE, FAKE, FAKE, 0, 4096, 4, 0, sink, None) == 0
