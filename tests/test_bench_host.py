"""Host logic of bench.py, checked without a GPU: the algorithmic byte count
of a step, the counter-record arithmetic behind `roofline.traffic`, the
source-hash guard on that record, and the one-GPU refusal."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import torch

import bench
from kv_cache_decode_quest_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_step_bytes_hand_count():
    """Two requests, 2 KV heads, D 128, P 16, bf16.  Metadata: every live page
    of every KV head, 512 B each.  K/V: the valid tokens of each selected page
    only (entries past num_sel, -1 here, never count)."""
    w = workloads.Workload("hand", 2, 16, 2, 128, 16, "bf16", ctx=32)
    ctx_after = torch.tensor([33, 16], dtype=torch.int32)       # 3 pages and 1 page
    sel = torch.tensor([[[0, 2, -1], [1, -1, -1]],
                        [[0, -1, -1], [0, -1, -1]]], dtype=torch.int32)
    nsel = torch.tensor([[2, 1], [1, 1]], dtype=torch.int32)
    meta, kv = bench.step_bytes(w, ctx_after, sel, nsel)
    assert meta == (3 + 1) * 2 * 512
    tokens = (16 + 1) + 16 + 16 + 16                            # page 2 of request 0 holds 1
    assert kv == tokens * 2 * 128 * 2


def _pmc_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_from_pmc_scales_by_the_copy(tmp_path):
    """Per-launch bytes = mean raw KiB of the scoring kernel x 1024 x (known
    copy bytes / what the same counter read for the copy); the copy is the
    mean of the three largest buffer copies; other kernels are ignored."""
    scores = "void quest::page_scores_mfma_kernel<128, true>(int)"
    copy = "__amd_rocclr_copyBuffer"
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _pmc_csv(fetch, "FETCH_SIZE", [(scores, 1000.0), (scores, 1200.0), (copy, 3.0),
                                   (copy, 500.0), (copy, 500.0), (copy, 500.0),
                                   ("quest::merge_kernel", 99999.0)])
    _pmc_csv(write, "WRITE_SIZE", [(scores, 10.0), (scores, 30.0), (copy, 1.0),
                                   (copy, 1000.0), (copy, 1000.0), (copy, 1000.0)])
    copy_bytes = 1024 * 1024
    rec = bench.traffic_from_pmc(str(fetch), str(write), copy_bytes)
    f_scale = copy_bytes / (500.0 * 1024)
    w_scale = copy_bytes / (1000.0 * 1024)
    assert abs(rec["fetch_scale"] - f_scale) < 1e-12
    assert abs(rec["write_scale"] - w_scale) < 1e-12
    assert abs(rec["fetch_bytes_per_launch"] - 1100.0 * 1024 * f_scale) < 1e-6
    assert abs(rec["write_bytes_per_launch"] - 20.0 * 1024 * w_scale) < 1e-6
    assert rec["bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert rec["source_hash"] == bench.source_hash(bench.SCORE_SOURCES)


def test_traffic_reported_only_for_the_current_source(tmp_path, monkeypatch):
    rec = {"bytes_per_launch": 123.0, "workload": "bench128k",
           "source_hash": bench.source_hash(bench.SCORE_SOURCES)}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(path))
    assert bench.measured_traffic("bench128k") == 123.0
    # a record of another workload's launches says nothing about this one's
    assert bench.measured_traffic("ragged") is None
    rec["source_hash"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic("bench128k") is None
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("bench128k") is None


def test_committed_traffic_record_is_consistent():
    """The committed counter record: fetch + write = total, and at least the
    algorithmic bytes of a bench128k launch (131,088,384 B of metadata)."""
    rec = json.load(open(bench.TRAFFIC_JSON))
    assert abs(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
               - rec["bytes_per_launch"]) < 1.0
    assert rec["bytes_per_launch"] >= 131088384


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""
