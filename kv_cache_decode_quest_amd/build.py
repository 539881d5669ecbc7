"""Builds libquest.so in-tree with hipcc for gfx950.

    python -m kv_cache_decode_quest_amd.build

Every source is compiled on every call (objects under _build/, then linked).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libquest.so")
# HBM read probes (measurement only), a library of their own
PROBE_SOURCES = ["hbm_probe.hip"]
PROBE_PATH = os.path.join(HERE, "libquest_probe.so")

SOURCES = ["append_kv.hip", "page_scores.hip", "topk_pages.hip", "sparse_decode.hip",
           "static_scratch.hip", "plan.cpp", "quest_abi.cpp"]

ARCH = "gfx950"
# Packed fp32 instructions are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, path):
    tmp = path + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB_PATH)
    _link(objs[len(SOURCES):], PROBE_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {PROBE_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
