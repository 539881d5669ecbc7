"""The fp64 oracle under the host address and undefined-behaviour sanitizers.

tests/oracle_sanitize_driver.c calls every oracle entry point on a tiny paged
cache (fp32 and bf16, a partial last page, a permuted page table, unused pool
pages) and checks identities that hold on any input (a budget covering every
page reproduces dense attention; one page's bounds equal its row of the
request's bounds; the selection is the top k under (score desc, page asc)).
Built with gcc -fsanitize=address,undefined; any sanitizer report fails it.
CPU only.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_clean_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_sanitize_driver")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined", "-Wall", "-Wextra",
           "-Werror", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "quest_oracle.c"), "-lm", "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in (build.stderr + build.stdout).lower():
        pytest.skip("the sanitizer runtime is not installed: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "oracle driver ok" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
