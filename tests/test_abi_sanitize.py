"""The C ABI's host code under the host address and undefined-behaviour
sanitizers.

quest_abi.cpp (validation, dispatch) and plan.cpp (launch plans, workspace
sizes) are built with g++ -fsanitize=address,undefined, with the kernel
launchers replaced by host stand-ins (tests/abi_sanitize_stubs.cpp), and
driven by tests/abi_sanitize_driver.c: every entry point of include/quest.h,
each documented rejection (which must launch nothing), and a seeded sweep of
layouts and sizes with extreme values (the 1Cat page, "Change a native
binding": reject unsupported combinations before doing any work).  Any
sanitizer report fails it.  CPU only; no HIP library or GPU is involved.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_decode_quest_amd", "csrc")


def test_abi_host_code_clean_under_asan_ubsan(tmp_path):
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    rocm_inc = "/opt/rocm/include"
    if gxx is None or gcc is None:
        pytest.skip("g++/gcc not found")
    if not os.path.isdir(os.path.join(rocm_inc, "hip")):
        pytest.skip("HIP runtime headers not found")
    san = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=undefined", "-Wall", "-Wextra"]
    inc = ["-D__HIP_PLATFORM_AMD__", "-I", rocm_inc, "-I", os.path.join(ROOT, "include"),
           "-I", CSRC]
    objs = []
    for src in (os.path.join(CSRC, "quest_abi.cpp"), os.path.join(CSRC, "plan.cpp"),
                os.path.join(ROOT, "tests", "abi_sanitize_stubs.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        build = subprocess.run([gxx, "-std=c++17", *san, *inc, "-c", src, "-o", obj],
                               capture_output=True, text=True)
        if build.returncode != 0 and "asan" in (build.stderr + build.stdout).lower():
            pytest.skip("the sanitizer runtime is not installed: " + build.stderr[-300:])
        assert build.returncode == 0, build.stderr
        objs.append(obj)
    drv = str(tmp_path / "abi_sanitize_driver.o")
    build = subprocess.run([gcc, "-std=c11", *san, "-I", os.path.join(ROOT, "include"), "-c",
                            os.path.join(ROOT, "tests", "abi_sanitize_driver.c"), "-o", drv],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    exe = str(tmp_path / "abi_sanitize_driver")
    link = subprocess.run([gxx, *san, drv, *objs, "-o", exe], capture_output=True, text=True)
    assert link.returncode == 0, link.stderr
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "abi driver ok" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
