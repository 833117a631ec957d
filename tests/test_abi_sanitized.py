"""The C-ABI layer (argument checks, workspace sizing and carving, the dQ
method choice, split planning) under AddressSanitizer and UndefinedBehavior-
Sanitizer, on the host.

fa_api.cpp is built with g++ (no GPU code) and linked against the host
stand-ins of tests/host_stubs/fa_launch_stubs.cpp, which touch every byte of
the workspace regions the real kernels use.  tests/host_stubs/abi_calls.py
then drives every entry point with exact-size host workspaces over ragged
shapes, every head dim, both masks, both dtypes, both layouts and every dQ
method, plus huge and invalid shapes.  A region carved past the size the
library reported, or signed overflow in the size arithmetic, aborts the run.

A second build plants a sizing mistake (the dS buffer's sink shrunk by half)
and must be caught, so a clean run means something.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_tiled_attention_online_amd", "csrc")
STUBS = os.path.join(ROOT, "tests", "host_stubs")


def _tool(name):
    p = shutil.which(name)
    if not p:
        pytest.skip(f"{name} not found")
    return p


def _runtime(lib):
    out = subprocess.run([_tool("g++"), f"-print-file-name={lib}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        pytest.skip(f"{lib} not available")
    return out


def _build(tmp_path, api_src, name):
    so = str(tmp_path / name)
    cmd = [_tool("g++"), "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=undefined", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           api_src, os.path.join(STUBS, "fa_launch_stubs.cpp"), "-o", so]
    if not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("HIP headers not found")
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return so


def _run(so):
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.pop("FA_DQ_MODE", None)
    return subprocess.run([sys.executable, os.path.join(STUBS, "abi_calls.py"), so], capture_output=True,
                          text=True, env=env, timeout=300, cwd=str(os.path.dirname(so)))


def test_abi_clean_under_asan_ubsan(tmp_path):
    so = _build(tmp_path, os.path.join(CSRC, "fa_api.cpp"), "libfa_host_san.so")
    r = _run(so)
    log = r.stdout + r.stderr
    assert r.returncode == 0, log[-6000:]
    assert "ALL OK" in r.stdout
    assert "runtime error" not in log and "AddressSanitizer" not in log, log[-6000:]


def test_planted_workspace_mistake_is_caught(tmp_path):
    with open(os.path.join(CSRC, "fa_api.cpp")) as f:
        src = f.read()
    planted = src.replace("constexpr size_t kDsSink = 4096;", "constexpr size_t kDsSink = 2048;")
    assert planted != src, "the sink constant moved; update the planted mistake"
    planted = planted.replace('#include "../../include/fa.h"', '#include "fa.h"')
    api = tmp_path / "fa_api_planted.cpp"
    api.write_text(planted)
    so = _build(tmp_path, str(api), "libfa_host_planted.so")
    r = _run(so)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr, r.stderr[-4000:]
