"""Builds libfa.so (gfx950) in-tree with hipcc.

    python -m exact_tiled_attention_online_amd.build [-v]

Every HIP source under csrc/ is compiled for gfx950 only, in parallel, then
linked into exact_tiled_attention_online_amd/libfa.so.  The compiler's
per-kernel resource report (VGPR/AGPR/LDS/scratch) is kept in
_build/resource_usage.txt at the repository root.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["fa_fwd_bf16.hip", "fa_fwd_fp8.hip", "fa_bwd_bf16.hip", "fa_bwd_kv256.hip", "fa_bwd_dq.hip",
           "fa_bwd_dq_ds.hip", "fa_aux.hip", "fa_fp32.hip", "fa_noalloc.hip", "fa_api.cpp"]

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in device code.
# -amdgpu-mfma-vgpr-form: MFMA results in VGPRs where they fit, so that fewer
# accumulators have to be copied out of AGPRs before vector work (measured
# about 2% on the dK/dV kernel).
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-munsafe-fp-atomics",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form",
                "-Rpass-analysis=kernel-resource-usage", "-Wno-unused-command-line-argument"]


def _compile(src: str):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + DEVICE_FLAGS + ["-I", os.path.join(ROOT, "include"), "-c", path, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, r.returncode, r.stdout + r.stderr, cmd


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    objs, report, failed = [], [], []
    with cf.ThreadPoolExecutor(jobs) as ex:
        for src, obj, rc, out, cmd in ex.map(_compile, SOURCES):
            objs.append(obj)
            report.append(f"==== {src}\n{out}")
            if rc != 0:
                failed.append((src, out, cmd))
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write("\n".join(report))
    if failed:
        msg = "\n".join(f"{s}: {' '.join(c)}\n{o[-4000:]}" for s, o, c in failed)
        raise RuntimeError("hipcc failed:\n" + msg)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("\n".join(report))
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
