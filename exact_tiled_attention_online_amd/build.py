"""Builds libfa.so (gfx950) in-tree with hipcc.

    python -m exact_tiled_attention_online_amd.build [-v]

Every HIP source under csrc/ is compiled for gfx950 only, in parallel, then
linked into exact_tiled_attention_online_amd/libfa.so.  The compiler's
per-kernel resource report (VGPR/AGPR/LDS/scratch) is kept in
_build/resource_usage.txt at the repository root.

Two checking variants are built beside it from the same sources (the tests
load them side by side with libfa.so):
  libfa_debug_sync.so  FA_DEBUG_SYNC: a full barrier after every prefetch of
                       a next tile; results must be bit-identical;
  libfa_tile_alt.so    another tile configuration (4-wave forward and dQ
                       workgroups, other operand read distances); results
                       must meet the same oracle bar.
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
# checking variants: name -> extra device flags
VARIANTS = {
    "debug_sync": ["-DFA_DEBUG_SYNC"],
    "tile_alt": ["-DFA_FWD_NW=4", "-DFA_DQ_NW=4", "-DFA_FWD_DIST=2", "-DFA_KV_DIST=2", "-DFA_DQ_DIST=2"],
}


def variant_path(name=None):
    """The built library of a variant (None: the library itself)."""
    return LIB if name is None else os.path.join(PKG, f"libfa_{name}.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["fa_fwd_bf16.hip", "fa_fwd_fp8.hip", "fa_bwd_bf16.hip", "fa_bwd_kv256.hip", "fa_bwd_kv256_drop.hip",
           "fa_bwd_kv2.hip", "fa_bwd_dq.hip",
           "fa_bwd_dq_ds.hip", "fa_aux.hip", "fa_fp32.hip", "fa_noalloc.hip", "fa_api.cpp"]

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in device code.
# -amdgpu-mfma-vgpr-form: MFMA results in VGPRs where they fit, so that fewer
# accumulators have to be copied out of AGPRs before vector work (measured
# about 2% on the dK/dV kernel).
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-munsafe-fp-atomics",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form",
                "-Rpass-analysis=kernel-resource-usage", "-Wno-unused-command-line-argument"]


def _compile(job):
    src, variant = job
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, (variant + "." if variant else "") + src + ".o")
    extra = VARIANTS[variant] if variant else []
    cmd = [HIPCC] + DEVICE_FLAGS + extra + ["-I", os.path.join(ROOT, "include"), "-c", path, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, variant, obj, r.returncode, r.stdout + r.stderr, cmd


def build(verbose: bool = False, variants=tuple(VARIANTS)) -> str:
    os.makedirs(BUILD, exist_ok=True)
    names = [None] + list(variants)
    jobs_list = [(src, v) for v in names for src in SOURCES]
    jobs = max(1, min(8, os.cpu_count() or 1))
    objs = {v: [] for v in names}
    report, failed = [], []
    with cf.ThreadPoolExecutor(jobs) as ex:
        for src, v, obj, rc, out, cmd in ex.map(_compile, jobs_list):
            objs[v].append(obj)
            if v is None:
                report.append(f"==== {src}\n{out}")
            if rc != 0:
                failed.append((src, out, cmd))
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write("\n".join(report))
    if failed:
        msg = "\n".join(f"{s}: {' '.join(c)}\n{o[-4000:]}" for s, o, c in failed)
        raise RuntimeError("hipcc failed:\n" + msg)
    for v in names:
        lib = variant_path(v)
        tmp = lib + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs[v]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
        os.replace(tmp, lib)
        if verbose:
            print("built", lib)
    if verbose:
        print("\n".join(report))
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, variants=() if "--no-variants" in sys.argv else tuple(VARIANTS))
