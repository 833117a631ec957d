"""Shared helpers of the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, run the fp64 oracle on the same values, compare.

Tolerances (stated per tensor): fp32 workloads max|gpu - ref| <= 1e-4 for
O, dQ, dK, dV; bf16 workloads max|gpu - ref| <= 2e-2 * max|ref| for each of
O, dQ, dK, dV; LSE max-abs <= 1e-3 for both.  Where a gradient is identically
zero by construction (N = 1, K = 0, constant V), 2e-2 * max|ref| is 0 while
the kernel reaches the zero through cancellation of rounded O(1) terms, so
the bf16 bar takes max|ref| as at least BF16_REF_FLOOR.
"""
from __future__ import annotations

import sys

import numpy as np

import exact_tiled_attention_online_amd as fa
from oracle import ref

FP32_ATOL = 1e-4
BF16_RTOL_OF_MAX = 2e-2
LSE_ATOL = 1e-3
BF16_REF_FLOOR = 1e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x, dtype, layout=0):
    """Upload a [B,H,N,d] array (or [B,H,N]) in the named layout."""
    import torch
    a = np.asarray(x, dtype=np.float32)
    if layout == fa.FA_LAYOUT_BNHD and a.ndim == 4:
        a = a.transpose(0, 2, 1, 3)
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def to_np(t, layout=0):
    """Download a device tensor as fp64 numpy, back in [B,H,N,d] order."""
    a = t.float().cpu().numpy().astype(np.float64)
    if layout == fa.FA_LAYOUT_BNHD and a.ndim == 4:
        a = np.ascontiguousarray(a.transpose(0, 2, 1, 3))
    return a


def run_gpu(x, dtype, causal, scale, bwd=True, stream=None, layout=0, method=fa.FA_DQ_HANDOFF):
    """fwd (+ bwd, with a workspace sized for the dQ method `method`) on
    device; returns dict of fp64 numpy arrays in [B,H,N,d] order whatever the
    device layout."""
    import torch
    q, k, v, do = (to_dev(x[n], dtype, layout) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal, scale, stream=stream, layout=layout)
    out = {"o_dev": o, "lse_dev": lse}
    if bwd:
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, causal, scale, stream=stream, layout=layout, method=method)
        out.update(dq_dev=dq, dk_dev=dk, dv_dev=dv)
    torch.cuda.synchronize()
    res = {"o": to_np(o, layout), "lse": to_np(lse)}
    if bwd:
        res.update(dq=to_np(dq, layout), dk=to_np(dk, layout), dv=to_np(dv, layout))
    res["_dev"] = out
    return res


def oracle_heads(x, causal, scale, heads):
    return ref.forward_backward(x["q"], x["k"], x["v"], x["do"], scale, causal, heads=heads)


def compare(gpu, want, dtype, names=("o", "lse", "dq", "dk", "dv"), where=""):
    """Assert the tolerances above; returns the max errors found."""
    errs = {}
    for n in names:
        g, r = np.asarray(gpu[n]), np.asarray(want[n])
        assert g.shape == r.shape, (n, g.shape, r.shape)
        assert np.isfinite(g).all(), f"{where} {n}: non-finite values"
        err = float(np.abs(g - r).max()) if g.size else 0.0
        errs[n] = err
        if n == "lse":
            tol = LSE_ATOL
        elif dtype == "fp32":
            tol = FP32_ATOL
        else:
            tol = BF16_RTOL_OF_MAX * max(BF16_REF_FLOOR, float(np.abs(r).max()))
        assert err <= tol, f"{where} {n}: max abs err {err:.3e} > tol {tol:.3e}"
    return errs


def head_slice(res, b, h):
    return {n: res[n][b, h] for n in ("o", "lse", "dq", "dk", "dv") if n in res}
