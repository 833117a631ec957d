"""The two checking builds of the library against the same calls.

libfa_debug_sync.so (FA_DEBUG_SYNC) puts a full workgroup barrier after every
prefetch of a next tile, so that no read can run ahead of a load into LDS
and no wave can refill a buffer another wave still reads.  The kernels
pipeline their LDS buffers with a single barrier per tile (and, in the dS
hand-off kernels, barriers that deliberately leave stores outstanding); a
missing wait there would show as a difference from the checking library.  Every output
must be bit-identical.

libfa_tile_alt.so is another tile configuration: 4-wave forward and
recomputing-dQ workgroups (128 query rows instead of 256) and other operand
read distances in the dK/dV, dQ and forward pipelines.  Its outputs must meet
the oracle bar.

The two-waves-per-SIMD dK/dV kernel (FA_KV_KERNEL=2, d = 128) is held to
the oracle bar and to the same bit identity with the checking build.
"""
import math
import os

import numpy as np
import pytest

import exact_tiled_attention_online_amd as fa
from exact_tiled_attention_online_amd import _lib
from exact_tiled_attention_online_amd import build as fab
from exact_tiled_attention_online_amd import inputs as gen
from gpu_util import compare, log, oracle_heads, run_gpu, to_dev, to_np
from oracle import ref

pytestmark = pytest.mark.gpu

DEBUG = fab.variant_path("debug_sync")
ALT = fab.variant_path("tile_alt")

# (B, H, N, d, causal)
SHAPES = [(1, 4, 1000, 128, True), (2, 3, 700, 64, False), (1, 3, 333, 96, True), (1, 2, 600, 256, True),
          (1, 2, 129, 128, False)]


def _step(x, d, causal, method):
    """Plain fwd + bwd (given dQ method), FP8 fwd, split fwd and dropout
    fwd + bwd on the same inputs; every output as a device tensor."""
    import torch
    scale = 1.0 / math.sqrt(d)
    out = {}
    r = run_gpu(x, "bf16", causal, scale, method=method)["_dev"]
    out.update({f"plain_{k}": v for k, v in r.items()})
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.forward_dropout(q, k, v, causal, scale, 0.125, seed=77, offset=3)
    g = fa.backward_dropout(q, k, v, o, do, lse, causal, scale, 0.125, seed=77, offset=3, method=method)
    out.update(drop_o=o, drop_lse=lse, drop_dq=g[0], drop_dk=g[1], drop_dv=g[2])
    if d != 256:
        qs = q[:, :, :7].contiguous()
        out["split_o"], out["split_lse"] = fa.forward_splitkv(qs, k, v, causal, scale, num_splits=3)
    if d == 128:
        x8 = gen.make_fp8_inputs(tuple(x["q"].shape), seed=11)
        q8, k8, v8 = (torch.from_numpy(x8[n]).cuda() for n in ("q8", "k8", "v8"))
        out["fp8_o"], out["fp8_lse"] = fa.forward_fp8(q8, k8, v8, x8["descale_q"], x8["descale_k"],
                                                      x8["descale_v"], causal, scale)
    torch.cuda.synchronize()
    return {k: v.clone() for k, v in out.items()}


@pytest.mark.parametrize("B,H,N,d,causal", SHAPES)
@pytest.mark.parametrize("method", [fa.FA_DQ_HANDOFF, fa.FA_DQ_RECOMPUTE])
def test_debug_sync_build_gives_the_same_bits(B, H, N, d, causal, method):
    import torch
    log(f"[debug-sync] B={B} H={H} N={N} d={d} causal={causal} method={method}")
    x = gen.make_inputs(gen.workload("c3"), shape=(B, H, N, d), seed=N + d)
    a = _step(x, d, causal, method)
    with _lib.using_library(DEBUG):
        b = _step(x, d, causal, method)
    for name in a:
        assert torch.equal(a[name], b[name]), f"{name} differs from the build with a barrier after every prefetch"


@pytest.mark.parametrize("B,H,N,d,causal", SHAPES + [(1, 8, 4099, 128, True)])
@pytest.mark.parametrize("method", [fa.FA_DQ_HANDOFF, fa.FA_DQ_RECOMPUTE])
def test_other_tile_configuration_meets_the_bar(B, H, N, d, causal, method):
    log(f"[tile-alt] B={B} H={H} N={N} d={d} causal={causal} method={method}")
    x = gen.make_inputs(gen.workload("c3"), shape=(B, H, N, d), seed=N + d + 1)
    scale = 1.0 / math.sqrt(d)
    heads = [(0, 0), (B - 1, H - 1)]
    want = oracle_heads(x, causal, scale, heads=heads)
    with _lib.using_library(ALT):
        res = run_gpu(x, "bf16", causal, scale, method=method)
    for bh, wv in want.items():
        compare({n: res[n][bh] for n in wv}, wv, "bf16", where=f"tile-alt d{d} N{N} head {bh}")


def test_variant_libraries_are_built_from_the_same_sources():
    for path in (DEBUG, ALT):
        assert os.path.exists(path), path


# the two-waves-per-SIMD dK/dV kernel (d = 128, selected per call with
# FA_KV_KERNEL=2): ragged tails, both masks, both dQ methods
KV2_CASES = [(1, 2, n, causal) for n in (1, 17, 64, 129, 300) for causal in (False, True)]
KV2_CASES += [(2, 3, 1000, True), (1, 4, 4099, False)]


@pytest.mark.parametrize("B,H,N,causal", KV2_CASES)
@pytest.mark.parametrize("method", [fa.FA_DQ_HANDOFF, fa.FA_DQ_RECOMPUTE])
def test_two_wave_dkdv_kernel_meets_the_bar(monkeypatch, B, H, N, causal, method):
    log(f"[kv2] B={B} H={H} N={N} causal={causal} method={method}")
    monkeypatch.setenv("FA_KV_KERNEL", "2")
    x = gen.make_inputs(gen.workload("c3"), shape=(B, H, N, 128), seed=N + 5)
    scale = 1.0 / math.sqrt(128)
    res = run_gpu(x, "bf16", causal, scale, method=method)
    want = oracle_heads(x, causal, scale, heads=None)
    for (b, h), w in want.items():
        got = {n: res[n][b, h] for n in ("o", "lse", "dq", "dk", "dv")}
        compare(got, w, "bf16", where=f"kv2 N{N} c{int(causal)} head ({b},{h})")


@pytest.mark.parametrize("B,H,N,causal", [(1, 4, 1000, True), (1, 2, 129, False)])
@pytest.mark.parametrize("method", [fa.FA_DQ_HANDOFF, fa.FA_DQ_RECOMPUTE])
def test_two_wave_dkdv_kernel_debug_sync_same_bits(monkeypatch, B, H, N, causal, method):
    import torch
    log(f"[kv2 debug-sync] B={B} H={H} N={N} causal={causal} method={method}")
    monkeypatch.setenv("FA_KV_KERNEL", "2")
    x = gen.make_inputs(gen.workload("c3"), shape=(B, H, N, 128), seed=N + 6)
    a = _step(x, 128, causal, method)
    with _lib.using_library(DEBUG):
        b = _step(x, 128, causal, method)
    for name in a:
        assert torch.equal(a[name], b[name]), f"{name} differs from the build with a barrier after every prefetch"
