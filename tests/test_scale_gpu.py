"""GPU parity at scales other than a positive one: negative, zero and below
2^-100 in magnitude (the ABI takes any finite scale).

S = scale * Q K^T for any finite scale; the bf16 and FP8 forwards find the row
maximum on raw dot products, so they fold the sign of a negative scale into Q
and run the softmax with |scale| (at least 2^-100, with which every score of a
row is the same to fp32 rounding, as it is for any smaller scale); the
backward's recompute P^ = 2^(scale log2 e (q.k - LSE/scale)) holds for either
sign.  Every path is compared with the fp64 oracle at the same scale, with the
tolerances of the other parity tests.
"""
import math

import numpy as np
import pytest

import exact_tiled_attention_online_amd as fa
from exact_tiled_attention_online_amd import inputs as gen
from fp8_bound import lse_bar, stat_ratio
from gpu_util import LSE_ATOL, compare, log, oracle_heads, run_gpu, to_dev, to_np
from oracle import dropout as dref
from oracle import ref

pytestmark = pytest.mark.gpu

# -1/sqrt(d) and a sharper negative scale are set per head dim below
FIXED = [0.0, -0.0, 1e-38, -3e-31]


def _scales(d):
    return [-1.0 / math.sqrt(d), -3.0 / math.sqrt(d)] + FIXED


def _compare_all(x, dtype, causal, scale, where, method=fa.FA_DQ_HANDOFF):
    res = run_gpu(x, dtype, causal, scale, method=method)
    want = oracle_heads(x, causal, scale, heads=None)
    for (b, h), w in want.items():
        got = {n: res[n][b, h] for n in ("o", "lse", "dq", "dk", "dv")}
        compare(got, w, dtype, where=f"{where} head ({b},{h})")
    return res


CASES = [(dtype, d, causal, n) for dtype in ("bf16", "fp32") for d in (64, 96, 128) for causal in (False, True)
         for n in (129, 300)]
CASES += [(dtype, 256, causal, n) for dtype in ("bf16", "fp32") for causal in (False, True) for n in (129, 300)]


@pytest.mark.parametrize("dtype,d,causal,n", CASES)
def test_step_at_other_scales(dtype, d, causal, n):
    x = gen.make_inputs(gen.workload("c2"), shape=(1, 2, n, d), seed=4000 + n + d, dtype=dtype)
    methods = (fa.FA_DQ_HANDOFF, fa.FA_DQ_RECOMPUTE) if dtype == "bf16" else (fa.FA_DQ_RECOMPUTE,)
    for scale in _scales(d):
        for m in methods:
            log(f"[scale] {dtype} d={d} causal={causal} N={n} scale={scale:.3g} method={m}")
            res = _compare_all(x, dtype, causal, scale, f"{dtype} d{d} c{int(causal)} N{n} s{scale:.3g}", m)
            if scale == 0.0:
                # every probability of a row equal: the gradients through the
                # scores vanish exactly (0 times a finite accumulator)
                assert not np.any(res["dq"]) and not np.any(res["dk"]), "scale 0: dQ, dK must be 0"


@pytest.mark.parametrize("causal", [False, True])
def test_negative_scale_larger_size_sampled_heads(causal):
    """A causal/non-causal 2 x 8 x 2048 x 128 step with scale -1/sqrt(d), in the
    launch configuration of the large workloads (every workgroup full), on
    two whole heads."""
    B, H, N, d = 2, 8, 2048, 128
    scale = -1.0 / math.sqrt(d)
    log(f"[scale] 2x8x2048x128 causal={causal} scale={scale:.3g}")
    x = gen.make_inputs(gen.workload("c3"), shape=(B, H, N, d), seed=4100 + int(causal))
    res = run_gpu(x, "bf16", causal, scale)
    heads = [(0, 0), (B - 1, H - 1)]
    want = oracle_heads(x, causal, scale, heads=heads)
    for (b, h), w in want.items():
        compare({n: res[n][b, h] for n in ("o", "lse", "dq", "dk", "dv")}, w, "bf16", where=f"head ({b},{h})")


@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_at_other_scales(d, causal):
    import torch
    x = gen.make_fp8_inputs((1, 3, 300, d), seed=4200 + d, sigma_qk=2.0)
    q8, k8, v8 = (torch.from_numpy(x[n]).cuda() for n in ("q8", "k8", "v8"))
    for scale in _scales(d):
        log(f"[scale] fp8 d={d} causal={causal} scale={scale:.3g}")
        o, lse = fa.forward_fp8(q8, k8, v8, x["descale_q"], x["descale_k"], x["descale_v"], causal, scale)
        torch.cuda.synchronize()
        got_o, got_l = to_np(o), to_np(lse)
        o_ref, l_ref = ref.forward(x["q"], x["k"], x["v"], scale, causal)
        for h in range(3):
            bar_l = lse_bar(x["q"][0, h].astype(np.float64), x["k"][0, h].astype(np.float64), scale, causal)
            assert (np.abs(got_l[0, h] - l_ref[0, h]) <= bar_l).all(), (scale, h)
            r = stat_ratio(x["q"][0, h], x["k"][0, h], x["v"][0, h], got_o[0, h], scale, causal)
            assert r <= 1.0, (scale, h, r)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_split_forward_at_other_scales(dtype):
    import torch
    B, H, Nq, Nk, d = 2, 2, 7, 1000, 128
    for causal in (False, True):
        for scale in _scales(d):
            log(f"[scale] split {dtype} causal={causal} scale={scale:.3g}")
            if dtype == "bf16":
                xq = gen.make_inputs(gen.workload("c2"), shape=(B, H, Nq, d), seed=4300)
                xk = gen.make_inputs(gen.workload("c2"), shape=(B, H, Nk, d), seed=4301)
                q, k, v = to_dev(xq["q"], "bf16"), to_dev(xk["k"], "bf16"), to_dev(xk["v"], "bf16")
                o, lse = fa.forward_splitkv(q, k, v, causal, scale, num_splits=5)
                qv, kv_, vv = xq["q"], xk["k"], xk["v"]
            else:
                xq = gen.make_fp8_inputs((B, H, Nq, d), seed=4302, sigma_qk=2.0)
                xk = gen.make_fp8_inputs((B, H, Nk, d), seed=4303, sigma_qk=2.0)
                q8, k8, v8 = (torch.from_numpy(a).cuda() for a in (xq["q8"], xk["k8"], xk["v8"]))
                o, lse = fa.forward_splitkv_fp8(q8, k8, v8, xq["descale_q"], xk["descale_k"], xk["descale_v"],
                                                causal, scale, num_splits=5)
                qv, kv_, vv = xq["q"], xk["k"], xk["v"]
            torch.cuda.synchronize()
            got_o, got_l = to_np(o), to_np(lse)
            ro, rl = ref.forward_rect(qv, kv_, vv, scale, causal)
            for b in range(B):
                for h in range(H):
                    if dtype == "bf16":
                        assert float(np.abs(got_l[b, h] - rl[b, h]).max()) <= LSE_ATOL, (scale, b, h)
                    else:
                        bar_l = lse_bar(qv[b, h].astype(np.float64), kv_[b, h].astype(np.float64), scale, causal)
                        assert (np.abs(got_l[b, h] - rl[b, h]) <= bar_l).all(), (scale, b, h)
                    if dtype == "bf16":
                        tol = 2e-2 * max(1e-2, float(np.abs(ro[b, h]).max()))
                    else:
                        vmax = float(np.abs(vv[b, h]).max())
                        tol = (2.0 ** -4 + Nk * 2.0 ** -17) * vmax + 2.0 ** -9 * float(np.abs(ro[b, h]).max())
                    assert float(np.abs(got_o[b, h] - ro[b, h]).max()) <= tol, (scale, b, h)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_at_negative_scale(causal):
    from test_dropout_gpu import compare_dropout, run_dropout
    d, scale, t, seed, off = 128, -1.0 / math.sqrt(128), 26, 91, 5
    log(f"[scale] dropout causal={causal} scale={scale:.3g}")
    x = gen.make_inputs(gen.workload("c2"), shape=(1, 2, 300, d), seed=4400)
    for method in (fa.FA_DQ_HANDOFF, fa.FA_DQ_RECOMPUTE):
        got = run_dropout(x, causal, scale, t, seed, off, method=method)
        want = dref.forward_backward_dropout(x["q"], x["k"], x["v"], x["do"], scale, causal, seed, off, t)
        for (b, h), w in want.items():
            compare_dropout({n: got[n][b, h] for n in w}, w, x, b, h, scale, causal,
                            f"dropout method {method} head ({b},{h})")
