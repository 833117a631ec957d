"""GPU parity of fa_fwd / fa_bwd (through the C ABI) against the fp64 oracle.

Small and ragged shapes are compared element by element on every head; the
five workloads run at their full sizes in the same launch configuration the
benchmark uses, and are compared on whole sampled heads (heads are
independent, so a head is an output the oracle can compute on its own), plus
properties that hold at any size.
"""
import math

import numpy as np
import pytest

import exact_tiled_attention_online_amd as fa
from exact_tiled_attention_online_amd import inputs as gen
from gpu_util import compare, log, oracle_heads, run_gpu, to_dev, to_np

pytestmark = pytest.mark.gpu


def _full_compare(x, dtype, causal, scale, where, layout=0, method=fa.FA_DQ_HANDOFF):
    res = run_gpu(x, dtype, causal, scale, layout=layout, method=method)
    B, H = x["q"].shape[:2]
    want = oracle_heads(x, causal, scale, heads=None)
    errs = {}
    for (b, h), w in want.items():
        got = {n: res[n][b, h] for n in ("o", "lse", "dq", "dk", "dv")}
        e = compare(got, w, dtype, where=f"{where} head ({b},{h})")
        for n, v in e.items():
            errs[n] = max(errs.get(n, 0.0), v)
    return errs, res


# bf16 runs both dQ methods (the dS hand-off and the recompute kernel); fp32
# has only the recompute kernels
EDGE = [(dtype, d, causal, n, m)
        for dtype in ("bf16", "fp32")
        for d in (64, 96, 128)
        for causal in (False, True)
        for n in (1, 17, 64, 129, 300)
        for m in ((fa.FA_DQ_HANDOFF, fa.FA_DQ_RECOMPUTE) if dtype == "bf16" else (fa.FA_DQ_RECOMPUTE,))]
# head dim 256 (fp32: four lanes per row in the forward, eight in the backward)
EDGE += [("bf16", 256, causal, n, m) for causal in (False, True) for n in (1, 17, 64, 129, 300)
         for m in (fa.FA_DQ_HANDOFF, fa.FA_DQ_RECOMPUTE)]
EDGE += [("fp32", 256, causal, n, fa.FA_DQ_RECOMPUTE) for causal in (False, True) for n in (1, 17, 64, 129, 300)]
METHOD_NAME = {fa.FA_DQ_HANDOFF: "handoff", fa.FA_DQ_RECOMPUTE: "recompute", fa.FA_DQ_ATOMIC: "atomic"}


@pytest.mark.parametrize("dtype,d,causal,n,method", EDGE)
def test_small_and_ragged(dtype, d, causal, n, method):
    log(f"[edge] dtype={dtype} d={d} causal={causal} N={n} dq={METHOD_NAME[method]}")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(1, 2, n, d), seed=1000 + n + d, dtype=dtype)
    _full_compare(x, dtype, causal, 1.0 / math.sqrt(d), f"edge {dtype} d{d} c{int(causal)} N{n}", method=method)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_other_scale_and_spread(dtype, causal):
    log(f"[scale] dtype={dtype} causal={causal}")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(2, 3, 200, 64), seed=77, sigma_qk=2.0, dtype=dtype)
    _full_compare(x, dtype, causal, 0.3, f"scale0.3 {dtype} c{int(causal)}")


def test_workload_c1_fp32():
    w = gen.workload("c1")
    log(f"[workload] {w.name}")
    x = gen.make_inputs(w)
    errs, _ = _full_compare(x, "fp32", w.causal, w.scale, w.name)
    log(f"  max errors {errs}")


def test_workload_c2_bf16():
    w = gen.workload("c2")
    log(f"[workload] {w.name}")
    x = gen.make_inputs(w)
    errs, _ = _full_compare(x, "bf16", w.causal, w.scale, w.name)
    log(f"  max errors {errs}")


# the first, a middle and the last head of each workload
SAMPLED = {"c3": [(0, 0), (1, 7), (1, 15)], "c4": [(0, 0), (0, 15), (0, 31)], "c5": [(0, 0), (0, 4), (0, 7)]}


@pytest.fixture(scope="module")
def big_runs():
    cache = {}

    def get(key):
        if key not in cache:
            w = gen.workload(key)
            log(f"[workload] {w.name}: inputs")
            x = gen.make_inputs(w)
            log(f"[workload] {w.name}: gpu fwd+bwd")
            res = run_gpu(x, "bf16", w.causal, w.scale, bwd=True)
            cache.clear()
            cache[key] = (w, x, res)
        return cache[key]

    return get


@pytest.mark.parametrize("key", ["c3", "c4", "c5"])
def test_full_size_sampled_heads(big_runs, key):
    w, x, res = big_runs(key)
    for b, h in SAMPLED[key]:
        log(f"[workload] {w.name}: oracle head ({b},{h})")
        want = oracle_heads(x, w.causal, w.scale, heads=[(b, h)])[(b, h)]
        got = {n: res[n][b, h] for n in ("o", "lse", "dq", "dk", "dv")}
        errs = compare(got, want, "bf16", where=f"{w.name} head ({b},{h})")
        log(f"  max errors {errs}")


@pytest.mark.parametrize("key", ["c3", "c4", "c5"])
def test_full_size_invariants(big_runs, key):
    """Sum_j dK_j = 0, Sum_j dV_j = Sum_i dO_i, O within the per-column range of V,
    on every head (consequences of sum_j dS_ij = 0 and of stochastic rows)."""
    w, x, res = big_runs(key)
    log(f"[invariants] {w.name}")
    dk_sum = res["dk"].sum(axis=2)
    dv_sum = res["dv"].sum(axis=2)
    do_sum = x["do"].astype(np.float64).sum(axis=2)
    # each row sum is over N bf16-rounded values; allow bf16 rounding per term
    n = w.N
    tol_k = 2e-2 * np.abs(res["dk"]).max() * math.sqrt(n)
    tol_v = 2e-2 * np.abs(res["dv"]).max() * math.sqrt(n)
    assert np.abs(dk_sum).max() <= tol_k, (np.abs(dk_sum).max(), tol_k)
    assert np.abs(dv_sum - do_sum).max() <= tol_v, (np.abs(dv_sum - do_sum).max(), tol_v)
    v = x["v"].astype(np.float64)
    if not w.causal:
        hi, lo = v.max(axis=2, keepdims=True), v.min(axis=2, keepdims=True)
    else:
        hi = np.maximum.accumulate(v, axis=2)
        lo = np.minimum.accumulate(v, axis=2)
    slack = 1e-2 * np.abs(v).max()
    assert (res["o"] <= hi + slack).all() and (res["o"] >= lo - slack).all()
    assert np.isfinite(res["lse"]).all()


@pytest.mark.parametrize("key,d", [("c4", 128), ("c3", 128), ("c2", 64), ("c3", 96), ("c3", 256)])
def test_dq_methods_at_size(key, d):
    """The dS hand-off against the recompute kernel, in the benchmark's launch
    configuration: dK and dV come from the same arithmetic in both (the
    hand-off kernel only adds the dS stores), so they must be bit-identical;
    dQ differs in rounding only, and both meet the oracle bar on sampled
    heads (the first and the last)."""
    import torch
    w = gen.workload(key)
    B, H, N = w.shape[:3]
    if d != w.shape[3]:   # the workload's geometry at another head dim
        B, H = 1, 8
    log(f"[dq methods] {w.name} B={B} H={H} N={N} d={d}")
    x = gen.make_inputs(w, shape=(B, H, N, d), seed=4000 + d)
    a = run_gpu(x, "bf16", w.causal, 1.0 / math.sqrt(d), method=fa.FA_DQ_HANDOFF)
    b = run_gpu(x, "bf16", w.causal, 1.0 / math.sqrt(d), method=fa.FA_DQ_RECOMPUTE)
    for n in ("o", "lse", "dk", "dv"):
        assert np.array_equal(a[n], b[n]), f"{n} differs between the dQ methods"
    heads = [(0, 0), (B - 1, H - 1)]
    want = oracle_heads(x, w.causal, 1.0 / math.sqrt(d), heads=heads)
    for bh, wv in want.items():
        for name, r in (("handoff", a), ("recompute", b)):
            errs = compare({"dq": r["dq"][bh]}, wv, "bf16", names=("dq",), where=f"{name} {w.name} d{d} head {bh}")
            log(f"  {name} head {bh} dq max error {errs['dq']:.3e}")
    del a, b
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_keys_and_constant_values(dtype, causal):
    log(f"[special] dtype={dtype} causal={causal}")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(1, 2, 256, 128), seed=9, dtype=dtype)
    x0 = dict(x, k=np.zeros_like(x["k"]))
    _full_compare(x0, dtype, causal, 1 / math.sqrt(128), f"K=0 {dtype}")
    vc = np.broadcast_to(x["v"][:, :, :1, :], x["v"].shape).copy()
    xc = dict(x, v=vc)
    _full_compare(xc, dtype, causal, 1 / math.sqrt(128), f"V const {dtype}")


@pytest.mark.parametrize("causal", [False, True])
def test_backward_alone_from_oracle_forward(causal):
    """fa_bwd fed the oracle's O (rounded to bf16) and LSE: isolates the backward's error."""
    import torch
    log(f"[bwd-only] causal={causal}")
    w = gen.workload("c3")
    x = gen.make_inputs(w, shape=(1, 2, 1024, 128), seed=31)
    want = oracle_heads(x, causal, w.scale, heads=None)
    o = np.stack([want[(0, h)]["o"] for h in range(2)])[None].astype(np.float32)
    lse = np.stack([want[(0, h)]["lse"] for h in range(2)])[None].astype(np.float32)
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    od = to_dev(o, "bf16")
    ld = torch.from_numpy(lse).cuda()
    dq, dk, dv = fa.backward(q, k, v, od, do, ld, causal, w.scale)
    torch.cuda.synchronize()
    for h in range(2):
        got = {"dq": to_np(dq[0, h]), "dk": to_np(dk[0, h]), "dv": to_np(dv[0, h])}
        compare(got, want[(0, h)], "bf16", names=("dq", "dk", "dv"), where=f"bwd-only head {h}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_deterministic_outputs(dtype):
    """O, LSE, dQ, dK, dV are bitwise reproducible (no atomics on the default
    path)."""
    log(f"[determinism] {dtype}")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(2, 4, 512, 128), seed=5, dtype=dtype)
    a = run_gpu(x, dtype, True, 1 / math.sqrt(128))
    b = run_gpu(x, dtype, True, 1 / math.sqrt(128))
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(a[n], b[n]), n


def test_non_default_stream():
    import torch
    log("[stream] side stream")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(1, 2, 384, 64), seed=13)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        res = run_gpu(x, "bf16", True, 0.125, stream=s)
    want = oracle_heads(x, True, 0.125, heads=None)
    for (b, h), wv in want.items():
        compare({n: res[n][b, h] for n in wv}, wv, "bf16", where=f"stream head {h}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [129, 300, 1024])
def test_atomic_dq_mode(monkeypatch, d, causal, n):
    """The alternative dQ path (fp32 atomics from the key/value-outer kernel,
    selected with FA_DQ_MODE=atomic) meets the same bar."""
    monkeypatch.setenv("FA_DQ_MODE", "atomic")
    log(f"[atomic-dq] d={d} causal={causal} N={n}")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(1, 3, n, d), seed=4242 + n, dtype="bf16")
    _full_compare(x, "bf16", causal, 1.0 / math.sqrt(d), f"atomic d{d} c{int(causal)} N{n}")


# [B, N, H, d] inputs (fa.FA_LAYOUT_BNHD): the kernels run the same arithmetic
# in the same order and only address rows H*d elements apart, so the results
# must be bit-identical to the [B, H, N, d] run on the transposed data, and
# meet the oracle bar on their own.
BNHD = [(dtype, d, causal, n)
        for dtype in ("bf16", "fp32")
        for d in (64, 96, 128)
        for causal in (False, True)
        for n in (17, 300)]
BNHD += [("fp32", 256, causal, n) for causal in (False, True) for n in (17, 300)]   # bf16: its own test


@pytest.mark.parametrize("dtype,d,causal,n", BNHD)
def test_bnhd_layout(dtype, d, causal, n):
    log(f"[bnhd] dtype={dtype} d={d} causal={causal} N={n}")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(2, 3, n, d), seed=5150 + n + d, dtype=dtype)
    scale = 1.0 / math.sqrt(d)
    _, got = _full_compare(x, dtype, causal, scale, f"bnhd {dtype} d{d} c{int(causal)} N{n}",
                           layout=fa.FA_LAYOUT_BNHD)
    ref_res = run_gpu(x, dtype, causal, scale)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(got[name], ref_res[name]), f"bnhd {name} differs from the BHND run"


@pytest.mark.parametrize("causal", [False, True])
def test_bnhd_atomic_dq_mode(monkeypatch, causal):
    monkeypatch.setenv("FA_DQ_MODE", "atomic")
    log(f"[bnhd-atomic] causal={causal}")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(2, 3, 300, 128), seed=616, dtype="bf16")
    _full_compare(x, "bf16", causal, 1.0 / math.sqrt(128), f"bnhd atomic c{int(causal)}",
                  layout=fa.FA_LAYOUT_BNHD)


def test_bnhd_full_size_matches_bhnd():
    """At the causal (1, 32, 8192, 128) bf16 size the [B, N, H, d] run is
    bit-identical to the [B, H, N, d] run, which the sampled-head tests tie to
    the oracle."""
    import torch
    w = gen.workload("c4")
    log(f"[bnhd-full] {w.name} {w.shape}")
    x = gen.make_inputs(w)
    a = run_gpu(x, w.dtype, w.causal, w.scale)
    a.pop("_dev")
    b = run_gpu(x, w.dtype, w.causal, w.scale, layout=fa.FA_LAYOUT_BNHD)
    b.pop("_dev")
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(a[name], b[name]), f"bnhd {name} differs from the BHND run"
    torch.cuda.empty_cache()


def _rising_inputs(dtype):
    """Scores that grow with the key index (k_j has a component along q that
    rises with j), so that every key tile raises each row's maximum and the
    forward's lagging reference has to move on nearly every tile; plus one
    very sharp row (spread 8)."""
    n, d = 700, 64
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(1, 2, n, d), seed=808, dtype=dtype)
    ramp = np.linspace(0.0, 12.0, n, dtype=np.float32)[None, None, :, None]
    k = x["k"] * np.float32(0.1) + ramp * np.float32(1.0 / math.sqrt(d))
    q = np.abs(x["q"]) + np.float32(1.0)
    q[:, :, 5] *= np.float32(8.0)
    if dtype == "bf16":
        k, q = gen.round_bf16(k), gen.round_bf16(q)
    return dict(x, k=k, q=q), 1.0 / math.sqrt(d)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_scores_rising_along_the_keys(dtype, causal):
    """O, LSE, dK and dV on rows whose scores rise along the keys (fp32: dQ
    too).  The backward does not use the forward's lagging reference (it
    recomputes from the final LSE).  bf16 dQ is the separate, expected
    failure below."""
    log(f"[rising] dtype={dtype} causal={causal}")
    x, scale = _rising_inputs(dtype)
    names = ("o", "lse", "dq", "dk", "dv") if dtype == "fp32" else ("o", "lse", "dk", "dv")
    res = run_gpu(x, dtype, causal, scale)
    want = oracle_heads(x, causal, scale, heads=None)
    for (b, h), wv in want.items():
        compare({n: res[n][b, h] for n in names}, wv, dtype, names=names,
                where=f"rising {dtype} c{int(causal)} head ({b},{h})")


RISING_DQ_XFAIL = ("bf16 dQ misses the 2e-2 max|dQ| bar on these non-causal rows: D = rowsum(dO o O) is formed "
                   "from the stored bf16 O, and with rows this peaked dP - D cancels to about 1% of its terms, so "
                   "max|dQ| is that remainder and O's 2^-9 rounding in D dominates the error")


@pytest.mark.parametrize("causal", [pytest.param(False, marks=pytest.mark.xfail(strict=True, reason=RISING_DQ_XFAIL)),
                                    True])
def test_scores_rising_along_the_keys_bf16_dq(causal):
    """bf16 dQ on the rising rows (the default dQ method, the dS hand-off).
    Causal rows pass the bar; the non-causal ones are a known, explicit
    failure (reason above)."""
    log(f"[rising dq] bf16 causal={causal}")
    x, scale = _rising_inputs("bf16")
    res = run_gpu(x, "bf16", causal, scale)
    want = oracle_heads(x, causal, scale, heads=None)
    for (b, h), wv in want.items():
        err = float(np.abs(res["dq"][b, h] - wv["dq"]).max())
        log(f"  head ({b},{h}) dq error / bar {err / (2e-2 * max(1e-2, float(np.abs(wv['dq']).max()))):.3f}")
        compare({"dq": res["dq"][b, h]}, wv, "bf16", names=("dq",), where=f"rising bf16 dq c{int(causal)} ({b},{h})")


def test_head_dim_96_larger_size_sampled_heads():
    """d = 96 (192-byte rows in 256-byte LDS slots) at a causal 2 x 12 x 4096
    size in the launch configuration of the other sizes, on sampled heads."""
    import torch
    log("[d96] 2x12x4096x96 causal bf16")
    w = gen.workload("c3")
    x = gen.make_inputs(w, shape=(2, 12, 4096, 96), seed=96)
    scale = 1.0 / math.sqrt(96)
    res = run_gpu(x, "bf16", True, scale)
    heads = [(0, 0), (1, 11)]
    want = oracle_heads(x, True, scale, heads=heads)
    for (b, h), wv in want.items():
        compare({n: res[n][b, h] for n in wv}, wv, "bf16", where=f"d96 head ({b},{h})")
    torch.cuda.empty_cache()


def test_head_dim_96_atomic_mode_falls_back(monkeypatch):
    """FA_DQ_MODE=atomic has no d = 96 variant; d = 96 keeps the query-outer
    dQ kernel and the same results."""
    log("[d96] atomic mode request")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(1, 2, 300, 96), seed=961)
    a = run_gpu(x, "bf16", True, 0.1)
    monkeypatch.setenv("FA_DQ_MODE", "atomic")
    b = run_gpu(x, "bf16", True, 0.1)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(a[n], b[n]), n


def test_maximum_size_sampled_heads():
    """The largest shape the library takes with the headline geometry: B=63,
    H=32, N=8192, d=128 causal, 2.11e9 elements per tensor (the ABI limit is
    2^31), so every per-head base and row offset runs through the 64-bit
    address arithmetic.  Inputs come from a seeded device generator; three
    whole heads (the first, one in the middle, the last) go to the oracle with
    the exact bf16 values the kernels saw.  Both dQ methods: the hand-off
    buffer is 136 GB here, so its byte offsets run far past 2^32."""
    import torch
    B, H, N, d = 63, 32, 8192, 128
    assert B * H * N * d < 2 ** 31 and 64 * H * N * d >= 2 ** 31
    log(f"[max size] B={B} H={H} N={N} d={d} causal, {B * H * N * d:.3e} elements per tensor")
    scale = 1.0 / math.sqrt(d)
    g = torch.Generator(device="cuda").manual_seed(63)
    q, k, v, do = (torch.randn((B, H, N, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
                   for _ in range(4))
    o, lse = fa.forward(q, k, v, True, scale)
    heads = ((0, 0), (31, 17), (B - 1, H - 1))
    want = {}
    for b, h in heads:
        x = {n: t[b, h].float().cpu().numpy().astype(np.float64)[None, None] for n, t in
             (("q", q), ("k", k), ("v", v), ("do", do))}
        want[(b, h)] = oracle_heads(x, True, scale, heads=[(0, 0)])[(0, 0)]
    for method in (fa.FA_DQ_HANDOFF, fa.FA_DQ_RECOMPUTE):
        log(f"  backward, dQ by {METHOD_NAME[method]}")
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, True, scale, method=method)
        torch.cuda.synchronize()
        for b, h in heads:
            got = {"o": to_np(o[b, h]), "lse": to_np(lse[b, h]), "dq": to_np(dq[b, h]), "dk": to_np(dk[b, h]),
                   "dv": to_np(dv[b, h])}
            errs = compare(got, want[(b, h)], "bf16", where=f"max size {METHOD_NAME[method]} head ({b},{h})")
            log(f"  head ({b},{h}) max errors {errs}")
        del dq, dk, dv
        torch.cuda.empty_cache()
    del q, k, v, do, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [False, True])
def test_fp32_head_dim_256_larger_size(causal):
    """The fp32 path at d = 256 (four lanes per row in the forward, eight in
    the backward) on whole heads of 1 x 2 x 1024 x 256: 64 row blocks of the
    backward kernels and 32 streamed tiles per row."""
    log(f"[fp32 d256] 1x2x1024 causal={causal}")
    x = gen.make_inputs(gen.workload("c1"), shape=(1, 2, 1024, 256), seed=25600 + int(causal))
    _full_compare(x, "fp32", causal, 1.0 / 16.0, f"fp32 d256 1024 c{int(causal)}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_more_heads_than_a_grid_dimension_holds(dtype):
    """70000 heads (B=2, H=35000) of N=3, d=64: more workgroups along the
    head index than a grid's second dimension can hold (65535), so every
    kernel must take the head from a one-dimensional grid; the first, a
    middle and the last head against the oracle, causal and not."""
    B, H, N, d = 2, 35000, 3, 64
    log(f"[many heads] {dtype} B={B} H={H} N={N} d={d}")
    x = gen.make_inputs(gen.workload("c1" if dtype == "fp32" else "c2"), shape=(B, H, N, d), seed=70000)
    for causal in (False, True):
        res = run_gpu(x, dtype, causal, 0.125)
        heads = [(0, 0), (1, 17499), (B - 1, H - 1)]
        want = oracle_heads(x, causal, 0.125, heads)
        for b, h in heads:
            compare({n: res[n][b, h] for n in ("o", "lse", "dq", "dk", "dv")}, want[(b, h)], dtype,
                    where=f"many heads {dtype} c{int(causal)} head ({b},{h})")


def test_maximum_size_d256_sampled_heads():
    """The largest d = 256 shape of the same kind: B=63, H=16, N=8192 causal,
    2.11e9 elements per tensor (one batch more reaches the 2^31 limit), through
    the d = 256 forward, preprocess, dK/dV and dQ kernels; three whole heads
    against the oracle as above, for both dQ methods."""
    import torch
    B, H, N, d = 63, 16, 8192, 256
    assert B * H * N * d < 2 ** 31 and (B + 1) * H * N * d >= 2 ** 31
    log(f"[max size d256] B={B} H={H} N={N} d={d} causal, {B * H * N * d:.3e} elements per tensor")
    scale = 1.0 / math.sqrt(d)
    g = torch.Generator(device="cuda").manual_seed(256)
    q, k, v, do = (torch.randn((B, H, N, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
                   for _ in range(4))
    o, lse = fa.forward(q, k, v, True, scale)
    heads = ((0, 0), (31, 9), (B - 1, H - 1))
    want = {}
    for b, h in heads:
        x = {n: t[b, h].float().cpu().numpy().astype(np.float64)[None, None] for n, t in
             (("q", q), ("k", k), ("v", v), ("do", do))}
        want[(b, h)] = oracle_heads(x, True, scale, heads=[(0, 0)])[(0, 0)]
    for method in (fa.FA_DQ_HANDOFF, fa.FA_DQ_RECOMPUTE):
        log(f"  backward, dQ by {METHOD_NAME[method]}")
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, True, scale, method=method)
        torch.cuda.synchronize()
        for b, h in heads:
            got = {"o": to_np(o[b, h]), "lse": to_np(lse[b, h]), "dq": to_np(dq[b, h]), "dk": to_np(dk[b, h]),
                   "dv": to_np(dv[b, h])}
            errs = compare(got, want[(b, h)], "bf16", where=f"max size d256 {METHOD_NAME[method]} head ({b},{h})")
            log(f"  head ({b},{h}) max errors {errs}")
        del dq, dk, dv
        torch.cuda.empty_cache()
    del q, k, v, do, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [False, True])
def test_head_dim_256_bnhd_layout(causal):
    log(f"[d256 bnhd] causal={causal}")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(2, 3, 333, 256), seed=256)
    _full_compare(x, "bf16", causal, 1.0 / 16.0, f"d256 bnhd c{int(causal)}", layout=fa.FA_LAYOUT_BNHD)


def test_head_dim_256_larger_size_sampled_heads():
    """d = 256 with several query blocks and key tiles per head and many
    workgroups: causal 1 x 16 x 4096 x 256, two whole heads."""
    import torch
    w = gen.workload("c3")
    log("[d256 large] 1x16x4096x256 causal")
    x = gen.make_inputs(w, shape=(1, 16, 4096, 256), seed=2561)
    res = run_gpu(x, "bf16", True, 1.0 / 16.0)
    want = oracle_heads(x, True, 1.0 / 16.0, heads=[(0, 0), (0, 15)])
    for (b, h), wv in want.items():
        errs = compare({n: res[n][b, h] for n in wv}, wv, "bf16", where=f"d256 large head ({b},{h})")
        log(f"  head ({b},{h}) max errors {errs}")
    del res
    torch.cuda.empty_cache()



@pytest.mark.parametrize("d,n", [(128, 8155), (256, 4099)])
def test_large_ragged_sampled_heads(d, n):
    """A ragged last tile behind many full ones (N not a multiple of any tile
    or block size), causal, on two whole heads."""
    import torch
    log(f"[large ragged] d={d} N={n}")
    w = gen.workload("c4")
    x = gen.make_inputs(w, shape=(1, 3, n, d), seed=n)
    scale = 1.0 / math.sqrt(d)
    res = run_gpu(x, "bf16", True, scale)
    want = oracle_heads(x, True, scale, heads=[(0, 0), (0, 2)])
    for (b, h), wv in want.items():
        errs = compare({k: res[k][b, h] for k in wv}, wv, "bf16", where=f"large ragged d{d} head ({b},{h})")
        log(f"  head ({b},{h}) max errors {errs}")
    del res
    torch.cuda.empty_cache()


def test_conveniences_reject_mismatched_buffers():
    """Outputs, LSE, gradients and workspaces handed to the torch
    conveniences are checked before any launch: each mismatched buffer raises
    ValueError, and the outputs given alongside stay untouched."""
    import torch
    B, H, N, d = 1, 2, 64, 128
    log(f"[buffers] B={B} H={H} N={N} d={d}")
    q, k, v, do = (torch.randn((B, H, N, d), device="cuda").to(torch.bfloat16) for _ in range(4))
    o, lse = fa.forward(q, k, v, True, 0.125)
    short_o = torch.full((B, H, N - 1, d), 7.0, dtype=torch.bfloat16, device="cuda")
    f32_o = torch.full((B, H, N, d), 7.0, dtype=torch.float32, device="cuda")
    short_l = torch.full((B, H, N - 1), 7.0, dtype=torch.float32, device="cuda")
    strided_l = torch.full((B, N, H), 7.0, dtype=torch.float32, device="cuda").transpose(1, 2)
    for kw in (dict(out=short_o), dict(out=f32_o), dict(lse=short_l), dict(lse=strided_l)):
        with pytest.raises(ValueError):
            fa.forward(q, k, v, True, 0.125, **kw)
        with pytest.raises(ValueError):
            fa.forward_dropout(q, k, v, True, 0.125, 0.1, 3, **kw)
    good = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    for kw in (dict(grads=(good[0], good[1], short_o)), dict(ws=torch.empty(1 << 20, device="cuda")),
               dict(ws=torch.empty(1 << 20, dtype=torch.uint8, device="cuda")[::2])):
        with pytest.raises(ValueError):
            fa.backward(q, k, v, o, do, lse, True, 0.125, **kw)
        with pytest.raises(ValueError):
            fa.backward_dropout(q, k, v, o, do, lse, True, 0.125, 0.1, 3, **kw)
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, do, short_l, True, 0.125)
    # FP8 forward: bf16 output of the inputs' shape
    q8, k8, v8 = (torch.zeros((B, H, N, d), dtype=torch.uint8, device="cuda") for _ in range(3))
    for kw in (dict(out=f32_o), dict(out=short_o), dict(lse=short_l)):
        with pytest.raises(ValueError):
            fa.forward_fp8(q8, k8, v8, 1.0, 1.0, 1.0, True, 0.125, **kw)
    # split-key-range forward: 4 queries against the 64 keys; uint8 workspace
    qd, q8d = q[:, :, :4].contiguous(), q8[:, :, :4].contiguous()
    o4 = torch.full((B, H, 4, d), 7.0, dtype=torch.bfloat16, device="cuda")
    l4 = torch.full((B, H, 4), 7.0, dtype=torch.float32, device="cuda")
    bad_split = (dict(out=short_o, lse=l4), dict(out=o4, lse=short_l),
                 dict(out=o4, lse=l4, ws=torch.empty(1 << 20, device="cuda")),
                 dict(out=o4, lse=l4, ws=torch.empty(1 << 20, dtype=torch.uint8, device="cuda")[1::2]))
    for kw in bad_split:
        with pytest.raises(ValueError):
            fa.forward_splitkv(qd, k, v, True, 0.125, **kw)
        with pytest.raises(ValueError):
            fa.forward_splitkv_fp8(q8d, k8, v8, 1.0, 1.0, 1.0, True, 0.125, **kw)
    # a key/value cache with fewer heads (grouped-query shape) or another head
    # dim than q: the kernels would read K and V with q's head offsets
    for kc in (k[:, :1].contiguous(), k[..., :64].contiguous()):
        with pytest.raises(ValueError):
            fa.forward_splitkv(qd, kc, kc, True, 0.125, out=o4, lse=l4)
        k8c = torch.zeros(kc.shape, dtype=torch.uint8, device="cuda")
        with pytest.raises(ValueError):
            fa.forward_splitkv_fp8(q8d, k8c, k8c, 1.0, 1.0, 1.0, True, 0.125, out=o4, lse=l4)
    torch.cuda.synchronize()
    for t in (short_o, f32_o, short_l, strided_l, o4, l4):
        assert bool((t == 7.0).all())
