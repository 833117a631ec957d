"""GPU parity of fa_fwd_dropout / fa_bwd_dropout (through the C ABI) against
the fp64 dropout oracle (oracle/dropout.py).

Two kinds of checks:
- the keep mask itself, bit for bit, in each of the three kernels that
  regenerate it: with identity operands (N <= d) an output is the masked
  probability matrix or dS, whose kept and dropped entries differ by
  P * keep_scale, so every entry's mask bit can be read off;
- values: O, LSE, dQ, dK, dV against the oracle with the bf16 tolerances of
  the plain path (for dQ and dK plus the derived effect of forming D from the
  stored bf16 O, see ``compare_dropout``), on small and ragged shapes, both
  layouts, several heads, seeds and offsets, and on sampled heads of a large
  causal shape (plain bar).
"""
import math

import numpy as np
import pytest

import exact_tiled_attention_online_amd as fa
from exact_tiled_attention_online_amd import inputs as gen
from gpu_util import compare, log, to_dev, to_np
from oracle import dropout as dr
from oracle import ref

pytestmark = pytest.mark.gpu


def run_dropout(x, causal, scale, t, seed, offset, layout=0, bwd=True, method=fa.FA_DQ_HANDOFF):
    import torch
    q, k, v, do = (to_dev(x[n], "bf16", layout) for n in ("q", "k", "v", "do"))
    p = t / 256.0
    assert fa.drop_threshold(p) == t
    o, lse = fa.forward_dropout(q, k, v, causal, scale, p, seed, offset, layout=layout)
    res = {"o": o, "lse": lse}
    if bwd:
        dq, dk, dv = fa.backward_dropout(q, k, v, o, do, lse, causal, scale, p, seed, offset, layout=layout,
                                         method=method)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: to_np(tns, layout if n != "lse" else 0) for n, tns in res.items()}


def _bf16(a):
    import torch
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def _identity_inputs(B, H, N, d, seed, which, do_eye=False):
    """Random rows for the operands in `which`, identity rows (e_j) for the
    other ones among q, k, v; dO all ones (or identity rows)."""
    r = np.random.default_rng(seed)
    eye = np.zeros((N, d))
    eye[np.arange(N), np.arange(N)] = 1.0
    x = {}
    for n in ("q", "k", "v", "do"):
        if n in which:
            x[n] = _bf16(r.standard_normal((B, H, N, d)))
        elif n == "do" and not do_eye:
            x[n] = np.ones((B, H, N, d))
        else:
            x[n] = np.broadcast_to(eye, (B, H, N, d)).copy()
    return x


MASK_CASES = [(d, n, causal) for d in (64, 96, 128, 256) for n in (d, 37) for causal in (False, True)]


@pytest.mark.parametrize("d,n,causal", MASK_CASES)
@pytest.mark.parametrize("layout", [0, 1])
def test_forward_mask_bit_exact(d, n, causal, layout):
    """V = I: O[:, :N] = keep_scale * (P o Z), so Z = (O != 0) where P > 0."""
    log(f"[drop-mask fwd] d={d} N={n} causal={causal} layout={layout}")
    B, H, t, seed, off = 2, 3, 77, 0x9E3779B97F4A7C15, 11
    x = _identity_inputs(B, H, n, d, 5 + d + n, which=("q", "k"))
    scale = 1.0 / math.sqrt(d)
    got = run_dropout(x, causal, scale, t, seed, off, layout=layout, bwd=False)
    for b in range(B):
        for h in range(H):
            _, _, s, p = ref.head_forward(x["q"][b, h], x["k"][b, h], x["v"][b, h], scale, causal)
            z = dr.keep_mask(b * H + h, seed, off, t, n, n)
            live = p > 0
            zg = got["o"][b, h][:, :n] != 0
            assert (zg[live] == z[live]).all(), f"head ({b},{h}): {int((zg[live] != z[live]).sum())} mask bits differ"
            assert not zg[~live].any()
            np.testing.assert_allclose(got["o"][b, h][:, :n], dr.keep_scale(t) * np.where(z, p, 0.0),
                                       rtol=2 ** -7, atol=1e-6)
            assert (got["o"][b, h][:, n:] == 0).all()


def _ds_and_bits(x, b, h, H, n, scale, causal, t, seed, off):
    """Oracle P, D and dS for the identity inputs, and the oracle mask."""
    z = dr.keep_mask(b * H + h, seed, off, t, n, n)
    _, _, _, it = dr.head_backward_dropout(x["q"][b, h], x["k"][b, h], x["v"][b, h], x["do"][b, h], scale,
                                           causal, z, t, want_intermediates=True)
    return it["p"], it["D"], z


@pytest.mark.parametrize("d,n,causal", MASK_CASES)
def test_dkdv_kernel_mask_bit_exact(d, n, causal):
    """Q = V = I.  With dO = I, dV[:N] = s (P o Z)^T.  With dO = 1,
    dK[:N] = scale dS^T, where a kept dS entry is P (s - D) and a dropped one
    -P D: their difference P s exceeds the rounding by far, so each bit is
    read from how far dS sits above -P D."""
    log(f"[drop-mask dkdv] d={d} N={n} causal={causal}")
    B, H, t, seed, off = 1, 2, 128, 12345, 0
    scale = 1.0 / math.sqrt(d)
    sk = dr.keep_scale(t)
    xv = _identity_inputs(B, H, n, d, 17 + d + n, which=("k",), do_eye=True)
    gv = run_dropout(xv, causal, scale, t, seed, off)
    x = _identity_inputs(B, H, n, d, 17 + d + n, which=("k",))
    got = run_dropout(x, causal, scale, t, seed, off)
    for h in range(H):
        p, D, z = _ds_and_bits(x, 0, h, H, n, scale, causal, t, seed, off)
        live = p > 1e-3
        zv = gv["dv"][0, h][:n, :n].T != 0
        assert (zv[live] == z[live]).all(), f"dV: {int((zv[live] != z[live]).sum())} mask bits differ"
        np.testing.assert_allclose(gv["dv"][0, h][:n, :n].T, sk * np.where(z, p, 0.0), rtol=2 ** -7, atol=1e-6)
        ds = got["dk"][0, h][:n, :n].T / scale
        frac = (ds + p * D[:, None]) / (p * sk + 1e-300)
        zk = frac > 0.5
        assert (zk[live] == z[live]).all(), f"dK: {int((zk[live] != z[live]).sum())} mask bits differ"
        assert np.abs(frac[live] - z[live]).max() < 0.25


@pytest.mark.parametrize("d,n,causal", MASK_CASES)
@pytest.mark.parametrize("method", [fa.FA_DQ_RECOMPUTE, fa.FA_DQ_HANDOFF])
def test_dq_kernel_mask_bit_exact(d, n, causal, method):
    """K = V = I, dO = 1: dQ[:, :N] = scale dS; bits as in the dK/dV test.
    The recompute kernel regenerates the mask; with the hand-off dQ comes
    from the dS the key/value-outer kernel stored."""
    log(f"[drop-mask dq] d={d} N={n} causal={causal} method={method}")
    B, H, t, seed, off = 1, 2, 128, 987654321, 42
    x = _identity_inputs(B, H, n, d, 29 + d + n, which=("q",))
    scale = 1.0 / math.sqrt(d)
    sk = dr.keep_scale(t)
    got = run_dropout(x, causal, scale, t, seed, off, method=method)
    for h in range(H):
        p, D, z = _ds_and_bits(x, 0, h, H, n, scale, causal, t, seed, off)
        live = p > 1e-3
        ds = got["dq"][0, h][:, :n] / scale
        frac = (ds + p * D[:, None]) / (p * sk + 1e-300)
        zq = frac > 0.5
        assert (zq[live] == z[live]).all(), f"dQ: {int((zq[live] != z[live]).sum())} mask bits differ"
        assert np.abs(frac[live] - z[live]).max() < 0.25


def compare_dropout(got, want, x, b, h, scale, causal, where):
    """O, LSE, dV with the plain path's bf16 bar.  dQ and dK add the effect
    of D being formed from the stored bf16 O: each D_i may be off by
    dD_i = 2^-8 sum_c |dO_ic O_ic| (rounding of O to bf16 and O's own
    error), which enters dS as P_ij dD_i, so dQ_ic by at most
    scale dD_i max|K| and dK_jc by at most scale (sum_i P_ij dD_i) max|Q|.
    This matters where the exact gradient cancels to nearly zero (one key:
    dS = 0): with dropout, O = keep_scale * V is not a bf16 value, so the
    cancellation leaves the rounding of D behind."""
    errs = compare({n: got[n] for n in ("o", "lse", "dv")}, want, "bf16", names=("o", "lse", "dv"), where=where)
    q, k, v, do = (x[n][b, h] for n in ("q", "k", "v", "do"))
    _, _, _, p = ref.head_forward(q, k, v, scale, causal)
    dD = 2.0 ** -8 * np.abs(do * want["o"]).sum(axis=1)
    extra = {"dq": abs(scale) * dD.max() * np.abs(k).max(),
             "dk": abs(scale) * (p * dD[:, None]).sum(axis=0).max() * np.abs(q).max()}
    for n in ("dq", "dk"):
        g, r = np.asarray(got[n]), np.asarray(want[n])
        assert np.isfinite(g).all(), f"{where} {n}: non-finite values"
        err = float(np.abs(g - r).max())
        tol = 2e-2 * max(1e-2, float(np.abs(r).max())) + extra[n]
        assert err <= tol, f"{where} {n}: max abs err {err:.3e} > tol {tol:.3e}"
        errs[n] = err
    return errs


def _compare_all(x, causal, scale, t, seed, off, layout=0, where="", method=fa.FA_DQ_HANDOFF):
    got = run_dropout(x, causal, scale, t, seed, off, layout=layout, method=method)
    want = dr.forward_backward_dropout(x["q"], x["k"], x["v"], x["do"], scale, causal, seed, off, t)
    errs = {}
    for (b, h), w in want.items():
        e = compare_dropout({n: got[n][b, h] for n in w}, w, x, b, h, scale, causal, f"{where} head ({b},{h})")
        for n, v in e.items():
            errs[n] = max(errs.get(n, 0.0), v)
    return errs


VALUE_CASES = [(d, n, causal, t) for d in (64, 96, 128) for n in (1, 64, 129, 300)
               for causal in (False, True) for t in (26, 128)]
VALUE_CASES += [(256, n, causal, 77) for n in (1, 129, 300) for causal in (False, True)]


@pytest.mark.parametrize("d,n,causal,t", VALUE_CASES)
@pytest.mark.parametrize("method", [fa.FA_DQ_HANDOFF, fa.FA_DQ_RECOMPUTE])
def test_values_small_and_ragged(d, n, causal, t, method):
    log(f"[drop-values] d={d} N={n} causal={causal} t={t} method={method}")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(2, 2, n, d), seed=3000 + n + d + t)
    _compare_all(x, causal, 1.0 / math.sqrt(d), t, seed=1000 + n, off=t, where=f"d{d} N{n} c{int(causal)} t{t}",
                 method=method)


@pytest.mark.parametrize("causal", [False, True])
def test_values_bnhd_layout(causal):
    log(f"[drop-values bnhd] causal={causal}")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(2, 3, 200, 128), seed=41)
    _compare_all(x, causal, 0.3, 51, seed=7, off=9, layout=fa.FA_LAYOUT_BNHD, where=f"bnhd c{int(causal)}")


def test_threshold_zero_is_the_plain_path_bit_for_bit():
    """t = 0 keeps every probability with scale 1: the dropout kernels then do
    the plain kernels' arithmetic and must give the same bits."""
    import torch
    log("[drop t=0 == plain]")
    w = gen.workload("c3")
    x = gen.make_inputs(w, shape=(1, 4, 1000, 128), seed=8)
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    o0, l0 = fa.forward(q, k, v, True, w.scale)
    g0 = fa.backward(q, k, v, o0, do, l0, True, w.scale)
    o1, l1 = fa.forward_dropout(q, k, v, True, w.scale, 0.0, seed=5)
    g1 = fa.backward_dropout(q, k, v, o1, do, l1, True, w.scale, 0.0, seed=5)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)


def test_same_seed_same_bits_other_offset_other_mask():
    import torch
    log("[drop determinism]")
    w = gen.workload("c2")
    x = gen.make_inputs(w, shape=(1, 2, 512, 64), seed=12)
    q, k, v = (to_dev(x[n], "bf16") for n in ("q", "k", "v"))
    a = fa.forward_dropout(q, k, v, False, 0.125, 0.1, seed=99, offset=1)[0]
    b = fa.forward_dropout(q, k, v, False, 0.125, 0.1, seed=99, offset=1)[0]
    c = fa.forward_dropout(q, k, v, False, 0.125, 0.1, seed=99, offset=2)[0]
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert not torch.equal(a, c)


def test_sampled_heads_large_causal():
    """The headline shape's launch configuration (B=1, H=32, N=8192, d=128,
    causal) with 10% dropout; two whole heads against the oracle."""
    import torch
    w = gen.workload("c4")
    log(f"[drop-large] {w.name} t=26")
    x = gen.make_inputs(w)
    q, k, v, do = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.forward_dropout(q, k, v, True, w.scale, 26 / 256, seed=2024, offset=7)
    dq, dk, dv = fa.backward_dropout(q, k, v, o, do, lse, True, w.scale, 26 / 256, seed=2024, offset=7)
    torch.cuda.synchronize()
    got = {"o": to_np(o), "lse": to_np(lse), "dq": to_np(dq), "dk": to_np(dk), "dv": to_np(dv)}
    for b, h in ((0, 0), (0, 31)):
        want = dr.forward_backward_dropout(x["q"], x["k"], x["v"], x["do"], w.scale, True, 2024, 7, 26,
                                           heads=[(b, h)])[(b, h)]
        errs = compare({n: got[n][b, h] for n in want}, want, "bf16", where=f"large head ({b},{h})")
        assert errs["dq"] <= 2e-2 * np.abs(want["dq"]).max()
        log(f"  head ({b},{h}) max errors {errs}")


def test_maximum_size_sampled_heads():
    """Dropout at the largest shape of the headline geometry: B=63, H=32,
    N=8192, d=128 causal, 2.11e9 elements per tensor, p = 26/256.  The mask
    counter carries the flattened head index (up to 2015) and the tensors'
    64-bit offsets run through every dropout kernel; three whole heads (the
    first, a middle and the last) against the dropout oracle with the exact
    bf16 values the kernels saw."""
    import torch
    B, H, N, d = 63, 32, 8192, 128
    scale, seed, off, t = 1.0 / math.sqrt(d), 0xABCDEF0123456789, 11, 26
    log(f"[drop max size] B={B} H={H} N={N} d={d} causal t={t}")
    g = torch.Generator(device="cuda").manual_seed(6326)
    q, k, v, do = (torch.randn((B, H, N, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
                   for _ in range(4))
    o, lse = fa.forward_dropout(q, k, v, True, scale, t / 256, seed=seed, offset=off)
    dq, dk, dv = fa.backward_dropout(q, k, v, o, do, lse, True, scale, t / 256, seed=seed, offset=off)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (40, 13), (B - 1, H - 1)):
        hx = {n: tt[b, h].float().cpu().numpy().astype(np.float64) for n, tt in
              (("q", q), ("k", k), ("v", v), ("do", do))}
        want = dr.head_panel_dropout(hx["q"], hx["k"], hx["v"], hx["do"], scale, True, b * H + h, seed, off, t)
        got = {"o": to_np(o[b, h]), "lse": to_np(lse[b, h]), "dq": to_np(dq[b, h]), "dk": to_np(dk[b, h]),
               "dv": to_np(dv[b, h])}
        errs = compare(got, want, "bf16", where=f"drop max size head ({b},{h})")
        log(f"  head ({b},{h}) max errors {errs}")
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
