"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: closed
forms, invariants, finite differences, an independently written tiled model
of the method and a library autograd.  ``test_pins_catch_planted_mistakes``
plants plausible mistakes in copies of the oracle's backward and checks that
the pins reject every one of them.
"""
import math

import numpy as np
import pytest

from oracle import ref
from tiled_model import tiled_backward, tiled_forward

RNG = np.random.default_rng(20261202)


def rand_head(n, d, sig=1.0, seed=None):
    rng = np.random.default_rng(seed) if seed is not None else RNG
    return [rng.standard_normal((n, d)) * sig for _ in range(4)]


CASES = [(n, d, causal, scale)
         for n, d in ((1, 4), (5, 3), (16, 8), (33, 16))
         for causal in (False, True)
         for scale in (None, 0.3)]


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else scale


# P-ROW: every softmax row sums to one (page "flash-attention-backpropagation",
# section 显存困境, the softmax definition).
@pytest.mark.parametrize("n,d,causal,scale", CASES)
def test_rows_sum_to_one(n, d, causal, scale):
    q, k, v, _ = rand_head(n, d)
    _, _, _, p = ref.head_forward(q, k, v, _scale(scale, d), causal)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert (p >= 0).all()
    if causal:
        assert (np.triu(p, 1) == 0).all()


# P-DS0 and P-DID: sum_j dS_ij = 0 and rowsum(dO o O) = rowsum(dP o P)
# (section Softmax梯度: D_i stands for the term the normalisation adds).
@pytest.mark.parametrize("n,d,causal,scale", CASES)
def test_ds_rows_sum_to_zero(n, d, causal, scale):
    q, k, v, do = rand_head(n, d)
    _, _, _, it = ref.head_backward(q, k, v, do, _scale(scale, d), causal,
                                    want_intermediates=True)
    ds = it["ds"]
    tol = 1e-13 * max(1.0, np.abs(ds).max() * n)
    np.testing.assert_allclose(ds.sum(axis=1), 0.0, atol=tol)
    np.testing.assert_allclose(it["D"], (it["dp"] * it["p"]).sum(axis=1), rtol=1e-12, atol=1e-13)


# P-LSE: exp(S - LSE) reproduces P, and max_j S <= LSE <= max_j S + ln(#keys)
# (section 数值稳定: recomputing P from the stored statistics).
@pytest.mark.parametrize("n,d,causal,scale", CASES)
def test_lse_reproduces_p(n, d, causal, scale):
    q, k, v, _ = rand_head(n, d, sig=2.0)
    sc = _scale(scale, d)
    _, lse, s, p = ref.head_forward(q, k, v, sc, causal)
    np.testing.assert_allclose(np.exp(s - lse[:, None]), p, rtol=1e-12, atol=1e-300)
    smax = s.max(axis=1)
    kept = np.arange(1, n + 1) if causal else np.full(n, n)
    assert (lse >= smax - 1e-12).all()
    assert (lse <= smax + np.log(kept) + 1e-12).all()


# P-K0: K = 0 gives uniform attention over the kept keys.
@pytest.mark.parametrize("causal", [False, True])
def test_zero_keys_closed_form(causal):
    n, d = 12, 5
    q, _, v, do = rand_head(n, d)
    k = np.zeros((n, d))
    o, lse, _, _ = ref.head_forward(q, k, v, 0.7, causal)
    dq, dk, dv = ref.head_backward(q, k, v, do, 0.7, causal)
    cnt = np.arange(1, n + 1) if causal else np.full(n, n)
    if causal:
        o_ref = np.cumsum(v, axis=0) / cnt[:, None]
        # dV_j = sum_{i >= j} dO_i / (i + 1)
        w = do / cnt[:, None]
        dv_ref = np.cumsum(w[::-1], axis=0)[::-1]
    else:
        o_ref = np.broadcast_to(v.mean(axis=0), (n, d))
        dv_ref = np.broadcast_to(do.sum(axis=0) / n, (n, d))
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, np.log(cnt), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dv, dv_ref, rtol=1e-12, atol=1e-13)
    # dK_j = scale * sum_i dS_ij Q_i is not zero in general, but dQ is:
    # dQ = scale * dS K = 0 for K = 0.
    assert np.abs(dq).max() == 0.0
    # the column sums of dK vanish (sum_j dS_ij = 0)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)


# P-N1: a single key.
def test_single_token_closed_form():
    q, k, v, do = rand_head(1, 6)
    o, lse, _, _ = ref.head_forward(q, k, v, 0.4, False)
    dq, dk, dv = ref.head_backward(q, k, v, do, 0.4, False)
    np.testing.assert_allclose(o, v, rtol=1e-15)
    np.testing.assert_allclose(lse, 0.4 * (q * k).sum(axis=1), rtol=1e-14)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    np.testing.assert_allclose(dv, do, rtol=1e-15)


def test_first_causal_row():
    q, k, v, do = rand_head(9, 4)
    o, lse, _, _ = ref.head_forward(q, k, v, 0.5, True)
    dq, _, _ = ref.head_backward(q, k, v, do, 0.5, True)
    np.testing.assert_allclose(o[0], v[0], rtol=1e-14)
    np.testing.assert_allclose(lse[0], 0.5 * q[0] @ k[0], rtol=1e-14)
    assert np.abs(dq[0]).max() < 1e-15


# P-VC: constant values make the output constant and the score gradient zero.
@pytest.mark.parametrize("causal", [False, True])
def test_constant_values(causal):
    n, d = 10, 4
    q, k, _, do = rand_head(n, d)
    c = RNG.standard_normal(d)
    v = np.broadcast_to(c, (n, d)).copy()
    o, _, _, _ = ref.head_forward(q, k, v, 0.6, causal)
    dq, dk, _ = ref.head_backward(q, k, v, do, 0.6, causal)
    np.testing.assert_allclose(o, v, rtol=1e-13)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


# P-SHIFT: K -> K + 1 u^T shifts each score row by a constant.
@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    n, d, sc = 14, 6, 0.35
    q, k, v, do = rand_head(n, d)
    u = RNG.standard_normal(d)
    o1, l1, _, _ = ref.head_forward(q, k, v, sc, causal)
    o2, l2, _, _ = ref.head_forward(q, k + u, v, sc, causal)
    g1 = ref.head_backward(q, k, v, do, sc, causal)
    g2 = ref.head_backward(q, k + u, v, do, sc, causal)
    np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l2, l1 + sc * q @ u, rtol=1e-11, atol=1e-12)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(b, a, rtol=1e-10, atol=1e-11)


# P-SUM: consequences of the zero row sums of dS and of P being stochastic.
@pytest.mark.parametrize("causal", [False, True])
def test_gradient_sums_and_hull(causal):
    n, d = 40, 8
    q, k, v, do = rand_head(n, d, sig=1.5)
    o, _, _, _ = ref.head_forward(q, k, v, 0.25, causal)
    dq, dk, dv = ref.head_backward(q, k, v, do, 0.25, causal)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=1e-12, atol=1e-12)
    assert (o <= v.max(axis=0) + 1e-12).all() and (o >= v.min(axis=0) - 1e-12).all()


def _loss(q, k, v, do, sc, causal):
    o, _, _, _ = ref.head_forward(q, k, v, sc, causal)
    return float((do * o).sum())


def fd_check(backward, n, d, causal, sc, seed, h=1e-5):
    """Central finite differences of L = sum(dO o O) against `backward`."""
    q, k, v, do = rand_head(n, d, seed=seed)
    grads = backward(q, k, v, do, sc, causal)
    worst = 0.0
    for which, (x, g) in enumerate(zip((q, k, v), grads)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            orig = x[idx]
            x[idx] = orig + h
            lp = _loss(q, k, v, do, sc, causal)
            x[idx] = orig - h
            lm = _loss(q, k, v, do, sc, causal)
            x[idx] = orig
            num[idx] = (lp - lm) / (2 * h)
        worst = max(worst, np.abs(num - g).max() / max(1e-30, np.abs(g).max()))
    return worst


# P-FD: the analytic gradients match central finite differences of the loss.
@pytest.mark.parametrize("n,d", [(1, 3), (7, 5), (16, 8)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [None, 0.3])
def test_finite_differences(n, d, causal, scale):
    err = fd_check(ref.head_backward, n, d, causal, _scale(scale, d), seed=n * 100 + d)
    assert err < 1e-7, err


def p3_formula_inputs(n=8, d=4):
    """The deterministic inputs of the pure-Python demo on page
    "flash-attention-v2-sram-tiling", section Python 演示 (n=8, d=4)."""
    i = np.arange(n)[:, None] + 1.0
    t = np.arange(d)[None, :]
    return i * 0.5 + t, i * 0.3 - t, i * 0.2 + 0.1 * t


# P-BLK: the tiled online-softmax forward and recompute backward equal the
# materialised oracle for any block sizes, including ones not dividing N
# (the demos of pages "flash-attention-backpropagation" and
# "flash-attention-v2-sram-tiling" check exactly this equivalence in fp64).
@pytest.mark.parametrize("br,bc", [(1, 1), (2, 2), (3, 2), (2, 3), (16, 16), (5, 7)])
@pytest.mark.parametrize("causal", [False, True])
def test_blocking_invariance(br, bc, causal):
    cases = []
    rng = np.random.default_rng(0)
    q = rng.standard_normal((6, 8)); k = rng.standard_normal((6, 8))
    v = rng.standard_normal((6, 8)); do = rng.standard_normal((6, 8))
    cases.append((q, k, v, do, 1 / math.sqrt(8)))
    q, k, v = p3_formula_inputs()
    do = np.cos(np.arange(32.0)).reshape(8, 4)
    cases.append((q, k, v, do, 1 / math.sqrt(4)))
    q, k, v, do = rand_head(37, 16, sig=2.0, seed=5)
    cases.append((q, k, v, do, 0.25))
    for q, k, v, do, sc in cases:
        o, lse, _, _ = ref.head_forward(q, k, v, sc, causal)
        dq, dk, dv = ref.head_backward(q, k, v, do, sc, causal)
        to, tl = tiled_forward(q, k, v, sc, causal, br, bc)
        tq, tk, tv = tiled_backward(q, k, v, to, do, tl, sc, causal, br, bc)
        for a, b in ((o, to), (lse, tl), (dq, tq), (dk, tk), (dv, tv)):
            np.testing.assert_allclose(b, a, rtol=0, atol=1e-10 * max(1.0, np.abs(a).max()))


# The panel walk over full rows equals the unpanelled definition.
@pytest.mark.parametrize("causal", [False, True])
def test_panels_match_whole(causal):
    q, k, v, do = rand_head(50, 8)
    whole_o, whole_l, _, _ = ref.head_forward(q, k, v, 0.3, causal)
    gq, gk, gv = ref.head_backward(q, k, v, do, 0.3, causal)
    out = ref.head_panel(q, k, v, do, 0.3, causal, panel_rows=7)
    for a, b in ((whole_o, out["o"]), (whole_l, out["lse"]), (gq, out["dq"]),
                 (gk, out["dk"]), (gv, out["dv"])):
        np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-13)


# P-LIB: fp64 autograd of plain softmax attention in torch (CPU).
@pytest.mark.parametrize("causal", [False, True])
def test_torch_autograd_cross_check(causal):
    torch = pytest.importorskip("torch")
    n, d, sc = 24, 8, 0.31
    q, k, v, do = rand_head(n, d)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = sc * tq @ tk.T
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    lse = torch.logsumexp(s, dim=-1)
    (o * torch.tensor(do)).sum().backward()
    ro, rl, _, _ = ref.head_forward(q, k, v, sc, causal)
    gq, gk, gv = ref.head_backward(q, k, v, do, sc, causal)
    np.testing.assert_allclose(ro, o.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(rl, lse.detach().numpy(), rtol=1e-12, atol=1e-13)
    for a, t in ((gq, tq), (gk, tk), (gv, tv)):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=1e-11, atol=1e-12)


# The 4-D wrappers walk every (b, h) head.
def test_batched_wrappers():
    rng = np.random.default_rng(3)
    q, k, v, do = (rng.standard_normal((2, 3, 9, 4)) for _ in range(4))
    o, lse = ref.forward(q, k, v, 0.5, True)
    dq, dk, dv = ref.backward(q, k, v, do, 0.5, True)
    allh = ref.forward_backward(q, k, v, do, 0.5, True, panel_rows=4)
    for b in range(2):
        for h in range(3):
            ho, hl, _, _ = ref.head_forward(q[b, h], k[b, h], v[b, h], 0.5, True)
            np.testing.assert_allclose(o[b, h], ho, rtol=1e-14)
            np.testing.assert_allclose(lse[b, h], hl, rtol=1e-14)
            e = allh[(b, h)]
            np.testing.assert_allclose(e["dq"], dq[b, h], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(e["dk"], dk[b, h], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(e["dv"], dv[b, h], rtol=1e-12, atol=1e-13)


# ---- planted mistakes: each mutant of the backward must fail a pin ----------

def _mutant(kind):
    def bwd(q, k, v, do, sc, causal):
        s = ref.scores(q, k, sc, causal)
        p, _, _ = ref.softmax_rows(s)
        o = p @ v
        drow = (do * o).sum(axis=1)
        dp = do @ v.T
        if kind == "dropped_D":
            ds = p * dp
        elif kind == "sign_D":
            ds = p * (dp + drow[:, None])
        else:
            ds = p * (dp - drow[:, None])
        dv = (p @ do) if kind == "untransposed_P" else p.T @ do
        dq = (ds @ k) if kind == "missing_scale" else sc * (ds @ k)
        dk = sc * (ds @ q) if kind == "untransposed_dS" else sc * (ds.T @ q)
        if kind == "scale_squared":
            dq = sc * dq
        return dq, dk, dv
    return bwd


@pytest.mark.parametrize("kind", ["dropped_D", "sign_D", "untransposed_P",
                                  "missing_scale", "untransposed_dS", "scale_squared"])
def test_pins_catch_planted_mistakes(kind):
    err = max(fd_check(_mutant(kind), 6, 3, causal, 0.3, seed=11) for causal in (False, True))
    assert err > 1e-3, (kind, err)


def test_closed_form_two_tokens():
    """N=2, d=1 worked by hand: q=(1,2), k=(0,1), v=(3,5), scale 1.

    Row 0 scores (0, 1): P = (1, e)/(1+e), O = (3+5e)/(1+e), LSE = ln(1+e).
    Row 1 scores (0, 2): P = (1, e^2)/(1+e^2), O = (3+5e^2)/(1+e^2),
    LSE = ln(1+e^2).  Causal: row 0 keeps only key 0, so O = 3, LSE = 0.
    """
    e = math.e
    q = np.array([[1.0], [2.0]]); k = np.array([[0.0], [1.0]]); v = np.array([[3.0], [5.0]])
    want = {False: ([(3 + 5 * e) / (1 + e), (3 + 5 * e * e) / (1 + e * e)],
                    [math.log1p(e), math.log1p(e * e)]),
            True: ([3.0, (3 + 5 * e * e) / (1 + e * e)], [0.0, math.log1p(e * e)])}
    for causal, (o_w, l_w) in want.items():
        o, lse, _, _ = ref.head_forward(q, k, v, 1.0, causal)
        np.testing.assert_allclose(o[:, 0], o_w, rtol=1e-15)
        np.testing.assert_allclose(lse, l_w, rtol=1e-15, atol=1e-16)


def test_golden_p3_formula_case():
    """Regression lock on the demo inputs of page "flash-attention-v2-sram-tiling"
    (section Python 演示), values written by tests/golden/make_golden.py."""
    import json, os
    path = os.path.join(os.path.dirname(__file__), "golden", "p3_formula_case.json")
    g = json.load(open(path))
    q, k, v = p3_formula_inputs()
    for key, causal in (("full", False), ("causal", True)):
        o, lse, _, _ = ref.head_forward(q, k, v, g["scale"], causal)
        np.testing.assert_allclose(o, np.array(g[key]["O"]), rtol=1e-14)
        np.testing.assert_allclose(lse, np.array(g[key]["LSE"]), rtol=1e-14)
