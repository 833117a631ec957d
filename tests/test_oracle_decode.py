"""Pins of the oracle's rectangular forward (Nq queries against Nk >= Nq keys,
the decode shape), each against something other than the function itself:

* Nq == Nk reduces to the square oracle, which test_oracle.py pins;
* a causal row equals the non-causal attention of that query over the keys
  its position allows (the mask reading: query i sits at position Nk - Nq + i);
* brute force with Python loops and math.exp on tiny inputs;
* PyTorch's own attention routine on CPU in float64 with an explicit mask;
* the merge rule for two partial softmax results (page
  "flash-attention-v2-sram-tiling" (aiqz.cc), quiz question 10: take the
  larger maximum and rescale each partial sum to it), applied to the oracle on
  two halves of the keys, reproduces the oracle on all keys.
"""
import math

import numpy as np
import pytest

from oracle import ref


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_square_case_is_the_square_oracle(causal):
    rng = np.random.default_rng(11)
    q, k, v = _rand(rng, 37, 16), _rand(rng, 37, 16), _rand(rng, 37, 16)
    o, lse = ref.head_forward_rect(q, k, v, 0.3, causal)
    o2, lse2, _, _ = ref.head_forward(q, k, v, 0.3, causal)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("nq,nk", [(1, 50), (5, 50), (50, 50), (17, 300)])
def test_causal_row_is_noncausal_over_its_prefix(nq, nk):
    rng = np.random.default_rng(nq * 1000 + nk)
    q, k, v = _rand(rng, nq, 8), _rand(rng, nk, 8), _rand(rng, nk, 8)
    o, lse = ref.head_forward_rect(q, k, v, 0.5, True)
    for i in range(nq):
        last = i + nk - nq          # the query's own position
        oi, li = ref.head_forward_rect(q[i:i + 1], k[:last + 1], v[:last + 1], 0.5, False)
        np.testing.assert_allclose(o[i], oi[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[i], li[0], rtol=0, atol=1e-13)


def _brute(q, k, v, scale, causal):
    nq, nk, dv = len(q), len(k), len(v[0])
    o, lse = [], []
    for i in range(nq):
        keep = [j for j in range(nk) if not causal or j <= i + nk - nq]
        s = {j: scale * sum(q[i][c] * k[j][c] for c in range(len(q[i]))) for j in keep}
        z = sum(math.exp(s[j]) for j in keep)
        o.append([sum(math.exp(s[j]) / z * v[j][c] for j in keep) for c in range(dv)])
        lse.append(math.log(z))
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(1, 1), (1, 6), (2, 5), (3, 3)])
def test_brute_force_tiny(causal, nq, nk):
    rng = np.random.default_rng(7 + nq + 10 * nk)
    q, k, v = _rand(rng, nq, 3), _rand(rng, nk, 3), _rand(rng, nk, 2)
    o, lse = ref.head_forward_rect(q, k, v, 0.7, causal)
    ob, lb = _brute(q.tolist(), k.tolist(), v.tolist(), 0.7, causal)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_cpu_attention_cross_check(causal):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 2, 3, 9, 32), _rand(rng, 2, 3, 70, 32), _rand(rng, 2, 3, 70, 32)
    o, _ = ref.forward_rect(q, k, v, 0.2, causal)
    mask = None
    if causal:
        rows = np.arange(9)[:, None] + (70 - 9)
        mask = torch.from_numpy(np.arange(70)[None, :] <= rows)
    t = lambda a: torch.from_numpy(a)
    ot = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask, scale=0.2)
    np.testing.assert_allclose(o, ot.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("cut", [1, 13, 40, 63])
def test_merge_rule_of_two_key_ranges(cut):
    rng = np.random.default_rng(cut)
    q, k, v = _rand(rng, 4, 16) * 2, _rand(rng, 64, 16) * 2, _rand(rng, 64, 16)
    o1, lse1 = ref.head_forward_rect(q, k[:cut], v[:cut], 0.4, False)
    o2, lse2 = ref.head_forward_rect(q, k[cut:], v[cut:], 0.4, False)
    # each partial as (m, l, O) with l relative to its own maximum m: LSE = m + ln l
    m1, m2 = lse1, lse2            # any reference works; take l = 1 at m = LSE
    m = np.maximum(m1, m2)
    l = np.exp(m1 - m) + np.exp(m2 - m)
    o = (np.exp(m1 - m)[:, None] * o1 + np.exp(m2 - m)[:, None] * o2) / l[:, None]
    o_all, lse_all = ref.head_forward_rect(q, k, v, 0.4, False)
    np.testing.assert_allclose(o, o_all, rtol=0, atol=1e-13)
    np.testing.assert_allclose(m + np.log(l), lse_all, rtol=0, atol=1e-13)


def test_causal_needs_nq_not_above_nk():
    rng = np.random.default_rng(0)
    with pytest.raises(ValueError):
        ref.scores_rect(_rand(rng, 5, 4), _rand(rng, 4, 4), 1.0, True)


def test_heads_dict_matches_full():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 2, 2, 3, 8), _rand(rng, 2, 2, 20, 8), _rand(rng, 2, 2, 20, 8)
    o, lse = ref.forward_rect(q, k, v, 0.3, True)
    d = ref.forward_rect(q, k, v, 0.3, True, heads=[(1, 0)])
    np.testing.assert_array_equal(d[(1, 0)]["o"], o[1, 0])
    np.testing.assert_array_equal(d[(1, 0)]["lse"], lse[1, 0])


# ---- planted mistakes in the causal offset: each must fail the brute force --

def _mutant_scores(kind):
    def scores(q, k, scale, causal):
        nq, nk = q.shape[0], k.shape[0]
        s = scale * (q @ k.T)
        off = {"top_left": 0, "off_by_one": nk - nq - 1, "sign": nq - nk}[kind]
        rows = np.arange(nq)[:, None] + off
        return np.where(np.arange(nk)[None, :] > rows, -np.inf, s)
    return scores


@pytest.mark.parametrize("kind", ["top_left", "off_by_one", "sign"])
def test_offset_mistakes_fail_brute_force(monkeypatch, kind):
    rng = np.random.default_rng(19)
    q, k, v = _rand(rng, 3, 3), _rand(rng, 7, 3), _rand(rng, 7, 2)
    ob, _ = _brute(q.tolist(), k.tolist(), v.tolist(), 0.7, True)
    monkeypatch.setattr(ref, "scores_rect", _mutant_scores(kind))
    with np.errstate(invalid="ignore"):
        o, _ = ref.head_forward_rect(q, k, v, 0.7, True)
    assert not np.allclose(o, ob, atol=1e-6), kind
