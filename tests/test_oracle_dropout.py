"""Pins of the dropout oracle (oracle/dropout.py) against things other than
itself: numpy's own Philox4x64-10 for the generator's rounds, a per-element
loop for the block mapping, binomial bounds for the drop rate, t = 0 against
the plain oracle, central finite differences for the gradients with the
mask held fixed, and the expectation over seeds for the keep scale.  Each
pin is shown to catch a planted mistake."""
import numpy as np
import pytest

from oracle import dropout as dr
from oracle import ref

RNG = np.random.default_rng(20261202)
U64 = (1 << 64) - 1


# ---- generator ---------------------------------------------------------------

@pytest.mark.parametrize("case", range(6))
def test_philox_rounds_match_numpy_philox4x64(case):
    """The round function at width 64 is numpy's Philox4x64-10: numpy advances
    its 256-bit counter (word 0 first, carrying upward) before each block of
    four outputs, so its first block is the oracle's on counter + 1."""
    key = [int(x) for x in RNG.integers(0, 1 << 63, 2, dtype=np.uint64)]
    ctr = [int(x) for x in RNG.integers(0, 1 << 63, 4, dtype=np.uint64)]
    if case == 5:
        ctr[0], ctr[1] = U64, U64   # the increment carries into word 2
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
    raw = [int(x) for x in g.random_raw(12)]
    c = ctr[0] | (ctr[1] << 64) | (ctr[2] << 128) | (ctr[3] << 192)
    for blk in range(3):
        n = (c + 1 + blk) % (1 << 256)
        words = [(n >> (64 * w)) & U64 for w in range(4)]
        assert list(dr.philox_scalar(words, key, width=64)) == raw[4 * blk:4 * blk + 4]


def _kat():
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "philox4x32_10_kat.json")
    return [([int(w, 16) for w in v["ctr"]], [int(w, 16) for w in v["key"]], [int(w, 16) for w in v["out"]])
            for v in json.load(open(path))["vectors"]]


def test_philox4x32_known_answers():
    """The 32-bit generator (the one the mask uses) reproduces the published
    Philox4x32-10 known-answer vectors, scalar and vectorised: this pins its
    constants, which the width-64 comparison with numpy does not reach."""
    for ctr, key, want in _kat():
        assert list(dr.philox_scalar(ctr, key, width=32)) == want
        got = dr.philox4x32_10(*(np.array([c]) for c in ctr), *key)
        assert [int(x[0]) for x in got] == want


@pytest.mark.parametrize("name", ["M0", "M1", "W0", "W1"])
def test_philox4x32_known_answers_catch_a_mistyped_constant(monkeypatch, name):
    """One flipped bit in any of the four 32-bit constants fails the vectors."""
    bad = dict(dr.PHILOX[32])
    bad[name] ^= 1 << 7
    monkeypatch.setitem(dr.PHILOX, 32, bad)
    assert any(list(dr.philox_scalar(ctr, key, width=32)) != want for ctr, key, want in _kat())


def test_philox_width64_catches_swapped_outputs():
    """A round that swaps its two multiplier lanes no longer matches numpy."""
    key, ctr = [3, 5], [7, 11, 13, 17]
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
    want = [int(x) for x in g.random_raw(4)]
    c = dr.PHILOX[64]
    mask = U64
    x0, x1, x2, x3 = ctr[0] + 1, ctr[1], ctr[2], ctr[3]
    k0, k1 = key
    for _ in range(10):
        p0, p1 = c["M0"] * x0, c["M1"] * x2
        # planted: the high halves xor the wrong words
        x0, x1, x2, x3 = ((p0 >> 64) ^ x1 ^ k0, p1 & mask, (p1 >> 64) ^ x3 ^ k1, p0 & mask)
        k0, k1 = (k0 + c["W0"]) & mask, (k1 + c["W1"]) & mask
    assert [x0, x1, x2, x3] != want
    assert list(dr.philox_scalar([ctr[0] + 1] + ctr[1:], key, width=64)) == want


def test_philox4x32_vectorised_matches_scalar():
    n = 300
    ctr = RNG.integers(0, 1 << 32, (4, n), dtype=np.uint64)
    ctr[:, :4] = 0xFFFFFFFF
    ctr[:, 4:8] = 0
    key = [int(x) for x in RNG.integers(0, 1 << 32, 2, dtype=np.uint64)]
    xs = dr.philox4x32_10(ctr[0], ctr[1], ctr[2], ctr[3], key[0], key[1])
    for i in range(n):
        want = dr.philox_scalar([int(ctr[w, i]) for w in range(4)], key, width=32)
        assert tuple(int(xs[w][i]) for w in range(4)) == want


def test_philox4x32_words_are_uniform():
    """Each output word is uniform on 32 bits: byte histograms of 2^16 blocks
    pass a chi-square bound (p < 1e-6 would fail)."""
    j = np.arange(1 << 16, dtype=np.uint64)
    xs = dr.philox4x32_10(j, 0, 3, 9, 0x1234, 0x5678)
    for x in xs:
        for b in range(4):
            cnt = np.bincount(((x >> np.uint64(8 * b)) & np.uint64(0xFF)).astype(np.int64), minlength=256)
            e = len(j) / 256
            chi2 = float(((cnt - e) ** 2 / e).sum())
            assert chi2 < 380.0   # 255 degrees of freedom; P(chi2 > 380) ~ 1e-6


# ---- block mapping -------------------------------------------------------------

@pytest.mark.parametrize("nq,nk,row0,rows", [(13, 13, 0, None), (9, 22, 0, None), (30, 30, 5, 11)])
def test_keep_mask_matches_per_element_definition(nq, nk, row0, rows):
    bh, seed, offset, t = 5, 0x0123456789ABCDEF, 77, 100
    z = dr.keep_mask(bh, seed, offset, t, nq, nk, row0=row0, rows=rows)
    nrows = nq - row0 if rows is None else rows
    assert z.shape == (nrows, nk)
    for i in range(row0, row0 + nrows):
        for j in range(nk):
            x = dr.philox_scalar([j // 4, i // 4, bh, offset], [seed & 0xFFFFFFFF, seed >> 32], width=32)
            byte = (x[i % 4] >> (8 * (j % 4))) & 0xFF
            assert z[i - row0, j] == (byte >= t), (i, j)


@pytest.mark.parametrize("t", [0, 1, 26, 64, 128, 255])
def test_drop_rate_is_t_over_256(t):
    n = 512
    z = dr.keep_mask(0, 42, 0, t, n, n)
    p = t / 256
    drop = 1.0 - z.mean()
    sd = np.sqrt(p * (1 - p) / z.size)
    assert abs(drop - p) <= 6 * sd + 1e-12
    if t == 0:
        assert z.all()


def test_masks_differ_across_heads_seeds_offsets():
    """Two masks that share any of (bh, seed, offset) but not all agree on a
    fraction p^2 + (1-p)^2 of entries, as independent draws do."""
    n, t = 256, 128
    base = dr.keep_mask(0, 9, 0, t, n, n)
    for other in (dr.keep_mask(1, 9, 0, t, n, n), dr.keep_mask(0, 10, 0, t, n, n),
                  dr.keep_mask(0, 9, 1, t, n, n), dr.keep_mask(0, 9 + (1 << 32), 0, t, n, n)):
        agree = (base == other).mean()
        assert abs(agree - 0.5) < 6 * np.sqrt(0.25 / base.size)
    assert (dr.keep_mask(0, 9, 0, t, n, n) == base).all()


# ---- attention with dropout ---------------------------------------------------------

def _head(n, d, seed):
    r = np.random.default_rng(seed)
    return [r.standard_normal((n, d)) for _ in range(4)]


@pytest.mark.parametrize("causal", [False, True])
def test_t0_is_the_plain_oracle(causal):
    q, k, v, do = _head(21, 8, 1)
    sc = 8 ** -0.5
    got = dr.head_panel_dropout(q, k, v, do, sc, causal, 3, 99, 0, 0, panel_rows=8)
    want = ref.head_panel(q, k, v, do, sc, causal)
    for n in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_allclose(got[n], want[n], rtol=0, atol=1e-13)


def _loss(q, k, v, do, sc, causal, keep, t):
    o, _, _, _ = dr.head_forward_dropout(q, k, v, sc, causal, keep, t)
    return float((do * o).sum())


def _fd_errors(backward, n, d, causal, t, seed, h=1e-5):
    q, k, v, do = _head(n, d, seed)
    sc = 0.7
    keep = dr.keep_mask(2, 1234, 5, t, n, n)
    got = backward(q, k, v, do, sc, causal, keep, t)
    errs = []
    for x, g in zip((q, k, v), got):
        num = np.empty_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, sc, causal, keep, t)
            x[idx] = old - h
            lm = _loss(q, k, v, do, sc, causal, keep, t)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        errs.append(float(np.abs(num - g).max() / max(1.0, np.abs(num).max())))
    return errs, keep


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("t", [64, 160])
def test_gradients_match_finite_differences(causal, t):
    errs, keep = _fd_errors(dr.head_backward_dropout, 9, 4, causal, t, seed=7)
    assert not keep.all() and keep.any()
    assert max(errs) < 1e-7, errs


def _bwd_unmasked_dp(q, k, v, do, sc, causal, keep, t):
    """Planted mistake: dP taken without the mask and the keep scale."""
    o, lse, p, pd = dr.head_forward_dropout(q, k, v, sc, causal, keep, t)
    d_row = (do * o).sum(axis=1)
    ds = p * (do @ v.T - d_row[:, None])
    return sc * (ds @ k), sc * (ds.T @ q), pd.T @ do


def _bwd_unscaled_dv(q, k, v, do, sc, causal, keep, t):
    """Planted mistake: dV from the masked probabilities without the keep scale."""
    dq, dk, dv, it = dr.head_backward_dropout(q, k, v, do, sc, causal, keep, t, want_intermediates=True)
    return dq, dk, dv / dr.keep_scale(t)


@pytest.mark.parametrize("mutant", [_bwd_unmasked_dp, _bwd_unscaled_dv])
def test_finite_differences_catch_planted_mistakes(mutant):
    errs, _ = _fd_errors(mutant, 9, 4, True, 64, seed=7)
    assert max(errs) > 1e-3, errs


def test_row_term_identity_with_dropout():
    q, k, v, do = _head(17, 6, 3)
    keep = dr.keep_mask(0, 5, 0, 90, 17, 17)
    _, _, _, it = dr.head_backward_dropout(q, k, v, do, 0.4, True, keep, 90, want_intermediates=True)
    np.testing.assert_allclose((it["p"] * it["dp"]).sum(axis=1), it["D"], rtol=1e-12, atol=1e-12)


def test_expectation_over_seeds_is_the_plain_output():
    """E_Z[O] = O: the keep scale undoes the dropped mass on average.  The
    mean over 3000 seeds is within 6 standard errors of the plain O; without
    the keep scale it would sit at (1 - t/256) O."""
    n, d, t = 8, 3, 96
    q, k, v, _ = _head(n, d, 11)
    sc = 0.9
    o_plain, _, _, _ = ref.head_forward(q, k, v, sc, False)
    samples = np.stack([dr.head_forward_dropout(q, k, v, sc, False, dr.keep_mask(0, s, 0, t, n, n), t)[0]
                        for s in range(3000)])
    mean, se = samples.mean(axis=0), samples.std(axis=0) / np.sqrt(len(samples))
    assert (np.abs(mean - o_plain) <= 6 * se + 1e-12).all()
    unscaled = mean / dr.keep_scale(t)
    assert not (np.abs(unscaled - o_plain) <= 6 * se + 1e-12).all()


@pytest.mark.parametrize("causal", [False, True])
def test_panels_match_whole_head(causal):
    """Panels of 5 rows (not a multiple of the 4-row blocks) give the same
    result as the whole head with the whole mask."""
    n, d, t = 23, 5, 77
    q, k, v, do = _head(n, d, 4)
    keep = dr.keep_mask(6, 31, 2, t, n, n)
    dq, dk, dv, it = dr.head_backward_dropout(q, k, v, do, 0.5, causal, keep, t, want_intermediates=True)
    got = dr.head_panel_dropout(q, k, v, do, 0.5, causal, 6, 31, 2, t, panel_rows=5)
    for name, want in (("o", it["o"]), ("lse", it["lse"]), ("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_allclose(got[name], want, rtol=1e-12, atol=1e-12)


def test_batched_wrapper_head_index():
    """forward_backward_dropout numbers heads b*H + h."""
    r = np.random.default_rng(0)
    x = [r.standard_normal((2, 3, 10, 4)) for _ in range(4)]
    out = dr.forward_backward_dropout(*x, 0.5, True, 8, 1, 128, heads=[(1, 2)])
    want = dr.head_panel_dropout(*(a[1, 2] for a in x), 0.5, True, 5, 8, 1, 128)
    for n in want:
        np.testing.assert_array_equal(out[(1, 2)][n], want[n])
