"""GPU parity of the FP8 forward (fa_fwd_fp8, through the C ABI) against the
fp64 oracle on the values the e4m3fn codes stand for (code times descale,
exact in fp64).

Bar, derived from the arithmetic: S comes from the FP8 matrix instruction,
whose dot products of e4m3 codes are within 2^-14 sum_c |q_c k_c| of the exact
sum (measured on single dot products: test_fp8_score_error), so LSE meets the
bf16 bar of 1e-3 plus 2^-14 times the row's largest |scale| sum_c |q_c k_c|
(fp8_bound.lse_bar).  O differs from the exact result only through rounding each
probability (taken as 2^7 p, with every row holding one value 2^7) to e4m3
for the P V product: relative error <= 2^-4 in the normal range, absolute
<= 2^-10 below it, hence |O - O_ref| <= (2^-4 + N 2^-17) max|V| per head, plus
the bf16 rounding of O (2^-9 max|O|).  Inputs with sharp scores (q, k spread
3) are included so that a misplaced key cannot hide inside that bound: there
O follows a few rows of V closely.

That worst-case bound grows with max|V| while O of a long causal row
shrinks, so on its own it cannot see a misplaced key tile at N = 8192.  A
second, per-element bound uses that the roundings are independent: the error
of O_ic is sum_j P_ij e_ij V_jc with |e_ij| <= 2^-4, RMS <= 2^-4/sqrt(3), in
e4m3's normal range (2^7 p >= 2^-6), and absolute rounding <= 2^-17 on p
below it (RMS 2^-17/sqrt(12); the row sum l >= 1), so
  |O_ic - O_ref_ic| <= 7 sqrt(sum_j V_jc^2 (P_ij^2 2^-8 / 3 + 2^-34 / 12))
                       + 2^-9 |O_ref_ic|.
At seven standard deviations the chance that a correct kernel exceeds it is
below 1e-11 per element; a planted mistake in the oracle (one key tile
displaced by one tile) fails it at the full size.
"""
import math

import numpy as np
import pytest

import exact_tiled_attention_online_amd as fa
from exact_tiled_attention_online_amd import inputs as gen
from fp8_bound import SCORE_REL, displaced_tile, lse_bar, stat_ratio
from gpu_util import LSE_ATOL, log, to_np
from oracle import ref

pytestmark = pytest.mark.gpu


def run_fp8(x, causal, scale, layout=0):
    import torch
    def dev(a):
        a = np.ascontiguousarray(a.transpose(0, 2, 1, 3) if layout == fa.FA_LAYOUT_BNHD else a)
        return torch.from_numpy(a).cuda()
    q8, k8, v8 = (dev(x[n]) for n in ("q8", "k8", "v8"))
    o, lse = fa.forward_fp8(q8, k8, v8, x["descale_q"], x["descale_k"], x["descale_v"], causal, scale,
                            layout=layout)
    torch.cuda.synchronize()
    return {"o": to_np(o, layout), "lse": to_np(lse)}


def check(x, got, causal, scale, where):
    o_ref, lse_ref = ref.forward(x["q"], x["k"], x["v"], scale, causal)
    n = x["q"].shape[2]
    worst = 0.0
    for b in range(o_ref.shape[0]):
        for h in range(o_ref.shape[1]):
            vmax = float(np.abs(x["v"][b, h]).max())
            tol_o = (2.0 ** -4 + n * 2.0 ** -17) * vmax + 2.0 ** -9 * float(np.abs(o_ref[b, h]).max())
            err_o = float(np.abs(got["o"][b, h] - o_ref[b, h]).max())
            err_l = np.abs(got["lse"][b, h] - lse_ref[b, h])
            bar_l = lse_bar(x["q"][b, h].astype(np.float64), x["k"][b, h].astype(np.float64), scale, causal)
            assert np.isfinite(got["o"][b, h]).all() and np.isfinite(got["lse"][b, h]).all(), where
            assert (err_l <= bar_l).all(), f"{where} head ({b},{h}): LSE err {float(err_l.max()):.3e}"
            assert err_o <= tol_o, f"{where} head ({b},{h}): O err {err_o:.3e} > {tol_o:.3e}"
            worst = max(worst, err_o / tol_o)
    return worst


CASES = [(n, causal, sig) for n in (1, 17, 64, 129, 300, 1000) for causal in (False, True) for sig in (1.0, 3.0)]


@pytest.mark.parametrize("n,causal,sig", CASES)
def test_fp8_forward_matches_oracle(n, causal, sig):
    log(f"[fp8] N={n} causal={causal} sigma_qk={sig}")
    x = gen.make_fp8_inputs((2, 3, n, 128), seed=300 + n, sigma_qk=sig)
    scale = 1.0 / math.sqrt(128)
    got = run_fp8(x, causal, scale)
    r = check(x, got, causal, scale, f"fp8 N{n} c{int(causal)} s{sig}")
    rs = max(stat_ratio(x["q"][b, h], x["k"][b, h], x["v"][b, h], got["o"][b, h], scale, causal)
             for b in range(2) for h in range(3))
    log(f"  worst O error / bound {r:.3f}, / per-element bound {rs:.3f}")
    assert rs <= 1.0, rs


def test_fp8_forward_other_descales_and_bnhd():
    log("[fp8] descales, BNHD")
    x = gen.make_fp8_inputs((1, 4, 500, 128), seed=71, sigma_qk=2.0, descale=2.0 ** -5)
    x["descale_v"] = 0.37          # any positive descale: the values are code * descale
    x["v"] = gen.e4m3_to_f32(x["v8"]) * np.float32(0.37)
    for layout in (fa.FA_LAYOUT_BHND, fa.FA_LAYOUT_BNHD):
        for causal in (False, True):
            got = run_fp8(x, causal, 0.11, layout)
            check(x, got, causal, 0.11, f"fp8 layout{layout} c{int(causal)}")


def test_fp8_forward_full_size_sampled_heads():
    """The causal 1 x 32 x 8192 x 128 shape in the benchmark's launch
    configuration, checked on whole sampled heads."""
    import torch
    log("[fp8] full size")
    shape = (1, 32, 8192, 128)
    x = gen.make_fp8_inputs(shape, seed=4)
    q8, k8, v8 = (torch.from_numpy(x[n]).cuda() for n in ("q8", "k8", "v8"))
    scale = 1.0 / math.sqrt(128)
    o, lse = fa.forward_fp8(q8, k8, v8, x["descale_q"], x["descale_k"], x["descale_v"], True, scale)
    torch.cuda.synchronize()
    got_o, got_l = to_np(o), to_np(lse)
    assert np.isfinite(got_o).all() and np.isfinite(got_l).all()
    for h in (0, 15, 31):
        want = ref.forward_rect(x["q"], x["k"], x["v"], scale, True, heads=[(0, h)])[(0, h)]
        vmax = float(np.abs(x["v"][0, h]).max())
        tol = (2.0 ** -4 + 8192 * 2.0 ** -17) * vmax + 2.0 ** -9 * float(np.abs(want["o"]).max())
        assert float(np.abs(got_o[0, h] - want["o"]).max()) <= tol, h
        bar_l = lse_bar(x["q"][0, h].astype(np.float64), x["k"][0, h].astype(np.float64), scale, True)
        assert (np.abs(got_l[0, h] - want["lse"]) <= bar_l).all(), h
        r = stat_ratio(x["q"][0, h], x["k"][0, h], x["v"][0, h], got_o[0, h], scale, True)
        log(f"  head {h}: O error / per-element bound {r:.3f}")
        assert r <= 1.0, (h, r)
    # the per-element bound sees a displaced key tile that the worst-case
    # bound lets pass: checked against an oracle with that planted mistake
    k2, v2 = displaced_tile(x["k"][0, 0], x["v"][0, 0], at=40)
    r_bad = stat_ratio(x["q"][0, 0], k2, v2, got_o[0, 0], scale, True)
    log(f"  planted displaced tile: ratio {r_bad:.2f}")
    assert r_bad > 1.0, r_bad
    del q8, k8, v8, o, lse
    torch.cuda.empty_cache()


SPLIT_CASES = [
    # B, H, Nq, Nk, causal, num_splits
    (2, 3, 1, 1000, True, 0),
    (1, 4, 7, 513, False, 3),
    (2, 2, 32, 4096, True, 0),
    (1, 2, 33, 2000, True, 5),
    (1, 2, 100, 100, True, 0),
    (3, 2, 5, 31, False, 0),
]


@pytest.mark.parametrize("B,H,Nq,Nk,causal,ns", SPLIT_CASES)
def test_fp8_split_forward_matches_oracle(B, H, Nq, Nk, causal, ns):
    """The split-key-range FP8 forward (decode against an FP8 cache) meets the
    same bound: each range's O is a convex combination with the bound above
    (N = its keys), and the merge mixes them with weights summing to one."""
    import torch
    log(f"[fp8-split] B={B} H={H} Nq={Nq} Nk={Nk} causal={causal} splits={ns}")
    xq = gen.make_fp8_inputs((B, H, Nq, 128), seed=500 + Nq + Nk, sigma_qk=2.0)
    xk = gen.make_fp8_inputs((B, H, Nk, 128), seed=600 + Nq + Nk, sigma_qk=2.0)
    q8, k8, v8 = (torch.from_numpy(a).cuda() for a in (xq["q8"], xk["k8"], xk["v8"]))
    scale = 1.0 / math.sqrt(128)
    o, lse = fa.forward_splitkv_fp8(q8, k8, v8, xq["descale_q"], xk["descale_k"], xk["descale_v"], causal, scale,
                                    num_splits=ns)
    torch.cuda.synchronize()
    got_o, got_l = to_np(o), to_np(lse)
    ro, rl = ref.forward_rect(xq["q"], xk["k"], xk["v"], scale, causal)
    for b in range(B):
        for h in range(H):
            vmax = float(np.abs(xk["v"][b, h]).max())
            tol = (2.0 ** -4 + Nk * 2.0 ** -17) * vmax + 2.0 ** -9 * float(np.abs(ro[b, h]).max())
            assert float(np.abs(got_o[b, h] - ro[b, h]).max()) <= tol, (b, h)
            bar_l = lse_bar(xq["q"][b, h].astype(np.float64), xk["k"][b, h].astype(np.float64), scale, causal)
            assert (np.abs(got_l[b, h] - rl[b, h]) <= bar_l).all(), (b, h)


@pytest.mark.parametrize("H,d", [(32, 128), (16, 256)])
def test_fp8_forward_maximum_size_sampled_heads(H, d):
    """The FP8 forward at the largest shape of the headline geometry: B=63,
    H=32, N=8192, d=128 causal (and its d = 256 counterpart, H=16), 2.11e9
    one-byte codes per tensor (generated on the device: normal values over
    the descale, clipped to the largest finite e4m3fn value); three whole
    heads against the oracle on the values the codes stand for, with the
    bound above."""
    import torch
    B, N = 63, 8192
    ds, scale = 2.0 ** -5, 1.0 / math.sqrt(d)
    log(f"[fp8 max size] B={B} H={H} N={N} d={d} causal")
    g = torch.Generator(device="cuda").manual_seed(8863)

    def codes():
        x = torch.randn((B, H, N, d), generator=g, device="cuda", dtype=torch.float32)
        x.mul_(1.0 / ds).clamp_(-448.0, 448.0)
        return x.to(torch.float8_e4m3fn).view(torch.uint8)

    q8, k8, v8 = codes(), codes(), codes()
    o, lse = fa.forward_fp8(q8, k8, v8, ds, ds, ds, True, scale)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (25, 7), (B - 1, H - 1)):
        x = {n: (gen.e4m3_to_f32(t[b, h].cpu().numpy()).astype(np.float64) * ds)[None, None]
             for n, t in (("q", q8), ("k", k8), ("v", v8))}
        got = {"o": to_np(o[b, h])[None, None], "lse": to_np(lse[b, h])[None, None]}
        r = check(x, got, True, scale, f"fp8 max size head ({b},{h})")
        rs = stat_ratio(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], got["o"][0, 0], scale, True)
        log(f"  head ({b},{h}) worst O error / bound {r:.3f}, / per-element bound {rs:.3f}")
        assert rs <= 1.0, rs
    del q8, k8, v8, o, lse
    torch.cuda.empty_cache()


# head dims 64 and 96: LDS rows of 128 bytes with 4 or 6 chunks of data; at d =
# 96 the second 64-wide K-step of S multiplies the padding chunks by the
# zeros Q holds past d.  d = 256: LDS rows of 256 bytes, four 64-wide K-steps
HD_CASES = [(d, n, causal, sig) for d in (64, 96, 256) for n in (1, 17, 129, 300) for causal in (False, True)
            for sig in (1.0, 3.0)]


@pytest.mark.parametrize("d,n,causal,sig", HD_CASES)
def test_fp8_forward_other_head_dims(d, n, causal, sig):
    log(f"[fp8 d{d}] N={n} causal={causal} sigma_qk={sig}")
    x = gen.make_fp8_inputs((2, 3, n, d), seed=700 + n + d, sigma_qk=sig)
    scale = 1.0 / math.sqrt(d)
    got = run_fp8(x, causal, scale)
    r = check(x, got, causal, scale, f"fp8 d{d} N{n} c{int(causal)} s{sig}")
    rs = max(stat_ratio(x["q"][b, h], x["k"][b, h], x["v"][b, h], got["o"][b, h], scale, causal)
             for b in range(2) for h in range(3))
    log(f"  worst O error / bound {r:.3f}, / per-element bound {rs:.3f}")
    assert rs <= 1.0, rs


@pytest.mark.parametrize("d", [64, 96, 256])
def test_fp8_forward_other_head_dims_larger_size(d):
    """Whole heads of a causal 1 x 4 x 4096 shape (64 key tiles) in both
    layouts, with the planted displaced tile that the per-element bound must
    reject."""
    log(f"[fp8 d{d}] 1x4x4096 causal")
    x = gen.make_fp8_inputs((1, 4, 4096, d), seed=800 + d)
    scale = 1.0 / math.sqrt(d)
    for layout in (fa.FA_LAYOUT_BHND, fa.FA_LAYOUT_BNHD):
        got = run_fp8(x, True, scale, layout)
        check(x, got, True, scale, f"fp8 d{d} 4096 layout{layout}")
        for h in range(4):
            r = stat_ratio(x["q"][0, h], x["k"][0, h], x["v"][0, h], got["o"][0, h], scale, True)
            assert r <= 1.0, (layout, h, r)
    k2, v2 = displaced_tile(x["k"][0, 1], x["v"][0, 1], at=30)
    r_bad = stat_ratio(x["q"][0, 1], k2, v2, got["o"][0, 1], scale, True)
    log(f"  planted displaced tile: ratio {r_bad:.2f}")
    assert r_bad > 1.0, r_bad


@pytest.mark.parametrize("d", [64, 96, 256])
@pytest.mark.parametrize("B,H,Nq,Nk,causal,ns", [(2, 3, 1, 1000, True, 0), (1, 2, 33, 2000, True, 5),
                                                 (1, 4, 7, 513, False, 3)])
def test_fp8_split_forward_other_head_dims(d, B, H, Nq, Nk, causal, ns):
    import torch
    log(f"[fp8-split d{d}] B={B} H={H} Nq={Nq} Nk={Nk} causal={causal} splits={ns}")
    xq = gen.make_fp8_inputs((B, H, Nq, d), seed=900 + Nq + Nk + d, sigma_qk=2.0)
    xk = gen.make_fp8_inputs((B, H, Nk, d), seed=950 + Nq + Nk + d, sigma_qk=2.0)
    q8, k8, v8 = (torch.from_numpy(a).cuda() for a in (xq["q8"], xk["k8"], xk["v8"]))
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.forward_splitkv_fp8(q8, k8, v8, xq["descale_q"], xk["descale_k"], xk["descale_v"], causal, scale,
                                    num_splits=ns)
    torch.cuda.synchronize()
    got_o, got_l = to_np(o), to_np(lse)
    ro, rl = ref.forward_rect(xq["q"], xk["k"], xk["v"], scale, causal)
    for b in range(B):
        for h in range(H):
            vmax = float(np.abs(xk["v"][b, h]).max())
            tol = (2.0 ** -4 + Nk * 2.0 ** -17) * vmax + 2.0 ** -9 * float(np.abs(ro[b, h]).max())
            assert float(np.abs(got_o[b, h] - ro[b, h]).max()) <= tol, (b, h)
            bar_l = lse_bar(xq["q"][b, h].astype(np.float64), xk["k"][b, h].astype(np.float64), scale, causal)
            assert (np.abs(got_l[b, h] - rl[b, h]) <= bar_l).all(), (b, h)


def test_fp8_score_error():
    """The accuracy of the FP8 matrix instruction's dot products, which the
    LSE bar above rests on: with one query and one key per head, LSE is
    exactly scale * q.k, so its error is the error of S.  4096 heads per
    head dim and input spread; every one within 2^-14 sum_c |q_c k_c|."""
    import torch
    worst = 0.0
    for d in (64, 96, 128, 256):
        for sig in (0.25, 1.0, 4.0):
            x = gen.make_fp8_inputs((1, 4096, 1, d), seed=11 + d, sigma_qk=sig)
            q8, k8, v8 = (torch.from_numpy(x[n]).cuda() for n in ("q8", "k8", "v8"))
            o, lse = fa.forward_fp8(q8, k8, v8, x["descale_q"], x["descale_k"], x["descale_v"], False, 1.0)
            torch.cuda.synchronize()
            q, k = x["q"].astype(np.float64), x["k"].astype(np.float64)
            s = (q * k).sum(axis=3)
            r = np.abs(to_np(lse) - s) / (SCORE_REL * np.abs(q * k).sum(axis=3) + 1e-30)
            log(f"  d={d} spread {sig}: worst error / (2^-14 sum|q_c k_c|) {float(r.max()):.3f}")
            worst = max(worst, float(r.max()))
    assert worst <= 1.0, worst
