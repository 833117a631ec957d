"""The per-element error bound of the FP8 forward (see tests/test_fp8_gpu.py):
the e4m3 rounding of each probability contributes sum_j P_ij e_ij V_jc to
O_ic, with independent e_ij of RMS <= 2^-4/sqrt(3) in e4m3's normal range
and absolute rounding <= 2^-17 of p below it, so
  |O_ic - O_ref_ic| <= 7 sqrt(sum_j V_jc^2 (P_ij^2 2^-8 / 3 + 2^-34 / 12))
                       + 2^-9 |O_ref_ic|,
and a planted mistake for the oracle (a displaced key tile).  Shared by the
GPU tests and the CPU test that calibrates the bound on an emulation."""
import numpy as np


def stat_ratio(q, k, v, o, scale, causal, panel=512):
    """Worst ratio of |O - O_ref| to the per-element bound of the module
    docstring, for one head (q [N, d], k and v [Nk, d] in fp64, o [N, d] from
    the kernel), computed in row panels of the fp64 probabilities."""
    n, nk = q.shape[0], k.shape[0]
    worst = 0.0
    v2 = v * v
    for r0 in range(0, n, panel):
        r1 = min(n, r0 + panel)
        s = scale * (q[r0:r1] @ k.T)
        if causal:
            off = nk - n
            rows = np.arange(r0, r1)[:, None] + off
            s = np.where(np.arange(nk)[None, :] > rows, -np.inf, s)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o_ref = p @ v
        var = (p * p) @ v2 * (2.0 ** -8 / 3.0) + v2.sum(axis=0)[None, :] * (2.0 ** -34 / 12.0)
        bound = 7.0 * np.sqrt(var) + 2.0 ** -9 * np.abs(o_ref) + 1e-7
        worst = max(worst, float((np.abs(o[r0:r1] - o_ref) / bound).max()))
    return worst


def displaced_tile(k, v, tile=64, at=1):
    """A planted mistake for the oracle: key/value rows of tile `at` replaced
    by those of the next tile (a kernel reading the wrong key tile)."""
    k2, v2 = k.copy(), v.copy()
    k2[at * tile:(at + 1) * tile] = k[(at + 1) * tile:(at + 2) * tile]
    v2[at * tile:(at + 1) * tile] = v[(at + 1) * tile:(at + 2) * tile]
    return k2, v2




# The FP8 matrix instruction does not add the 32 or 64 code products of a
# dot product exactly in fp32: measured on single dot products (N = 1, so that
# LSE = scale * q.k; tests/test_fp8_gpu.py::test_fp8_score_error), its result
# differs from the exact sum by up to 1.96e-5 (about 2^-15.6) times
# sum_c |q_c k_c|, for d = 64 and 128 and spreads 0.25 to 4.  The LSE bar of
# the FP8 forward therefore adds 2^-14 (three times that) times the largest
# |scale| sum_c |q_ic k_jc| of the row to the bf16 bar of 1e-3.
SCORE_REL = 2.0 ** -14


def lse_bar(q, k, scale, causal, lse_atol=1e-3, panel=512):
    """Per-row LSE tolerance of the FP8 forward for one head (q [Nq, d], k
    [Nk, d] in fp64; causal with the query rows at the end of the keys)."""
    n, nk = q.shape[0], k.shape[0]
    out = np.empty(n)
    aq, ak = np.abs(q), np.abs(k)
    for r0 in range(0, n, panel):
        r1 = min(n, r0 + panel)
        m = aq[r0:r1] @ ak.T
        if causal:
            rows = np.arange(r0, r1)[:, None] + (nk - n)
            m = np.where(np.arange(nk)[None, :] > rows, 0.0, m)
        out[r0:r1] = lse_atol + SCORE_REL * abs(scale) * m.max(axis=1)
    return out
