"""Calibration of the FP8 forward's per-element bound on the CPU: an fp64
emulation of the arithmetic the bound describes (probabilities against the
exact row maximum, scaled by 2^7 and rounded to e4m3 with the input encoder
of inputs.py, summed against V, divided by the row sum, O rounded to bf16)
stays inside it, and the same result measured against an oracle with one
displaced key tile exceeds it, while the worst-case bound cannot tell the
two apart."""
import math

import numpy as np

from exact_tiled_attention_online_amd import inputs as gen
from fp8_bound import displaced_tile, stat_ratio


def _emulated(n, seed):
    x = gen.make_fp8_inputs((1, 1, n, 128), seed=seed)
    q, k, v = (x[name][0, 0].astype(np.float64) for name in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(128)
    s = scale * (q @ k.T)
    s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    l = p.sum(axis=1, keepdims=True)
    pq = gen.e4m3_to_f32(gen.e4m3_bits((p * 128.0).astype(np.float32))).astype(np.float64) / 128.0
    o = gen.round_bf16(((pq @ v) / l).astype(np.float32)).astype(np.float64)
    return q, k, v, o, scale


def _worst_case_ratio(q, k, v, o, scale):
    n = q.shape[0]
    s = scale * (q @ k.T)
    s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    o_ref = p @ v
    tol = (2.0 ** -4 + n * 2.0 ** -17) * np.abs(v).max() + 2.0 ** -9 * np.abs(o_ref).max()
    return float(np.abs(o - o_ref).max() / tol)


def test_per_element_bound_holds_for_the_emulation_and_sees_a_displaced_tile():
    q, k, v, o, scale = _emulated(3072, seed=4)
    assert stat_ratio(q, k, v, o, scale, True) <= 0.8
    k2, v2 = displaced_tile(k, v, at=20)
    assert stat_ratio(q, k2, v2, o, scale, True) > 2.0
    # the worst-case bound passes both
    assert _worst_case_ratio(q, k, v, o, scale) < 0.5 and _worst_case_ratio(q, k2, v2, o, scale) < 0.5
