"""Seeded synthetic inputs for the attention workloads.

This module holds the workload table and the input recipe only: shapes,
value distributions, seeds and the fp32 -> bf16 rounding of the inputs.  It
contains none of the attention arithmetic, so both the HIP path's tests and the
fp64 oracle can be fed from it without sharing any of the method's code.

Recipe: ``numpy.random.default_rng(seed)``; draw order q, k, v, dO; each is
``standard_normal((B, H, N, d), float32) * sigma``; for bf16 workloads every
value is then rounded to the nearest bf16 (ties to even), so the GPU and the
oracle see identical numbers.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "round_bf16", "bf16_bits",
           "make_inputs", "default_scale", "DecodeWorkload", "DECODE", "make_decode_inputs",
           "e4m3_bits", "e4m3_to_f32", "make_fp8_inputs", "FP8_DESCALE"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "fp32" or "bf16"
    causal: bool
    sigma_qk: float     # std of q and k
    sigma_vdo: float    # std of v and dO
    seed: int

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    def flops(self):
        """Credited FLOPs (fwd, bwd): 4*B*H*N^2*d and 10*B*H*N^2*d, halved if causal."""
        base = self.B * self.H * self.N * self.N * self.d
        f = 0.5 if self.causal else 1.0
        return 4.0 * base * f, 10.0 * base * f


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


# The five workloads: a small fp32 case, a non-causal bf16 case, two causal
# d=128 cases (the 8192-token, 32-head one is the headline shape) and a
# 32768-token case with sharper scores (q, k drawn with std 2).
WORKLOADS = [
    Workload("c1_fp32_n128_d64", 1, 1, 128, 64, "fp32", False, 1.0, 1.0, 1),
    Workload("c2_bf16_b4h16_n1024_d64", 4, 16, 1024, 64, "bf16", False, 1.0, 1.0, 2),
    Workload("c3_bf16_b2h16_n4096_d128_causal", 2, 16, 4096, 128, "bf16", True, 1.0, 1.0, 3),
    Workload("c4_bf16_b1h32_n8192_d128_causal", 1, 32, 8192, 128, "bf16", True, 1.0, 1.0, 4),
    Workload("c5_bf16_b1h8_n32768_d128_causal", 1, 8, 32768, 128, "bf16", True, 2.0, 1.0, 5),
]


def workload(key) -> Workload:
    """Look a workload up by index (0..4), by short name ('c1'..'c5') or full name."""
    if isinstance(key, int):
        return WORKLOADS[key]
    for w in WORKLOADS:
        if w.name == key or w.name.split("_")[0] == key:
            return w
    raise KeyError(key)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even); float32 out."""
    return bf16_to_f32(bf16_bits(x))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bf16 encodings of float32 values, round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_inputs(w: Workload, shape=None, seed=None, sigma_qk=None, sigma_vdo=None,
                dtype=None):
    """Seeded q, k, v, dO as float32 numpy arrays (bf16-representable for bf16).

    The keyword arguments override the workload's own shape, seed, spreads or
    dtype, for edge-case tests that reuse the recipe at other sizes.
    """
    shape = tuple(shape) if shape is not None else w.shape
    seed = w.seed if seed is None else seed
    sqk = w.sigma_qk if sigma_qk is None else sigma_qk
    svd = w.sigma_vdo if sigma_vdo is None else sigma_vdo
    dtype = w.dtype if dtype is None else dtype
    rng = np.random.default_rng(seed)
    out = {}
    for name, sig in (("q", sqk), ("k", sqk), ("v", svd), ("do", svd)):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if sig != 1.0:
            x *= np.float32(sig)
        if dtype == "bf16":
            x = round_bf16(x)
        out[name] = x
    return out


@dataclass(frozen=True)
class DecodeWorkload:
    """Nq query rows per head against a cache of Nk key/value rows."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool
    sigma_qk: float
    sigma_v: float
    seed: int

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    def kv_bytes(self) -> int:
        """Bytes of K and V, each read once by the split-key-range forward."""
        return 2 * self.B * self.H * self.Nk * self.d * (2 if self.dtype == "bf16" else 4)


# One decode step of a 32-head, d = 128 model for a batch of 8 sequences with
# 16384 cached tokens each (the queries are the newest positions).
DECODE = DecodeWorkload("decode_bf16_b8h32_q1_k16384_d128", 8, 32, 1, 16384, 128, "bf16", True,
                        1.0, 1.0, 6)


def make_decode_inputs(B, H, Nq, Nk, d, seed, dtype="bf16", sigma_qk=1.0, sigma_v=1.0):
    """Seeded q [B,H,Nq,d], k and v [B,H,Nk,d] as float32 numpy arrays.

    Same recipe as ``make_inputs``: one generator, draw order q, k, v, each
    standard normal times its spread, rounded to bf16 for bf16 workloads.
    """
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape, sig in (("q", (B, H, Nq, d), sigma_qk), ("k", (B, H, Nk, d), sigma_qk),
                             ("v", (B, H, Nk, d), sigma_v)):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if sig != 1.0:
            x *= np.float32(sig)
        if dtype == "bf16":
            x = round_bf16(x)
        out[name] = x
    return out


# ---- FP8 (OCP e4m3fn) inputs ---------------------------------------------------
#
# e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; the
# codes S.1111.111 are NaN; largest finite value 448, smallest normal 2^-6,
# subnormals k * 2^-9.

def e4m3_to_f32(codes: np.ndarray) -> np.ndarray:
    """float32 values of uint8 e4m3fn codes (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int32)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return (sign * mag).astype(np.float32)


_E4M3_POS = e4m3_to_f32(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)   # codes 0 .. 0x7E


def e4m3_bits(x: np.ndarray) -> np.ndarray:
    """uint8 e4m3fn codes of float32 values, rounded to nearest, ties to the
    even code; NaN and magnitudes above 448 give the NaN code."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 1, len(_E4M3_POS) - 1)
    lo = hi - 1
    dlo, dhi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a <= _E4M3_POS[0], 0, code).astype(np.uint8)
    code = np.where(np.isnan(a) | (a > 448.0), 0x7F, code).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << 7)


# Per-tensor descale of the FP8 inputs: the stored code times 2^-6 is the
# value, so standard-normal data (|x| < 7 at these sizes) stays below 448.
FP8_DESCALE = 2.0 ** -6


def make_fp8_inputs(shape, seed, sigma_qk=1.0, sigma_v=1.0, descale=FP8_DESCALE):
    """Seeded FP8 q, k, v of one [B,H,N,d] shape: the e4m3fn codes (uint8),
    the per-tensor descales, and the values they stand for (float32, exact:
    code value times a power of two), which is what the oracle sees.

    Recipe: one generator, draw order q, k, v, each standard normal times its
    spread, divided by the descale, clipped to +-448 and rounded to e4m3fn."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, sig in (("q", sigma_qk), ("k", sigma_qk), ("v", sigma_v)):
        x = rng.standard_normal(size=tuple(shape), dtype=np.float32)
        if sig != 1.0:
            x *= np.float32(sig)
        codes = e4m3_bits(np.clip(x / np.float32(descale), -448.0, 448.0))
        out[name + "8"] = codes
        out[name] = (e4m3_to_f32(codes) * np.float32(descale)).astype(np.float32)
        out["descale_" + name] = float(descale)
    return out
