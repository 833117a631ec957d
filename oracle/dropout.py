"""Plain fp64 CPU oracle for attention with dropout on the probabilities.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only the tests, the smoke check and the CPU-baseline leg of
the benchmark use it.  It shares no code with the HIP kernels and imports
nothing from the product package.

Page "blog.xiaohack.org/tag/flops", section 7 (算子融合优化), lists dropout as
part of the fused softmax step, and says no more.  The reading taken here is
ordinary inverted dropout of the normalised attention probabilities, drawn
from a counter-based generator so that the backward can regenerate the same
mask instead of storing it:

  P    = softmax(S) as in the plain oracle; LSE unchanged
  Z_ij = 1 (kept) or 0 (dropped),  s_keep = 256 / (256 - t)
  Pd   = s_keep * (P o Z)
  O    = Pd V
  D_i  = sum_c dO_ic O_ic
  dPd  = dO V^T,  dP = s_keep * (dPd o Z)
  dS   = P o (dP - D 1^T)
  dV   = Pd^T dO,  dQ = scale dS K,  dK = scale dS^T Q

D is still the row sum of dO o O: sum_j P_ij dP_ij = sum_j Pd_ij dPd_ij =
dO_i . O_i, so the softmax-gradient step of page
"flash-attention-backpropagation" (aiqz.cc), section Softmax梯度, holds as is.

The generator is Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC 2011): ten rounds on a 4-word
counter under a 2-word key, each round two widening multiplies whose high
halves are xored with the other two words and the round key.  The key
advances by the Weyl constants between rounds.  Drop decision:

  4x4 block (I, J) = queries 4I..4I+3, keys 4J..4J+3 of head bh
  (x0, x1, x2, x3) = Philox4x32-10(counter (J, I, bh, offset),
                                   key (seed mod 2^32, seed div 2^32))
  Z[4I + a, 4J + b] = 1  iff  byte b of x_a (bits 8b .. 8b+7) >= t

So a score is dropped with probability t / 256, with t an integer in
0 .. 255.  bh = b * H + h is the head's index in [B, H] order.
"""
from __future__ import annotations

import numpy as np

from . import ref

__all__ = [
    "PHILOX",
    "philox_scalar",
    "philox4x32_10",
    "keep_mask",
    "keep_scale",
    "head_forward_dropout",
    "head_backward_dropout",
    "head_panel_dropout",
    "forward_backward_dropout",
]

# Published constants of the two Philox widths: round multipliers M0, M1 and
# key increments W0, W1 (the golden ratio and sqrt(3) - 1 in fixed point).
PHILOX = {
    32: dict(M0=0xD2511F53, M1=0xCD9E8D57, W0=0x9E3779B9, W1=0xBB67AE85),
    64: dict(M0=0xD2E7470EE14C6C93, M1=0xCA5A826395121157,
             W0=0x9E3779B97F4A7C15, W1=0xBB67AE8584CAA73B),
}


def philox_scalar(ctr, key, width=32, rounds=10):
    """Philox4xW-R on Python integers: one counter (4 words), one key (2 words).

    Round r (r = 0 .. R-1) uses the key advanced r times by (W0, W1):
      (hi0, lo0) = M0 * x0,  (hi1, lo1) = M1 * x2    (2W-bit products)
      x <- (hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0)
    """
    c = PHILOX[width]
    mask = (1 << width) - 1
    x0, x1, x2, x3 = (int(v) & mask for v in ctr)
    k0, k1 = (int(v) & mask for v in key)
    for _ in range(rounds):
        p0 = c["M0"] * x0
        p1 = c["M1"] * x2
        x0, x1, x2, x3 = ((p1 >> width) ^ x1 ^ k0, p1 & mask, (p0 >> width) ^ x3 ^ k1, p0 & mask)
        k0 = (k0 + c["W0"]) & mask
        k1 = (k1 + c["W1"]) & mask
    return x0, x1, x2, x3


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 over arrays of counters (broadcast), numpy uint64 holding
    32-bit words; the same rounds as ``philox_scalar(width=32)``."""
    c = PHILOX[32]
    m32 = np.uint64(0xFFFFFFFF)
    sh = np.uint64(32)
    x0, x1, x2, x3 = np.broadcast_arrays(*(np.asarray(v, dtype=np.uint64) & m32 for v in (c0, c1, c2, c3)))
    x0, x1, x2, x3 = (np.array(v) for v in (x0, x1, x2, x3))
    k0, k1 = int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF
    M0, M1 = np.uint64(c["M0"]), np.uint64(c["M1"])
    for _ in range(10):
        p0 = M0 * x0          # < 2^64: exact in uint64
        p1 = M1 * x2
        n0 = (p1 >> sh) ^ x1 ^ np.uint64(k0)
        n2 = (p0 >> sh) ^ x3 ^ np.uint64(k1)
        x0, x1, x2, x3 = n0, p1 & m32, n2, p0 & m32
        k0 = (k0 + c["W0"]) & 0xFFFFFFFF
        k1 = (k1 + c["W1"]) & 0xFFFFFFFF
    return x0, x1, x2, x3


def keep_scale(t: int) -> float:
    """Factor on kept probabilities when t/256 of them are dropped."""
    return 256.0 / (256 - int(t))


def keep_mask(bh: int, seed: int, offset: int, t: int, nq: int, nk: int,
              row0: int = 0, rows: int | None = None) -> np.ndarray:
    """Z for query rows row0 .. row0+rows-1 (all nq if rows is None) and keys
    0 .. nk-1 of head bh, as a bool array (True = kept)."""
    if rows is None:
        rows = nq - row0
    r1 = row0 + rows
    i_blk = np.arange(row0 // 4, (r1 + 3) // 4, dtype=np.uint64)
    j_blk = np.arange(0, (nk + 3) // 4, dtype=np.uint64)
    xs = philox4x32_10(j_blk[None, :], i_blk[:, None], bh, offset,
                       seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    nI, nJ = len(i_blk), len(j_blk)
    z = np.empty((nI, 4, nJ, 4), dtype=bool)
    for a in range(4):
        for b in range(4):
            z[:, a, :, b] = ((xs[a] >> np.uint64(8 * b)) & np.uint64(0xFF)) >= np.uint64(t)
    z = z.reshape(4 * nI, 4 * nJ)
    lo = row0 - 4 * (row0 // 4)
    return z[lo:lo + rows, :nk]


def head_forward_dropout(q, k, v, scale, causal, keep, t):
    """O and LSE of one head with the keep mask applied; returns (o, lse, p, pd)."""
    s = ref.scores(q, k, scale, causal)
    p, _, lse = ref.softmax_rows(s)
    pd = keep_scale(t) * np.where(keep, p, 0.0)
    return pd @ v, lse, p, pd


def head_backward_dropout(q, k, v, do, scale, causal, keep, t, want_intermediates=False):
    """dQ, dK, dV of one head with the keep mask, from the materialised P."""
    o, lse, p, pd = head_forward_dropout(q, k, v, scale, causal, keep, t)
    d_row = (do * o).sum(axis=1)
    dpd = do @ v.T
    dp = keep_scale(t) * np.where(keep, dpd, 0.0)
    ds = p * (dp - d_row[:, None])
    dv = pd.T @ do
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    if want_intermediates:
        return dq, dk, dv, dict(o=o, lse=lse, p=p, pd=pd, D=d_row, dp=dp, ds=ds)
    return dq, dk, dv


def head_panel_dropout(q, k, v, do, scale, causal, bh, seed, offset, t, panel_rows=2048):
    """Forward and backward of one head with dropout, full rows of S (and of
    the mask) in panels of rows, as ``ref.head_panel``.  Returns dict(o, lse,
    dq, dk, dv) in fp64."""
    n, dh = q.shape
    o = np.empty((n, dh))
    lse = np.empty(n)
    dq = np.empty((n, dh))
    dk = np.zeros((n, dh))
    dv = np.zeros((n, dh))
    sk = keep_scale(t)
    for r0 in range(0, n, panel_rows):
        r1 = min(n, r0 + panel_rows)
        keep = keep_mask(bh, seed, offset, t, n, n, row0=r0, rows=r1 - r0)
        s = ref.scores(q[r0:r1], k, scale, causal, row0=r0)
        p, _, lse_p = ref.softmax_rows(s)
        del s
        pd = sk * np.where(keep, p, 0.0)
        o_p = pd @ v
        d_row = (do[r0:r1] * o_p).sum(axis=1)
        dp = sk * np.where(keep, do[r0:r1] @ v.T, 0.0)
        del keep
        ds = p * (dp - d_row[:, None])
        del dp, p
        dv += pd.T @ do[r0:r1]
        del pd
        dq[r0:r1] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r0:r1])
        o[r0:r1] = o_p
        lse[r0:r1] = lse_p
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)


def forward_backward_dropout(q, k, v, do, scale, causal, seed, offset, t, heads=None, panel_rows=2048):
    """O, LSE, dQ, dK, dV with dropout for the listed (b, h) heads (all if
    None), keyed by (b, h), fp64."""
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    nb, nh = q.shape[:2]
    if heads is None:
        heads = [(bi, hi) for bi in range(nb) for hi in range(nh)]
    out = {}
    for bi, hi in heads:
        f64 = lambda x: np.asarray(x[bi, hi], dtype=np.float64)
        out[(bi, hi)] = head_panel_dropout(f64(q), f64(k), f64(v), f64(do), scale, causal,
                                           bi * nh + hi, seed, offset, t, panel_rows=panel_rows)
    return out
