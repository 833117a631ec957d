"""Plain fp64 CPU oracle for exact softmax attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only the tests, the smoke check and the CPU-baseline leg of
the benchmark use it.  It shares no code with the HIP kernels and imports
nothing from the product package.

What it computes is the plain, materialised definition, with no tiling, no
online softmax and no recompute; the tiled method reaches the same numbers up
to rounding order (page "flash-attention-backpropagation" (aiqz.cc),
sections 前向台账 and 反向总览; page "flash-attention-v2-sram-tiling"
(aiqz.cc), section 常见误区).

Per attention head, with Q, K, V, dO of shape (N, d), all fp64:

  S    = scale * Q K^T, with S_ij = -inf for j > i when causal
         (page "flash-attention-backpropagation", section 显存困境, the S_ij
         equation; causal masking as upper-triangle-above-diagonal in the
         PyTorch module of page "blog.xiaohack.org/tag/flops", 知识点13)
  m_i  = max_j S_ij,  l_i = sum_j exp(S_ij - m_i)            (前向台账)
  P    = exp(S - m) / l,  LSE_i = m_i + ln l_i               (数值稳定)
  O    = P V                        ("flash-attention-v2-sram-tiling", §1)
  D_i  = sum_c dO_ic O_ic                                    (Softmax梯度)
  dP   = dO V^T,  dS = P * (dP - D 1^T)                      (Softmax梯度)
  dV   = P^T dO,  dQ = scale dS K,  dK = scale dS^T Q        (反向总览)

The loss convention behind the gradients is L = sum_ic dO_ic O_ic, so that
dL/dO = dO.

Large N: ``head_panel`` walks full rows of S in panels of ``panel_rows`` rows.
Softmax is row-local, so each panel is the same definition; dK and dV are
sums over rows and are accumulated panel by panel.  Nothing else is blocked.

The scale: the pages put 1/sqrt(d) on S and the same factor on dQ and dK;
this oracle takes the factor as an argument (``scale``) and applies it in
exactly those three places.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "scores",
    "softmax_rows",
    "head_forward",
    "head_backward",
    "head_panel",
    "forward",
    "backward",
    "forward_backward",
    "scores_rect",
    "head_forward_rect",
    "forward_rect",
]


def scores(q: np.ndarray, k: np.ndarray, scale: float, causal: bool,
           row0: int = 0) -> np.ndarray:
    """S = scale * Q K^T for query rows row0.. of one head; -inf where j > i.

    ``q`` holds query rows row0 .. row0+len(q)-1 of the head; ``k`` holds all
    N key rows.  The causal mask keeps key j for query i iff j <= i.
    """
    s = scale * (q @ k.T)
    if causal:
        rows = np.arange(row0, row0 + q.shape[0])[:, None]
        cols = np.arange(k.shape[0])[None, :]
        s = np.where(cols > rows, -np.inf, s)
    return s


def softmax_rows(s: np.ndarray):
    """Row softmax with the row maximum subtracted.

    Returns (P, m, lse): P_ij = exp(S_ij - m_i) / l_i, m_i = max_j S_ij,
    lse_i = m_i + ln l_i with l_i = sum_j exp(S_ij - m_i).  Masked entries
    (-inf) give exactly 0 in P.  Every row must keep at least one key.
    """
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    p = e / l[:, None]
    lse = m + np.log(l)
    return p, m, lse


def head_forward(q, k, v, scale, causal):
    """O and LSE of one head, materialising S and P (returned too)."""
    s = scores(q, k, scale, causal)
    p, _, lse = softmax_rows(s)
    o = p @ v
    return o, lse, s, p


def head_backward(q, k, v, do, scale, causal, want_intermediates=False):
    """dQ, dK, dV of one head from the materialised P (no recompute trick).

    The forward is evaluated here in fp64 from q, k, v, so D uses the
    oracle's own O.
    """
    o, lse, s, p = head_forward(q, k, v, scale, causal)
    d_row = (do * o).sum(axis=1)
    dp = do @ v.T
    ds = p * (dp - d_row[:, None])
    dv = p.T @ do
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    if want_intermediates:
        return dq, dk, dv, dict(o=o, lse=lse, s=s, p=p, D=d_row, dp=dp, ds=ds)
    return dq, dk, dv


def head_panel(q, k, v, do, scale, causal, panel_rows=2048, rows=None):
    """Full forward and backward of one head, full rows of S in panels.

    Returns dict(o, lse, dq, dk, dv) in fp64.  Each panel materialises
    S[r0:r1, :] and P[r0:r1, :] in full.  If ``rows`` is given, only the query
    rows listed are returned for o, lse and dq (dk, dv still need every row,
    so every panel is still evaluated).
    """
    n, dh = q.shape
    o = np.empty((n, dh))
    lse = np.empty(n)
    dq = np.empty((n, dh))
    dk = np.zeros((n, dh))
    dv = np.zeros((n, dh))
    for r0 in range(0, n, panel_rows):
        r1 = min(n, r0 + panel_rows)
        s = scores(q[r0:r1], k, scale, causal, row0=r0)
        p, _, lse_p = softmax_rows(s)
        del s
        o_p = p @ v
        d_row = (do[r0:r1] * o_p).sum(axis=1)
        dp = do[r0:r1] @ v.T
        ds = p * (dp - d_row[:, None])
        del dp
        dv += p.T @ do[r0:r1]
        del p
        dq[r0:r1] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r0:r1])
        o[r0:r1] = o_p
        lse[r0:r1] = lse_p
    out = dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)
    if rows is not None:
        rows = np.asarray(rows)
        out["o"], out["lse"], out["dq"] = o[rows], lse[rows], dq[rows]
    return out


def _heads(x):
    b, h = x.shape[:2]
    for bi in range(b):
        for hi in range(h):
            yield bi, hi


def forward(q, k, v, scale, causal):
    """O [B,H,N,d] and LSE [B,H,N] (natural log, scaled-score units), fp64."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    b, h, n, dh = q.shape
    o = np.empty((b, h, n, dh))
    lse = np.empty((b, h, n))
    for bi, hi in _heads(q):
        o[bi, hi], lse[bi, hi], _, _ = head_forward(q[bi, hi], k[bi, hi], v[bi, hi], scale, causal)
    return o, lse


def backward(q, k, v, do, scale, causal):
    """dQ, dK, dV [B,H,N,d] in fp64."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    dq = np.empty(q.shape)
    dk = np.empty(q.shape)
    dv = np.empty(q.shape)
    for bi, hi in _heads(q):
        dq[bi, hi], dk[bi, hi], dv[bi, hi] = head_backward(
            q[bi, hi], k[bi, hi], v[bi, hi], do[bi, hi], scale, causal)
    return dq, dk, dv


def forward_backward(q, k, v, do, scale, causal, heads=None, panel_rows=2048):
    """O, LSE, dQ, dK, dV for the listed (b, h) heads (all heads if None).

    Returns a dict keyed by (b, h) of dict(o, lse, dq, dk, dv), fp64.  Uses
    full-row panels so that long sequences fit in host memory.
    """
    q, k, v, do = (np.asarray(t) for t in (q, k, v, do))
    if heads is None:
        heads = list(_heads(q))
    out = {}
    for bi, hi in heads:
        f64 = lambda t: np.asarray(t[bi, hi], dtype=np.float64)
        out[(bi, hi)] = head_panel(f64(q), f64(k), f64(v), f64(do), scale, causal,
                                   panel_rows=panel_rows)
    return out


# ---- queries against a longer key sequence (decode) --------------------------
#
# The split-key-range forward serves Nq query rows against Nk >= Nq key rows
# of the same head, the shape of decoding with a key/value cache (page
# "flash-attention-v2-sram-tiling", the long-document inference scenario; the
# decoding variant named on page "data.6616ai.com flash-attention").  The pages
# do not define the causal mask for Nq != Nk; the reading taken here is that
# the Nq queries are the last Nq positions of the sequence, so query i sits at
# position Nk - Nq + i and keeps key j iff j <= i + Nk - Nq.  With Nq == Nk
# this is the square mask above.


def scores_rect(q: np.ndarray, k: np.ndarray, scale: float, causal: bool) -> np.ndarray:
    """S = scale * Q K^T for Nq query rows against Nk key rows of one head.

    With ``causal``, S_ij = -inf for j > i + Nk - Nq (the queries are the
    last Nq positions).  Requires Nq <= Nk when causal.
    """
    nq, nk = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    if causal:
        if nq > nk:
            raise ValueError("causal attention needs Nq <= Nk")
        rows = np.arange(nq)[:, None] + (nk - nq)
        cols = np.arange(nk)[None, :]
        s = np.where(cols > rows, -np.inf, s)
    return s


def head_forward_rect(q, k, v, scale, causal):
    """O (Nq, d) and LSE (Nq,) of one head for Nq queries against Nk keys."""
    p, _, lse = softmax_rows(scores_rect(q, k, scale, causal))
    return p @ v, lse


def forward_rect(q, k, v, scale, causal, heads=None):
    """O [B,H,Nq,d] and LSE [B,H,Nq] for q [B,H,Nq,d] against k, v [B,H,Nk,d].

    With ``heads`` (a list of (b, h)), returns a dict keyed by (b, h) of
    dict(o, lse) for those heads only.
    """
    q, k, v = (np.asarray(t) for t in (q, k, v))
    f64 = lambda t, bi, hi: np.asarray(t[bi, hi], dtype=np.float64)
    if heads is not None:
        out = {}
        for bi, hi in heads:
            o, lse = head_forward_rect(f64(q, bi, hi), f64(k, bi, hi), f64(v, bi, hi), scale, causal)
            out[(bi, hi)] = dict(o=o, lse=lse)
        return out
    b, h, nq, dh = q.shape
    o = np.empty((b, h, nq, dh))
    lse = np.empty((b, h, nq))
    for bi, hi in _heads(q):
        o[bi, hi], lse[bi, hi] = head_forward_rect(f64(q, bi, hi), f64(k, bi, hi), f64(v, bi, hi),
                                                   scale, causal)
    return o, lse
