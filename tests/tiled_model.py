"""Tests-only fp64 model of the tiled method (online softmax forward,
recompute backward), used to pin the oracle by blocking invariance.

It follows the pages' block algorithm step by step, in fp64, on one head:

forward, per query block i and key block j in increasing j
  (page "flash-attention-v2-sram-tiling" (aiqz.cc), section 4 for the loop
  order and section 5 for the update; the l update takes the full block sum,
  as in the derivation of page "blog.xiaohack.org/tag/flops", 知识点13 §4):
    m_new = max(m, rowmax(S_ij))
    l     = l * exp(m - m_new) + rowsum(exp(S_ij - m_new))
    acc   = acc * exp(m - m_new) + exp(S_ij - m_new) V_j
  then O_i = acc / l and LSE_i = m + ln l (normalisation deferred to the end).

backward, key/value block outer, query block inner
  (page "flash-attention-backpropagation" (aiqz.cc), sections 数值稳定,
  Softmax梯度 and QKV梯度):
    D_i   = rowsum(dO_i o O_i)                     (full rows, before the loop)
    P^_ij = exp(S_ij - LSE_i)
    dV_j += P^_ij^T dO_i
    dS_ij = P^_ij o (dO_i V_j^T - D_i)
    dQ_i += scale dS_ij K_j ;  dK_j += scale dS_ij^T Q_i

Block sizes need not divide N.  Nothing here is shared with the oracle.
"""
from __future__ import annotations

import numpy as np


def _mask(s, r0, c0, causal):
    if not causal:
        return s
    rows = np.arange(r0, r0 + s.shape[0])[:, None]
    cols = np.arange(c0, c0 + s.shape[1])[None, :]
    return np.where(cols > rows, -np.inf, s)


def tiled_forward(q, k, v, scale, causal, br, bc):
    n, d = q.shape
    o = np.zeros((n, d))
    lse = np.zeros(n)
    for r0 in range(0, n, br):
        r1 = min(n, r0 + br)
        m = np.full(r1 - r0, -np.inf)
        l = np.zeros(r1 - r0)
        acc = np.zeros((r1 - r0, d))
        for c0 in range(0, n, bc):
            c1 = min(n, c0 + bc)
            s = _mask(scale * (q[r0:r1] @ k[c0:c1].T), r0, c0, causal)
            blk_max = s.max(axis=1)
            m_new = np.maximum(m, blk_max)
            # rows whose keys in this block are all masked and that have seen
            # nothing yet keep m = -inf; give them a finite shift of 0
            shift = np.where(np.isfinite(m_new), m_new, 0.0)
            e = np.exp(s - shift[:, None])
            corr = np.exp(m - shift)
            l = l * corr + e.sum(axis=1)
            acc = acc * corr[:, None] + e @ v[c0:c1]
            m = m_new
        o[r0:r1] = acc / l[:, None]
        lse[r0:r1] = m + np.log(l)
    return o, lse


def tiled_backward(q, k, v, o, do, lse, scale, causal, br, bc):
    n, d = q.shape
    dq = np.zeros((n, d))
    dk = np.zeros((n, d))
    dv = np.zeros((n, d))
    drow = (do * o).sum(axis=1)
    for c0 in range(0, n, bc):
        c1 = min(n, c0 + bc)
        for r0 in range(0, n, br):
            r1 = min(n, r0 + br)
            s = _mask(scale * (q[r0:r1] @ k[c0:c1].T), r0, c0, causal)
            p = np.exp(s - lse[r0:r1, None])
            dv[c0:c1] += p.T @ do[r0:r1]
            dp = do[r0:r1] @ v[c0:c1].T
            ds = p * (dp - drow[r0:r1, None])
            dq[r0:r1] += scale * (ds @ k[c0:c1])
            dk[c0:c1] += scale * (ds.T @ q[r0:r1])
    return dq, dk, dv
