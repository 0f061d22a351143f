"""Gradients of exact attention, written as their plain definition (float64, NumPy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages motivate the method by training (long-context models) and keep the
row logsumexp so that the backward pass can recompute the attention matrix
instead of storing it ([GN] "Rückblick auf den FlashAttention-Ansatz"). They
give no formulas for it; the gradients below are those of the function
``oracle.attention`` computes, by the chain rule, with the explicit score
matrix (S_q x S_k):

    S   = scale * Q K^T,  P = softmax over the allowed keys of each row
    O   = P V
    dV  = P^T dO
    dP  = dO V^T
    D_i = sum_d dO_id O_id  (= sum_j P_ij dP_ij)
    dS  = P * (dP - D)       (elementwise; 0 where a key is not allowed)
    dQ  = scale * dS K
    dK  = scale * dS^T Q

Causal alignment as in ``oracle.attention`` (key j allowed for query i iff
j <= i + S_k - S_q).
"""

from __future__ import annotations

import numpy as np

from .attention import allowed_mask, _check


def attention_backward(q, k, v, do, causal: bool, scale: float):
    """(dQ, dK, dV) float64 for [B, H, S, D] inputs and output gradient dO."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    b, h, s_q, s_k, d = _check(q, k, v, causal)
    if do.shape != q.shape[:3] + (v.shape[3],):
        raise ValueError("dO must match the output shape")
    allowed = allowed_mask(s_q, s_k, causal)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for bi in range(b):
        for hi in range(h):
            s = scale * (q[bi, hi] @ k[bi, hi].T)
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            p /= p.sum(axis=1, keepdims=True)
            o = p @ v[bi, hi]
            dv[bi, hi] = p.T @ do[bi, hi]
            dp = do[bi, hi] @ v[bi, hi].T
            dd = (do[bi, hi] * o).sum(axis=1, keepdims=True)
            ds = p * (dp - dd)
            dq[bi, hi] = scale * (ds @ k[bi, hi])
            dk[bi, hi] = scale * (ds.T @ q[bi, hi])
    return dq, dk, dv
