"""Exact attention, written as its plain definition (float64, NumPy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The computed function is softmax(scale * Q K^T [+ causal mask]) V, the
self-attention the pages set out to speed up ([NL] "Het probleem van het
aandachtsmechanisme"; [GN] "Ziele und Leistung von FlashAttention-3"). The
pages state that tiling plus softmax rescaling reaches the same output with no
approximation ([GN] "Rückblick auf den FlashAttention-Ansatz"), so the oracle
is the definition itself, with the full score matrix formed explicitly:

    S_ij   = scale * sum_d Q_id K_jd
    m_i    = max over allowed j of S_ij
    p_ij   = exp(S_ij - m_i)      (0 where j is not allowed)
    l_i    = sum_j p_ij
    O_i    = (sum_j p_ij V_j) / l_i
    LSE_i  = m_i + ln(l_i)        (natural-log logsumexp of the scaled scores)

Readings where the pages are silent:

* causal mask: key j is allowed for query i iff j <= i + (S_k - S_q)
  (aligned at the bottom-right diagonal; for S_q == S_k this is j <= i);
* a query row with no allowed key is rejected (ValueError) rather than given
  an invented value.

``attention_tiled`` and ``attention_partial``/``merge_partials`` restate the
block-wise method (online softmax over key tiles; split of the key range with a
logsumexp merge) in float64. They exist to pin the tiling arithmetic itself
against the definition (the exactness claim of [GN] "Rückblick auf den
FlashAttention-Ansatz"), not to check the GPU.
"""

from __future__ import annotations

import numpy as np

_ROW_CHUNK = 1024  # rows of the score matrix formed at a time (memory bound only)


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def allowed_mask(s_q: int, s_k: int, causal: bool, rows=None) -> np.ndarray:
    """Boolean [len(rows), S_k] mask: True where key j may be attended by query i."""
    if rows is None:
        rows = np.arange(s_q)
    rows = np.asarray(rows)
    if not causal:
        return np.ones((rows.shape[0], s_k), dtype=bool)
    j = np.arange(s_k)[None, :]
    return j <= (rows[:, None] + (s_k - s_q))


def _check(q, k, v, causal):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    b, h, s_q, d = q.shape
    if k.shape[:2] != (b, h) or v.shape[:2] != (b, h) or k.shape[3] != d:
        raise ValueError("shape mismatch between q, k, v")
    if k.shape[2] != v.shape[2]:
        raise ValueError("k and v must have the same sequence length")
    s_k = k.shape[2]
    if s_q < 1 or s_k < 1:
        raise ValueError("empty sequence")
    if causal and s_q > s_k:
        raise ValueError("causal with S_q > S_k leaves query rows with no allowed key")
    return b, h, s_q, s_k, d


def _rows_exact(qh, kh, vh, rows, s_q, causal, scale):
    """Definition applied to the query rows ``rows`` of one (b, h)."""
    s = scale * (qh[rows] @ kh.T)                      # [r, S_k], explicit scores
    allowed = allowed_mask(s_q, kh.shape[0], causal, rows)
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1)
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row has no allowed key")
    p = np.exp(s - m[:, None])                         # exp(-inf) = 0 for masked keys
    l = p.sum(axis=1)
    o = (p @ vh) / l[:, None]
    lse = m + np.log(l)
    return o, lse


def attention(q, k, v, causal: bool, scale: float):
    """Exact attention for [B, H, S, D] inputs; returns (O float64, LSE float64)."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    b, h, s_q, s_k, d = _check(q, k, v, causal)
    o = np.empty((b, h, s_q, v.shape[3]), dtype=np.float64)
    lse = np.empty((b, h, s_q), dtype=np.float64)
    for bi in range(b):
        for hi in range(h):
            for r0 in range(0, s_q, _ROW_CHUNK):
                rows = np.arange(r0, min(s_q, r0 + _ROW_CHUNK))
                o[bi, hi, rows], lse[bi, hi, rows] = _rows_exact(
                    q[bi, hi], k[bi, hi], v[bi, hi], rows, s_q, causal, scale)
    return o, lse


def attention_rows(qh, kh, vh, rows, causal: bool, scale: float, s_q: int | None = None):
    """The definition for selected query rows of a single head.

    ``qh`` is [S_q, D] (or only the selected rows when ``s_q`` is given, in which
    case ``rows`` are their absolute indices), ``kh``/``vh`` are [S_k, D].
    Used for sampled checks at sizes where the full oracle would take too long.
    """
    qh, kh, vh = _as64(qh), _as64(kh), _as64(vh)
    rows = np.asarray(rows)
    if s_q is None:
        s_q = qh.shape[0]
        qsel = qh[rows]
    else:
        qsel = qh
    if causal and s_q > kh.shape[0]:
        raise ValueError("causal with S_q > S_k")
    s = scale * (qsel @ kh.T)
    allowed = allowed_mask(s_q, kh.shape[0], causal, rows)
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    o = (p @ vh) / l[:, None]
    return o, m + np.log(l)


def attention_tiled(q, k, v, causal: bool, scale: float, bm: int, bn: int):
    """Block-wise attention with online softmax rescaling, float64.

    Query rows are taken bm at a time and keys bn at a time. For each key tile
    the running row maximum m, running sum l and unnormalised output acc are
    updated:  m' = max(m, rowmax(S_tile));  alpha = exp(m - m');
    l' = alpha*l + rowsum(exp(S_tile - m'));  acc' = alpha*acc + exp(S_tile - m') V_tile.
    At the end O = acc / l and LSE = m + ln(l).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    b, h, s_q, s_k, d = _check(q, k, v, causal)
    o = np.empty((b, h, s_q, v.shape[3]))
    lse = np.empty((b, h, s_q))
    for bi in range(b):
        for hi in range(h):
            for r0 in range(0, s_q, bm):
                rows = np.arange(r0, min(s_q, r0 + bm))
                qb = q[bi, hi, rows]
                m = np.full(rows.shape[0], -np.inf)
                l = np.zeros(rows.shape[0])
                acc = np.zeros((rows.shape[0], v.shape[3]))
                for c0 in range(0, s_k, bn):
                    cols = np.arange(c0, min(s_k, c0 + bn))
                    s = scale * (qb @ k[bi, hi, cols].T)
                    allowed = allowed_mask(s_q, s_k, causal, rows)[:, cols]
                    s = np.where(allowed, s, -np.inf)
                    m_new = np.maximum(m, s.max(axis=1))
                    # rows whose keys so far are all masked keep m = -inf; use 0 as reference
                    ref = np.where(np.isfinite(m_new), m_new, 0.0)
                    alpha = np.exp(np.where(np.isfinite(m), m, -np.inf) - ref)
                    p = np.exp(s - ref[:, None])
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ v[bi, hi, cols]
                    m = m_new
                if not np.all(np.isfinite(m)):
                    raise ValueError("a query row has no allowed key")
                o[bi, hi, rows] = acc / l[:, None]
                lse[bi, hi, rows] = m + np.log(l)
    return o, lse


def attention_partial(q, k, v, causal: bool, scale: float, key_lo: int, key_hi: int):
    """Attention restricted to keys [key_lo, key_hi): normalised partial output and LSE.

    Rows with no allowed key in the range get O = 0 and LSE = -inf, so they carry
    zero weight in ``merge_partials``.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    b, h, s_q, s_k, d = _check(q, k, v, causal)
    o = np.zeros((b, h, s_q, v.shape[3]))
    lse = np.full((b, h, s_q), -np.inf)
    cols = np.arange(key_lo, key_hi)
    if cols.size == 0:
        return o, lse
    allowed = allowed_mask(s_q, s_k, causal)[:, cols]
    for bi in range(b):
        for hi in range(h):
            s = scale * (q[bi, hi] @ k[bi, hi, cols].T)
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1)
            has = np.isfinite(m)
            ref = np.where(has, m, 0.0)
            p = np.exp(s - ref[:, None])
            l = p.sum(axis=1)
            l_safe = np.where(has, l, 1.0)
            o[bi, hi] = np.where(has[:, None], (p @ v[bi, hi, cols]) / l_safe[:, None], 0.0)
            lse[bi, hi] = np.where(has, m + np.log(l_safe), -np.inf)
    return o, lse


def merge_partials(parts):
    """Combine [(O_s, LSE_s), ...] over disjoint key ranges into (O, LSE).

    LSE = ln sum_s exp(LSE_s);  O = sum_s exp(LSE_s - LSE) O_s.
    """
    lses = np.stack([_as64(p[1]) for p in parts])        # [n, ...]
    outs = np.stack([_as64(p[0]) for p in parts])        # [n, ..., D]
    mx = lses.max(axis=0)
    ref = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(lses - ref)                                # exp(-inf) = 0
    tot = w.sum(axis=0)
    lse = ref + np.log(tot)
    o = (w[..., None] * outs).sum(axis=0) / tot[..., None]
    return o, lse
