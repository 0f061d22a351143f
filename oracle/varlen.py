"""Packed batches of sequences of different lengths, as the plain definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[GN] "Weitere Optimierungen und künftige Integration" names variable-length
sequences among the optimizations of the full paper and says nothing more.
The plainest reading: B independent sequences of different lengths stored back
to back without padding; each attends only to its own keys, exactly as the
dense definition (``oracle.attention``) treats one sequence on its own.

Layout (the packed convention):

* q, o  [total_q, H, D]; k, v  [total_k, H, D];
* sequence b owns rows cu_q[b] .. cu_q[b+1]-1 of q and cu_k[b] .. cu_k[b+1]-1
  of k and v (cu_* nondecreasing, starting at 0, ending at the totals);
* LSE  [H, total_q].

Per sequence and head, with S_q and S_k its lengths:

    S_ij  = scale * sum_d Q_id K_jd
    allowed(i, j) = (not causal) or j <= i + (S_k - S_q)
    O_i   = sum_j p_ij V_j / sum_j p_ij,   p_ij = exp(S_ij - max_j S_ij) on allowed j
    LSE_i = max_j S_ij + ln sum_j p_ij

Reading where the dense case rejects the input: with packing a caller cannot
avoid a query row that has no allowed key (an empty key sequence, or causal
rows above the diagonal when S_q > S_k), so such a row gets O = 0 and
LSE = -inf, the logarithm of an empty sum with nothing to average.
"""

from __future__ import annotations

import numpy as np


def attention_varlen(q, k, v, cu_q, cu_k, causal: bool, scale: float):
    """(O float64 [total_q, H, D], LSE float64 [H, total_q]) of a packed batch."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3 or k.shape != v.shape or q.shape[1:] != k.shape[1:]:
        raise ValueError("q must be [total_q, H, D] and k, v [total_k, H, D]")
    if cu_q.shape != cu_k.shape or cu_q.ndim != 1 or cu_q.size < 2:
        raise ValueError("cu_q and cu_k must hold B+1 offsets")
    for cu, total in ((cu_q, q.shape[0]), (cu_k, k.shape[0])):
        if cu[0] != 0 or cu[-1] != total or np.any(np.diff(cu) < 0):
            raise ValueError("offsets must start at 0, not decrease and end at the total")
    total_q, heads, _ = q.shape
    o = np.zeros((total_q, heads, v.shape[2]), dtype=np.float64)
    lse = np.full((heads, total_q), -np.inf, dtype=np.float64)
    for b in range(cu_q.size - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        s_q, s_k = q1 - q0, k1 - k0
        if s_q == 0 or s_k == 0:
            continue                                   # nothing to attend: O = 0, LSE = -inf
        i = np.arange(s_q)[:, None]
        j = np.arange(s_k)[None, :]
        allowed = np.ones((s_q, s_k), dtype=bool) if not causal else (j <= i + (s_k - s_q))
        has = allowed.any(axis=1)
        for h in range(heads):
            s = scale * (q[q0:q1, h] @ k[k0:k1, h].T)  # [S_q, S_k], explicit scores
            s = np.where(allowed, s, -np.inf)
            m = np.where(has, s.max(axis=1), 0.0)
            p = np.exp(s - m[:, None])                 # 0 on keys that are not allowed
            l = p.sum(axis=1)
            rows = np.nonzero(has)[0]
            o[q0 + rows, h] = (p[rows] @ v[k0:k1, h]) / l[rows, None]
            lse[h, q0 + rows] = m[rows] + np.log(l[rows])
    return o, lse
