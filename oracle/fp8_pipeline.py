"""Simulation of FP8 attention with and without incoherent processing.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages report that multiplying Q and K by a random-sign Hadamard matrix
before FP8 quantization lowers the attention error about 2.6-fold against plain
FP8, in an experiment where Q, K and V are standard normal with 0.1 % of the
entries made large to imitate outliers ([NL] "3. Lage precisie (FP8) met
reductie van kwantisatiefout"; [GN] "Niedrige FP8-Präzision und incoherent
processing"). This module simulates both schemes so that the expected error of
each, and their ratio, can be computed on the CPU.

Schemes (the plain per-tensor baseline is the pages' "FP8 without
transformations"):

* ``"hadamard"``: Q, K -> random-sign Hadamard, then per-``block_rows`` block
  scales (``oracle.fp8.hadamard_quantize``); V -> one per-tensor scale.
* ``"per_tensor"``: Q, K, V -> one per-tensor scale each, no transform.

Attention is then the float64 definition on the dequantized values. With
``p_quant`` the probabilities entering the P V product are also rounded to
E4M3 after multiplication by 2^8 (and divided by 2^8 again), with the row sum
taken from the unrounded probabilities, the reading used by the FP8 kernel.

Parity unpinned: the absolute error values of this simulation are not printed
by the pages; only the ratio between the two schemes is (2.6x), and that ratio
is what ``tests/test_oracle.py`` pins.
"""

from __future__ import annotations

import numpy as np

from .attention import allowed_mask
from .fp8 import (dequantize_blocks, e4m3_decode, e4m3_encode, hadamard_quantize,
                  quantize_per_tensor)

P_SHIFT = 256.0   # 2^8: keeps probabilities out of the E4M3 subnormal range


def rmse(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.sqrt(np.mean((a - b) ** 2)))


def dequantized_inputs(q, k, v, scheme: str, signs=None, block_rows: int = 64):
    """Quantize then dequantize Q, K, V under ``scheme``; returns float64 arrays."""
    if scheme == "hadamard":
        if signs is None:
            raise ValueError("hadamard scheme needs a sign vector")
        qc, qs = hadamard_quantize(q, signs, block_rows)
        kc, ks = hadamard_quantize(k, signs, block_rows)
        qh = dequantize_blocks(qc, qs, block_rows)
        kh = dequantize_blocks(kc, ks, block_rows)
    elif scheme == "per_tensor":
        qc, qs = quantize_per_tensor(q)
        kc, ks = quantize_per_tensor(k)
        qh = e4m3_decode(qc) * np.float64(qs)
        kh = e4m3_decode(kc) * np.float64(ks)
    else:
        raise ValueError(f"unknown scheme {scheme!r}")
    vc, vs = quantize_per_tensor(v)
    vh = e4m3_decode(vc) * np.float64(vs)
    return qh, kh, vh


def fp8_attention_sim(q, k, v, causal: bool, scale: float, scheme: str, signs=None,
                      block_rows: int = 64, p_quant: bool = True):
    """Simulated FP8 attention output (float64 O, LSE) under ``scheme``.

    When the Hadamard scheme is used the dequantized Q and K are in the
    rotated basis; Q K^T is the same as in the original basis up to
    quantization error, and V is never rotated, so O is directly comparable
    with exact attention on the original inputs.
    """
    qh, kh, vh = dequantized_inputs(q, k, v, scheme, signs, block_rows)
    b, h, s_q, d = qh.shape
    s_k = kh.shape[2]
    o = np.empty((b, h, s_q, vh.shape[3]))
    lse = np.empty((b, h, s_q))
    allowed = allowed_mask(s_q, s_k, causal)
    for bi in range(b):
        for hi in range(h):
            s = scale * (qh[bi, hi] @ kh[bi, hi].T)
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1)
            p = np.exp(s - m[:, None])
            l = p.sum(axis=1)
            if p_quant:
                pq = e4m3_decode(e4m3_encode((p * P_SHIFT).astype(np.float32))) / P_SHIFT
            else:
                pq = p
            o[bi, hi] = (pq @ vh[bi, hi]) / l[:, None]
            lse[bi, hi] = m + np.log(l)
    return o, lse
