"""Simulation of FP8 attention with and without incoherent processing.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages report that multiplying Q and K by a random-sign Hadamard matrix
before FP8 quantization lowers the attention error about 2.6-fold against plain
FP8, in an experiment where Q, K and V are standard normal with 0.1 % of the
entries made large to imitate outliers ([NL] "3. Lage precisie (FP8) met
reductie van kwantisatiefout"; [GN] "Niedrige FP8-Präzision und incoherent
processing"). This module simulates both schemes so that the expected error of
each, and their ratio, can be computed on the CPU.

Schemes (the plain per-tensor baseline is the pages' FP8 comparison with no
transform applied):

* ``"hadamard"``: Q, K -> random-sign Hadamard, then per-``block_rows`` block
  scales (``oracle.fp8.hadamard_quantize``); V -> one per-tensor scale.
* ``"per_tensor"``: Q, K, V -> one per-tensor scale each, no transform.

Attention is then the float64 definition on the dequantized values.

The pages do not say how the probabilities enter the FP8 P V product. Reading:
each p (relative to its row's maximum) is multiplied by 2^k, rounded to E4M3
and divided by 2^k again (``round_p``), and the row sum l is the sum of those
rounded values, so that O is the average of the V rows under the weights the
product actually uses and the LSE is the log of their sum. The factor keeps
small p out of the E4M3 subnormals. A kernel
that forms p against a running reference which trails the row's final maximum
by up to tau (log2) and scales by 2^k0 uses, relative to the final maximum,
factors between 2^k0 and 2^(k0 + tau); the FP8 kernel of this repository has
k0 = 7 and tau = 1.75. The simulation takes one factor 2^k for the whole row
against the row's final maximum (no tiling); evaluated at k = 7 and k = 8.75
it brackets that kernel's rounding. ``p_rounding_bound`` and
``p_rounding_lse_bound`` give the largest error the rounding of P can cause in
each output element and in each row's LSE for any k >= 7, whatever factor each
p was rounded with.

Parity unpinned: the absolute error values of this simulation are not printed
by the pages; only the ratio between the two schemes is (2.6x), and that ratio
is what ``tests/test_oracle.py`` pins, together with worked values of
``round_p`` and the bound.
"""

from __future__ import annotations

import numpy as np

from .attention import allowed_mask
from .fp8 import (dequantize_blocks, e4m3_decode, e4m3_encode, hadamard_quantize,
                  quantize_per_tensor)

P_EXP = 7.0        # default k of round_p: p * 2^7 keeps small p out of the E4M3 subnormals
P_EXP_RANGE = (7.0, 8.75)   # the factors a running reference trailing the maximum by <= 1.75 gives


def rmse(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.sqrt(np.mean((a - b) ** 2)))


def round_p(p, p_exp: float = P_EXP) -> np.ndarray:
    """E4M3(p * 2^p_exp) / 2^p_exp in float64: a probability as the P V product takes it.

    The product p * 2^p_exp is rounded once (nearest, ties to even, from its
    float64 value) and scaled back; no saturation is reached for p <= 1 and
    p_exp <= log2(448).
    """
    f = np.exp2(np.float64(p_exp))
    return e4m3_decode(e4m3_encode(np.asarray(p, dtype=np.float64) * f)) / f


def _p_and_rounding_bound(qh, kh, causal: bool, scale: float):
    """Per head: p relative to the row maximum, and b(p), the most ``round_p`` can move each p.

    For p * 2^k in the E4M3 normal range (>= 2^-6) rounding to nearest moves it
    by at most half a step, 2^-4 of its value (three mantissa bits); below that
    the step is 2^-9, so p moves by at most 2^-10 / 2^k <= 2^-17 for k >= 7:
    b(p) = 2^-4 p for p >= 2^-13, 2^-17 for 0 < p < 2^-13 and 0 for p = 0.
    Yields (bi, hi, p, b) for every head of the dequantized [B, H, S, D] inputs.
    """
    qh, kh = (np.asarray(x, dtype=np.float64) for x in (qh, kh))
    b, h, s_q, _ = qh.shape
    allowed = allowed_mask(s_q, kh.shape[2], causal)
    for bi in range(b):
        for hi in range(h):
            s = scale * (qh[bi, hi] @ kh[bi, hi].T)
            s = np.where(allowed, s, -np.inf)
            p = np.exp(s - s.max(axis=1)[:, None])
            bp = np.where(p >= 2.0 ** -13, p / 16.0, np.where(p > 0, 2.0 ** -17, 0.0))
            yield bi, hi, p, bp


def p_rounding_bound(qh, kh, vh, causal: bool, scale: float) -> np.ndarray:
    """Largest |O error| that rounding P with ``round_p`` can cause, per output element.

    With rounded weights p'_j = p_j + e_j (|e_j| <= b(p_j)) in both the sum and
    the normaliser, O'_i - O_i = sum_j e_ij (V_jd - O_id) / l'_i, and
    l'_i >= l_i - sum_j b(p_ij), so the error is at most
    (sum_j b(p_ij) |V_jd| + |O_id| sum_j b(p_ij)) / (l_i - sum_j b(p_ij)).
    Each p may be rounded with its own factor 2^k (k >= 7). qh, kh, vh are the
    dequantized [B, H, S, D] inputs.
    """
    vh = np.asarray(vh, dtype=np.float64)
    out = np.empty(tuple(np.shape(qh)[:3]) + (vh.shape[3],))
    for bi, hi, p, bp in _p_and_rounding_bound(qh, kh, causal, scale):
        l = p.sum(axis=1)
        o = (p @ vh[bi, hi]) / l[:, None]
        sb = bp.sum(axis=1)
        out[bi, hi] = (bp @ np.abs(vh[bi, hi]) + np.abs(o) * sb[:, None]) / (l - sb)[:, None]
    return out


def p_rounding_lse_bound(qh, kh, causal: bool, scale: float) -> np.ndarray:
    """Largest |LSE error| that rounding P with ``round_p`` can cause, per row ([B, H, S_q]).

    The LSE is m + ln l' with l' the sum of the rounded p, and
    |l' - l| <= sum_j b(p_j), so |ln l' - ln l| <= -ln(1 - sum_j b(p_j) / l).
    """
    out = np.empty(tuple(np.shape(qh)[:3]))
    for bi, hi, p, bp in _p_and_rounding_bound(qh, kh, causal, scale):
        out[bi, hi] = -np.log1p(-bp.sum(axis=1) / p.sum(axis=1))
    return out


def dequantized_inputs(q, k, v, scheme: str, signs=None, block_rows: int = 64, amax=None):
    """Quantize then dequantize Q, K, V under ``scheme``; returns float64 arrays.

    ``amax`` (optional) gives the per-tensor maxima {"q": a, "k": a, "v": a} of
    the whole tensors when q, k, v are only some of their heads; block scales
    depend on each head's own rows and need nothing more.
    """
    am = amax or {}
    if scheme == "hadamard":
        if signs is None:
            raise ValueError("hadamard scheme needs a sign vector")
        qc, qs = hadamard_quantize(q, signs, block_rows)
        kc, ks = hadamard_quantize(k, signs, block_rows)
        qh = dequantize_blocks(qc, qs, block_rows)
        kh = dequantize_blocks(kc, ks, block_rows)
    elif scheme == "per_tensor":
        qc, qs = quantize_per_tensor(q, am.get("q"))
        kc, ks = quantize_per_tensor(k, am.get("k"))
        qh = e4m3_decode(qc) * np.float64(qs)
        kh = e4m3_decode(kc) * np.float64(ks)
    else:
        raise ValueError(f"unknown scheme {scheme!r}")
    vc, vs = quantize_per_tensor(v, am.get("v"))
    vh = e4m3_decode(vc) * np.float64(vs)
    return qh, kh, vh


def fp8_attention_sim(q, k, v, causal: bool, scale: float, scheme: str, signs=None,
                      block_rows: int = 64, p_quant: bool = True, p_exp: float = P_EXP):
    """Simulated FP8 attention output (float64 O, LSE) under ``scheme``.

    When the Hadamard scheme is used the dequantized Q and K are in the
    rotated basis; Q K^T is the same as in the original basis up to
    quantization error, and V is never rotated, so O is directly comparable
    with exact attention on the original inputs. With ``p_quant`` the
    probabilities entering P V are ``round_p(p, p_exp)`` against the row's
    final maximum, and l and the LSE are their sum.
    """
    qh, kh, vh = dequantized_inputs(q, k, v, scheme, signs, block_rows)
    b, h, s_q, d = qh.shape
    o = np.empty((b, h, s_q, vh.shape[3]))
    lse = np.empty((b, h, s_q))
    rows = np.arange(s_q)
    for bi in range(b):
        for hi in range(h):
            o[bi, hi], lse[bi, hi] = fp8_attention_rows(qh[bi, hi], kh[bi, hi], vh[bi, hi], rows, causal,
                                                        scale, s_q, p_quant, p_exp)
    return o, lse


def fp8_attention_rows(qh, kh, vh, rows, causal: bool, scale: float, s_q: int, p_quant: bool = True,
                       p_exp: float = P_EXP):
    """Query rows ``rows`` of the simulated FP8 attention of one (b, h).

    qh [S_q, D], kh [S_k, D], vh [S_k, D] are the dequantized inputs of that
    head; returns (O rows float64, LSE rows). Same arithmetic as
    ``fp8_attention_sim``.
    """
    qh, kh, vh = (np.asarray(x, dtype=np.float64) for x in (qh, kh, vh))
    rows = np.asarray(rows)
    s = scale * (qh[rows] @ kh.T)
    s = np.where(allowed_mask(s_q, kh.shape[0], causal, rows), s, -np.inf)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    pq = round_p(p, p_exp) if p_quant else p
    lq = pq.sum(axis=1)
    return (pq @ vh) / lq[:, None], m + np.log(lq)
