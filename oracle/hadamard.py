"""Random-sign Hadamard transform ("incoherent processing").

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Before FP8 quantization, queries and keys are multiplied by a random orthogonal
matrix so that outliers are spread over all coordinates; because the matrix is
orthogonal, Q K^T is unchanged ([NL] "3. Lage precisie (FP8) met reductie van
kwantisatiefout"). The matrix used is a Hadamard matrix with random signs,
applied per head in O(d log d) ([GN] "Niedrige FP8-Präzision und incoherent
processing").

Reading (the pages give no normalisation, ordering or sign placement):
x' = H_D diag(s) x / sqrt(D), with H_D the Sylvester Hadamard matrix in natural
order (entries +-1, H_2n = [[H_n, H_n], [H_n, -H_n]]), one sign vector s in
{-1, +1}^D shared by Q and K (needed for Q K^T to be preserved) and by all
heads.

``fwht`` is the textbook in-place butterfly: log2(D) stages with strides
1, 2, 4, ..., D/2; each stage replaces (a, b) by (a + b, a - b). With
``dtype=np.float32`` every add/subtract is rounded to float32 in exactly that
stage order, which is the arithmetic the quantize kernel performs; the float64
form is the exact transform up to float64 rounding.
"""

from __future__ import annotations

import numpy as np


def sylvester(d: int) -> np.ndarray:
    """Explicit D x D Sylvester Hadamard matrix (entries +-1, float64)."""
    if d < 1 or d & (d - 1):
        raise ValueError("D must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht(x, dtype=np.float64) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis.

    Equals x @ sylvester(D) (H is symmetric) up to the rounding of ``dtype``.
    """
    y = np.array(x, dtype=dtype, copy=True)
    d = y.shape[-1]
    if d < 1 or d & (d - 1):
        raise ValueError("D must be a power of two")
    lead = y.shape[:-1]
    h = 1
    while h < d:
        y = y.reshape(lead + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b          # rounded to dtype
        y[..., 1, :] = a - b
        y = y.reshape(lead + (d,))
        h *= 2
    return y


def random_sign_hadamard(x, signs) -> np.ndarray:
    """x' = H_D diag(signs) x / sqrt(D) along the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    d = x.shape[-1]
    if s.shape != (d,) or not np.all(np.abs(s) == 1):
        raise ValueError("signs must be a +-1 vector of length D")
    return fwht(x * s) / np.sqrt(d)
