"""Rotary position embedding ahead of the Hadamard quantizer, as its plain definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[GN] "Niedrige FP8-Präzision und incoherent processing" notes that the
Hadamard transform is bound by memory bandwidth and costs nothing extra when
fused with a preceding memory-bound operation such as rotary embedding. The
pages do not define rotary embedding; the reading taken here is the usual
rotation of pairs of head-dimension coordinates by a position-dependent angle:
for position p and pair j,

    x'_a = x_a cos(theta_pj) - x_b sin(theta_pj)
    x'_b = x_b cos(theta_pj) + x_a sin(theta_pj)

with the pairs (a, b) = (2j, 2j+1) ("interleaved", mode 0) or (j, j + D/2)
("halves", mode 1). The angles reach the fused kernel as caller-supplied
cos/sin tables [S, D/2] (float32), as a model would pass them, so the method's
own arithmetic is only the rotation above. ``rope_angles`` gives the standard
angles theta_pj = p * base^(-2j/D) for the pins and the workloads.

``rotary_f32`` mirrors the kernel's float32 decisions (each product and each
sum rounded on its own, no fused multiply-add), because its output feeds the
quantizer, whose codes are compared bit for bit; ``rotary`` is the float64
definition used by the pins.
"""

from __future__ import annotations

import numpy as np

from .fp8 import hadamard_quantize


def rope_angles(s: int, d: int, base: float = 10000.0) -> np.ndarray:
    """theta[p, j] = p * base^(-2j/D), float64 [S, D/2]."""
    j = np.arange(d // 2, dtype=np.float64)
    return np.arange(s, dtype=np.float64)[:, None] * base ** (-2.0 * j / d)[None, :]


def _pairs(d: int, mode: int):
    j = np.arange(d // 2)
    if mode == 0:
        return 2 * j, 2 * j + 1
    if mode == 1:
        return j, j + d // 2
    raise ValueError("mode must be 0 (interleaved pairs) or 1 (halves)")


def rotary(x, cos, sin, mode: int) -> np.ndarray:
    """Rotation of [..., S, D] by per-position tables [S, D/2], float64."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    a, b = _pairs(x.shape[-1], mode)
    out = np.empty_like(x)
    out[..., a] = x[..., a] * c - x[..., b] * s
    out[..., b] = x[..., b] * c + x[..., a] * s
    return out


def rotary_f32(x, cos, sin, mode: int) -> np.ndarray:
    """The same rotation with float32 inputs and every operation rounded to float32."""
    x = np.asarray(x, dtype=np.float32)
    c = np.asarray(cos, dtype=np.float32)
    s = np.asarray(sin, dtype=np.float32)
    a, b = _pairs(x.shape[-1], mode)
    out = np.empty_like(x)
    out[..., a] = (x[..., a] * c).astype(np.float32) - (x[..., b] * s).astype(np.float32)
    out[..., b] = (x[..., b] * c).astype(np.float32) + (x[..., a] * s).astype(np.float32)
    return out


def rope_hadamard_quantize(x, cos, sin, mode: int, signs, block_rows: int = 64):
    """Rotary embedding (float32) followed by the random-sign Hadamard block quantizer."""
    return hadamard_quantize(rotary_f32(x, cos, sin, mode), signs, block_rows)
