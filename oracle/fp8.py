"""FP8 (OCP E4M3) encoding and the block / per-tensor quantizers.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages say only that FP8 doubles tensor-core throughput at the price of a
narrow dynamic range ([NL] "Nieuwe hardwaremogelijkheden van GPU Hopper
(H100)"; [GN] "Hopper-GPU-Funktionen: WGMMA, TMA, FP8") and that Q and K are
quantized after the Hadamard transform ([NL] "3. Lage precisie (FP8) met
reductie van kwantisatiefout"). Readings:

* format: OCP 8-bit floating point E4M3 ("E4M3FN"): 1 sign, 4 exponent bits
  (bias 7), 3 mantissa bits; subnormals when the exponent field is 0; no
  infinities; S.1111.111 is NaN; largest finite value 448. This is the format
  of the matrix cores on the target GPU.
* rounding: to nearest, ties to even, saturating at +-448 (a value is never
  turned into NaN by quantization).
* scales: per block of ``block_rows`` consecutive sequence rows x all D
  columns, per (b, h): a = max|x| over the block (exact), inv = fl32(448 / a),
  code = E4M3(fl32(x * inv)), scale = fl32(a / 448). An all-zero block has
  scale 1 and codes 0. Per-tensor quantization is the same with one block
  covering the whole tensor.
* with the Hadamard transform, u = FWHT(s * x) is formed in float32 with the
  stage order of ``oracle.hadamard.fwht`` (the transform is left unnormalised
  while choosing codes) and the block scale is then multiplied by
  r = fl32(1 / sqrt(D)) in float32, so that code * scale approximates
  H diag(s) x / sqrt(D). An all-zero block keeps scale 1 (no factor r).

All rounding decisions above are taken in float32, the precision of the
quantize kernel, so the expected codes are unique.
"""

from __future__ import annotations

import numpy as np

from .hadamard import fwht

E4M3_MAX = 448.0
_E4M3_BIAS = 7


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8 array) as float64; NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * (1.0 + m / 8.0) * np.exp2(e - _E4M3_BIAS)
    sub = sign * (m / 8.0) * np.exp2(1 - _E4M3_BIAS)
    val = np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & (m == 0x7), np.nan, val)


def _finite_table():
    """Sorted non-negative finite E4M3 values with their codes (0x00..0x7E)."""
    codes = np.arange(0x7F, dtype=np.uint8)
    return e4m3_decode(codes), codes


def e4m3_encode(x) -> np.ndarray:
    """Round float values to E4M3 codes: nearest, ties to even, saturate at 448.

    Works from the exact (float64) value of the input, so an input that is
    already float32 is rounded exactly once. NaN inputs give the NaN code.
    """
    x = np.asarray(x, dtype=np.float64)
    vals, codes = _finite_table()              # ascending, vals[i] is code i
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(vals, a, side="left")  # first value >= a
    hi = np.clip(hi, 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0))
    pick_hi = pick_hi | (vals[hi] == a)
    mag = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    neg = np.signbit(x)
    out = np.where(neg, mag | 0x80, mag).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0xFF), out).astype(np.uint8)


def _block_quant_f32(u32: np.ndarray, block_rows: int):
    """Quantize a float32 [B, H, S, D] array per (b, h, block of rows).

    Returns (codes, scales, nonzero) where nonzero flags the blocks with a > 0.
    """
    b, h, s, d = u32.shape
    nblk = -(-s // block_rows)
    codes = np.zeros((b, h, s, d), dtype=np.uint8)
    scales = np.ones((b, h, nblk), dtype=np.float32)
    nonzero = np.zeros((b, h, nblk), dtype=bool)
    for k in range(nblk):
        r0, r1 = k * block_rows, min(s, (k + 1) * block_rows)
        blk = u32[:, :, r0:r1, :]
        a = np.abs(blk).max(axis=(2, 3)).astype(np.float32)            # exact
        nz = a > 0
        a_safe = np.where(nz, a, np.float32(1))
        inv = (np.float32(E4M3_MAX) / a_safe).astype(np.float32)        # fl32 divide
        y = (blk * inv[:, :, None, None]).astype(np.float32)            # fl32 multiply
        codes[:, :, r0:r1, :] = np.where(nz[:, :, None, None], e4m3_encode(y), 0)
        scales[:, :, k] = np.where(nz, (a_safe / np.float32(E4M3_MAX)).astype(np.float32),
                                   np.float32(1))
        nonzero[:, :, k] = nz
    return codes, scales, nonzero


def quantize_blocks(x, block_rows: int = 64):
    """Block quantization without a transform: (codes uint8 [B,H,S,D], scales f32 [B,H,nblk])."""
    x32 = np.asarray(x, dtype=np.float32)
    codes, scales, _ = _block_quant_f32(x32, block_rows)
    return codes, scales


def hadamard_quantize(x, signs, block_rows: int = 64):
    """Random-sign Hadamard transform followed by block quantization.

    u = FWHT_f32(s * x) (stage order 1, 2, ..., D/2), codes and block scales as
    in ``quantize_blocks`` on u, then scale *= fl32(1/sqrt(D)) in float32.
    """
    x32 = np.asarray(x, dtype=np.float32)
    s = np.asarray(signs, dtype=np.float32)
    d = x32.shape[-1]
    u = fwht(x32 * s, dtype=np.float32)          # sign flips are exact
    codes, scales, nonzero = _block_quant_f32(u, block_rows)
    r = np.float32(1.0 / np.sqrt(np.float64(d)))
    scales = np.where(nonzero, (scales * r).astype(np.float32), np.float32(1)).astype(np.float32)
    return codes, scales


def quantize_per_tensor(x, amax=None):
    """One scale for the whole tensor: (codes uint8, scale float32 scalar).

    ``amax``, when given, is max |x| over the whole tensor of which x holds
    only a part (for example some heads); by default it is taken from x.
    """
    x32 = np.asarray(x, dtype=np.float32)
    if amax is not None:
        a = np.float32(amax)
        if x32.size and not np.float32(np.abs(x32).max()) <= a:
            raise ValueError("amax is smaller than max |x|")
    else:
        a = np.float32(np.abs(x32).max()) if x32.size else np.float32(0)
    if a == 0:
        return np.zeros(x32.shape, dtype=np.uint8), np.float32(1)
    inv = np.float32(np.float32(E4M3_MAX) / a)
    y = (x32 * inv).astype(np.float32)
    return e4m3_encode(y), np.float32(a / np.float32(E4M3_MAX))


def dequantize_blocks(codes, scales, block_rows: int = 64) -> np.ndarray:
    """codes [B,H,S,D] with scales [B,H,nblk] -> float64 values."""
    v = e4m3_decode(codes)
    s = np.asarray(scales, dtype=np.float64)
    rows = np.arange(v.shape[2]) // block_rows
    return v * s[:, :, rows][..., None]
