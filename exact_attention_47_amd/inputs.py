"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module draws random numbers and nothing else: it holds none of the
attention, transform or quantization arithmetic, so that the GPU path and the
CPU oracle can be fed identical inputs without sharing any method code.

Recipe (the workloads the pages describe: Q, K, V drawn from a standard normal,
optionally with 0.1 % of entries made large to imitate activation outliers):

* every tensor is drawn with its own ``torch.Generator`` seeded from
  ``(seed, tensor_id, chunk)`` through NumPy's ``SeedSequence``; a chunk is one
  batch index, so large tensors are generated one batch row at a time;
* values are float32 standard normal, then rounded to the requested dtype
  (torch's float32 -> bfloat16/float16 conversion rounds to nearest even);
* outliers: each entry is independently replaced, with probability ``prob``,
  by a draw from N(0, sigma^2) (sigma = 10: standard deviation, not variance);
* Hadamard signs: a +-1 int8 vector of length D.

The CPU and the GPU generators produce different streams for the same seed:
a test that compares the two paths draws once and copies the tensor across.
"""

from __future__ import annotations

import numpy as np
import torch

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_MASK, TENSOR_OUTLIER, TENSOR_SIGNS = range(6)


def _seed(*parts: int) -> int:
    return int(np.random.SeedSequence([int(p) & 0xFFFFFFFF for p in parts]).generate_state(1)[0])


def _gen(device, *parts):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def normal(shape, seed: int, tensor_id: int, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """Standard-normal tensor [B, ...] drawn per batch index, rounded to ``dtype``."""
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=dtype, device=device)
    for b in range(shape[0]):
        g = _gen(device, seed, tensor_id, b)
        x = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
        out[b].copy_(x.to(dtype))
        del x
    return out


def with_outliers(shape, seed: int, tensor_id: int, prob: float = 1e-3, sigma: float = 10.0,
                  dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """N(0,1) tensor with entries replaced by N(0, sigma^2) draws with probability ``prob``."""
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=dtype, device=device)
    for b in range(shape[0]):
        g = _gen(device, seed, tensor_id, b)
        x = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
        gm = _gen(device, seed, tensor_id, TENSOR_MASK, b)
        hit = torch.rand(shape[1:], generator=gm, device=device) < prob
        go = _gen(device, seed, tensor_id, TENSOR_OUTLIER, b)
        big = torch.randn(shape[1:], generator=go, device=device, dtype=torch.float32) * sigma
        out[b].copy_(torch.where(hit, big, x).to(dtype))
        del x, hit, big
    return out


def signs(d: int, seed: int) -> torch.Tensor:
    """Random +-1 vector of length ``d`` (int8, CPU)."""
    g = _gen("cpu", seed, TENSOR_SIGNS)
    bits = torch.randint(0, 2, (int(d),), generator=g)
    return (bits * 2 - 1).to(torch.int8)


def qkv(b, h, s_q, s_k, d, seed=0, dtype=torch.bfloat16, device="cpu", outliers=False):
    """The (Q, K, V) triple for one workload, [B, H, S, D] contiguous."""
    make = with_outliers if outliers else normal
    q = make((b, h, s_q, d), seed, TENSOR_Q, dtype=dtype, device=device)
    k = make((b, h, s_k, d), seed, TENSOR_K, dtype=dtype, device=device)
    v = make((b, h, s_k, d), seed, TENSOR_V, dtype=dtype, device=device)
    return q, k, v


TENSOR_LENGTHS = 6


def packed_qkv(lens_q, lens_k, h, d, seed=0, dtype=torch.bfloat16, device="cpu"):
    """(Q, K, V, cu_q, cu_k) of a packed batch: Q [sum(lens_q), H, D], K and V [sum(lens_k), H, D].

    Sequence b is drawn as its own chunk (its rows do not depend on the other
    sequences' lengths); cu_* are int32 offsets (0, running totals) on ``device``.
    """
    lens_q = [int(x) for x in lens_q]
    lens_k = [int(x) for x in lens_k]
    if len(lens_q) != len(lens_k) or min(lens_q + lens_k) < 0:
        raise ValueError("one non-negative query and key length per sequence")
    out = []
    for tid, lens in ((TENSOR_Q, lens_q), (TENSOR_K, lens_k), (TENSOR_V, lens_k)):
        t = torch.empty((sum(lens), h, d), dtype=dtype, device=device)
        row = 0
        for b, n in enumerate(lens):
            if n:
                g = _gen(device, seed, tid, b)
                t[row:row + n].copy_(torch.randn((n, h, d), generator=g, device=device, dtype=torch.float32).to(dtype))
            row += n
        out.append(t)
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(lens_q)]), dtype=torch.int32, device=device)
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(lens_k)]), dtype=torch.int32, device=device)
    return (*out, cu_q, cu_k)


def sequence_lengths(n_seq: int, total: int, seed: int, min_len: int = 1):
    """``n_seq`` lengths >= ``min_len`` summing to ``total``: a uniform random split of the total."""
    if n_seq < 1 or total < n_seq * min_len:
        raise ValueError("total too small for the number of sequences")
    g = _gen("cpu", seed, TENSOR_LENGTHS)
    cuts = torch.randperm(total - n_seq * min_len + n_seq - 1, generator=g)[:n_seq - 1].sort().values
    edges = [-1] + cuts.tolist() + [total - n_seq * min_len + n_seq - 1]
    return [edges[i + 1] - edges[i] - 1 + min_len for i in range(n_seq)]


def rope_tables(s: int, d: int, base: float = 10000.0, device="cpu"):
    """cos and sin tables float32 [S, D/2] of the standard rotary angles p * base^(-2j/D).

    Workload inputs for the fused rotary + Hadamard quantizer (a model supplies
    such tables); formed in float64 and rounded once to float32.
    """
    j = np.arange(d // 2, dtype=np.float64)
    th = np.arange(s, dtype=np.float64)[:, None] * base ** (-2.0 * j / d)[None, :]
    return (torch.from_numpy(np.cos(th).astype(np.float32)).to(device),
            torch.from_numpy(np.sin(th).astype(np.float32)).to(device))
