"""attn_fwd_noalloc, the entry point that allocates nothing, against attn_fwd through the C ABI.

attn_fwd_noalloc runs attn_fwd's kernels with the key-range split's partial
results staged in the library's fixed device scratch array instead of a fresh
allocation, so its outputs must be attn_fwd's, bit for bit. Two split calls in
a row, the second smaller (the array keeps the first call's contents), then a
shape that needs no split, then a shape whose split would overflow the array
(refused on the host before anything is enqueued).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_47_amd import attn, inputs

pytestmark = pytest.mark.gpu

P = 0x10000  # fake, 16-byte aligned addresses: the refused call never dereferences them


def note(msg):
    print(f"[case] {msg}", flush=True)


def test_noalloc_matches_attn_fwd_on_two_calls(gpu_lib):
    cases = [
        # B, H, S_q, S_k, D, dtype: first the larger split (short-range kernel, 16 query rows), then a
        # smaller one (decode kernel)
        (4, 8, 16, 12000, 128, torch.bfloat16),
        (2, 4, 1, 9000, 64, torch.float16),
    ]
    for B, H, S_q, S_k, D, dt in cases:
        n = attn.num_splits(B, H, S_q, S_k, D)
        need = attn.workspace_size(B, H, S_q, S_k, D)
        note(f"noalloc B{B} H{H} S_q{S_q} S_k{S_k} D{D} {dt}: {n} splits, {need} scratch bytes")
        assert n > 1 and 0 < need <= attn.NOALLOC_SCRATCH_BYTES
        q, k, v = inputs.qkv(B, H, S_q, S_k, D, seed=31, dtype=dt, device="cuda")
        o_ref, l_ref = gpu_lib.fwd(q, k, v, causal=False)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, H, S_q), float("nan"), device="cuda")
        gpu_lib.fwd_noalloc(q, k, v, causal=False, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        # and within the bf16/fp16 bounds of the oracle on two heads
        for b, h in ((0, 0), (B - 1, H - 1)):
            ro, rl = oracle.attention(q[b, h][None, None].float().cpu().numpy(),
                                      k[b, h][None, None].float().cpu().numpy(),
                                      v[b, h][None, None].float().cpu().numpy(), False, 1 / math.sqrt(D))
            d = np.abs(o[b, h].float().cpu().numpy() - ro[0, 0])
            le = float(np.abs(lse[b, h].cpu().numpy() - rl[0, 0]).max())
            assert d.max() <= 1e-2 and np.sqrt(np.mean(d ** 2)) <= 2e-3 and le <= 1e-3


def test_noalloc_low_occupancy_split(gpu_lib):
    """A grid too small for the chip against a long key range: attn_fwd splits it within the scratch
    array's size, so attn_fwd_noalloc takes the same split and gives the same bits."""
    B, H, S_q, S_k, D = 1, 4, 700, 20000, 128
    n = attn.num_splits(B, H, S_q, S_k, D)
    note(f"noalloc low-occupancy split B{B} H{H} S_q{S_q} S_k{S_k}: {n} splits")
    assert n > 1 and 0 < attn.workspace_size(B, H, S_q, S_k, D) <= attn.NOALLOC_SCRATCH_BYTES
    q, k, v = inputs.qkv(B, H, S_q, S_k, D, seed=33, dtype=torch.bfloat16, device="cuda")
    for causal in (False, True):
        o_ref, l_ref = gpu_lib.fwd(q, k, v, causal=causal)
        o, lse = gpu_lib.fwd_noalloc(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


def test_noalloc_without_split_and_refused_sizes(gpu_lib):
    note("noalloc: unsplit shape, then a split that would overflow the scratch array")
    q, k, v = inputs.qkv(1, 2, 300, 300, 128, seed=32, dtype=torch.bfloat16, device="cuda")
    o_ref, l_ref = gpu_lib.fwd(q, k, v, causal=True)
    o, lse = gpu_lib.fwd_noalloc(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    B, H, S_q, S_k, D = 8, 32, 64, 8192, 128
    assert attn.workspace_size(B, H, S_q, S_k, D) > attn.NOALLOC_SCRATCH_BYTES
    import ctypes
    rc = attn.load().attn_fwd_noalloc(P, P, P, P, P, B, H, S_q, S_k, D, 0, ctypes.c_float(0.125), attn.BF16, None)
    assert rc == attn.ERR_WORKSPACE
