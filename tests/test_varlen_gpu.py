"""GPU parity of attn_fwd_varlen (packed batches) against the CPU oracle, through the C ABI.

Same bar as the dense path for bfloat16/float16 with N(0,1) inputs: O max-abs
<= 1e-2, RMSE <= 2e-3, LSE max-abs <= 1e-3 on every row that has an allowed
key; rows without one must be exactly O = 0 and LSE = -inf. Equal-length
batches must match the dense entry point bit for bit (same kernel, only the
addressing differs).
"""

import numpy as np
import pytest
import torch

import oracle
from exact_attention_47_amd import inputs

pytestmark = pytest.mark.gpu

BF_MAX, BF_RMSE, LSE_MAX = 1e-2, 2e-3, 1e-3


def note(msg):
    print(f"[case] {msg}", flush=True)


def check(o, lse, q, k, v, cu_q, cu_k, causal, scale, what):
    ref, ref_lse = oracle.attention_varlen(q.float().cpu().numpy(), k.float().cpu().numpy(),
                                           v.float().cpu().numpy(), cu_q.cpu().numpy(), cu_k.cpu().numpy(),
                                           causal, scale)
    og = o.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    has = np.isfinite(ref_lse[0])                        # rows with at least one allowed key
    if (~has).any():
        assert np.all(og[~has] == 0.0), what
        assert np.all(lg[:, ~has] == -np.inf), what
    if has.any():
        d = np.abs(og[has] - ref[has])
        mx, rm = float(d.max()), float(np.sqrt(np.mean(d ** 2)))
        ls = float(np.abs(lg[:, has] - ref_lse[:, has]).max())
        print(f"    {what}: O max {mx:.2e} rmse {rm:.2e} LSE max {ls:.2e}")
        assert mx <= BF_MAX and rm <= BF_RMSE and ls <= LSE_MAX, what


CASES = [
    # (lens_q, lens_k, causal): ragged self-attention with an empty sequence and
    # lengths around the 256-row / 128-key tiles; cross lengths; causal rows
    # above the diagonal (S_q > S_k); an empty key sequence
    ([1, 100, 257, 513, 64, 0], [1, 100, 257, 513, 64, 0], False),
    ([1, 100, 257, 513, 64, 0], [1, 100, 257, 513, 64, 0], True),
    ([7, 300, 129], [50, 300, 700], False),
    ([7, 300, 129], [50, 300, 700], True),
    ([40, 10, 300], [20, 10, 260], True),
    ([5, 8], [0, 8], False),
    # longest key sequence past the short-range kernel's range at D = 128 (and at D = 64 for the
    # last case): the main kernel's packed form; the shorter cases above run on the short-range kernel
    # at D = 64 / 128
    ([1100, 2100, 50], [1100, 2100, 50], False),
    ([300, 2300, 700], [900, 2300, 700], True),
    ([4200, 100], [4200, 130], False),
]


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_varlen_against_oracle(gpu_lib, case, dtype, D):
    lens_q, lens_k, causal = CASES[case]
    note(f"varlen lens_q={lens_q} lens_k={lens_k} causal={causal} {dtype} D{D}")
    H, scale = 3, D ** -0.5
    q, k, v, cu_q, cu_k = inputs.packed_qkv(lens_q, lens_k, H, D, seed=11 + case, dtype=dtype, device="cuda")
    o, lse = gpu_lib.fwd_varlen(q, k, v, cu_q, cu_k, causal=causal, scale=scale)
    torch.cuda.synchronize()
    check(o, lse, q, k, v, cu_q, cu_k, causal, scale, f"case {case}")


@pytest.mark.parametrize("S,causal,D", [(2000, False, 128), (2500, True, 128), (700, False, 256),
                                        (1100, True, 256), (700, False, 128), (1500, True, 64)])
def test_varlen_equal_lengths_bitwise_equal_dense(gpu_lib, S, causal, D):
    """B sequences of one length: the packed path gives the dense path's bits, transposed in layout.

    (The packed and dense entry points pick the kernel alike: the main kernel at D = 128 beyond the
    short-range kernel's ranges, the short-range kernel within them, the D = 256 kernel at any
    length.)"""
    note(f"varlen vs dense S{S} causal={causal} D{D}")
    B, H = 2, 4
    q, k, v = inputs.qkv(B, H, S, S, D, seed=5, dtype=torch.bfloat16, device="cuda")
    o_d, lse_d = gpu_lib.fwd(q, k, v, causal=causal)
    pack = lambda t: t.transpose(1, 2).reshape(B * S, H, D).contiguous()
    cu = torch.arange(0, (B + 1) * S, S, dtype=torch.int32, device="cuda")
    o_v, lse_v = gpu_lib.fwd_varlen(pack(q), pack(k), pack(v), cu, cu, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o_v, pack(o_d))
    assert torch.equal(lse_v, lse_d.permute(1, 0, 2).reshape(H, B * S))


@pytest.mark.parametrize("H,D", [(16, 128), (8, 256)])
def test_varlen_fullsize_sampled_rows(gpu_lib, H, D):
    """The bench workload (8 causal sequences of random lengths summing to 16K tokens, H16 D128)
    launched as the bench launches it, and the same lengths at D = 256 (H8, the D = 256 shape's
    heads); sampled rows of every sequence against the oracle."""
    lens = inputs.sequence_lengths(8, 16384, 0, 256)
    note(f"varlen full size lens={lens} H{H} D{D} causal")
    scale = D ** -0.5
    q, k, v, cu_q, cu_k = inputs.packed_qkv(lens, lens, H, D, seed=0, device="cuda")
    o, lse = gpu_lib.fwd_varlen(q, k, v, cu_q, cu_k, causal=True, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    cu = cu_q.cpu().numpy()
    for b in range(len(lens)):
        rows = np.sort(rng.choice(lens[b], size=min(24, lens[b]), replace=False))
        heads = rng.choice(H, size=2, replace=False)
        kk = k[cu[b]:cu[b + 1]].float().cpu().numpy()
        vv = v[cu[b]:cu[b + 1]].float().cpu().numpy()
        qq = q[cu[b]:cu[b + 1]].float().cpu().numpy()
        for h in heads:
            ref, ref_lse = oracle.attention_rows(qq[rows, h], kk[:, h], vv[:, h], rows, True, scale,
                                                 s_q=lens[b])
            d = np.abs(o[cu[b] + rows, h].float().cpu().numpy() - ref)
            ls = np.abs(lse[h, cu[b] + rows].cpu().numpy() - ref_lse).max()
            assert d.max() <= BF_MAX and np.sqrt(np.mean(d ** 2)) <= BF_RMSE and ls <= LSE_MAX, (b, h)


def test_varlen_reuses_outputs_and_leaves_empty_sequences_alone(gpu_lib):
    """Given out/lse buffers are written in place; rows of empty key sequences come back as 0 / -inf."""
    note("varlen out= buffers")
    q, k, v, cu_q, cu_k = inputs.packed_qkv([33, 70], [0, 90], 2, 64, seed=3, device="cuda")
    out = torch.full_like(q, 7.0)
    lse = torch.full((2, q.shape[0]), 7.0, device="cuda")
    o2, l2 = gpu_lib.fwd_varlen(q, k, v, cu_q, cu_k, out=out, lse=lse)
    torch.cuda.synchronize()
    assert o2.data_ptr() == out.data_ptr() and l2.data_ptr() == lse.data_ptr()
    assert torch.all(out[:33] == 0) and torch.all(lse[:, :33] == float("-inf"))
    assert torch.isfinite(lse[:, 33:]).all()
