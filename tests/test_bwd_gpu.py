"""GPU parity of attn_bwd (dQ, dK, dV) against the CPU oracle's gradients, through the C ABI.

Inputs Q, K, V, dO iid N(0,1) in bf16/fp16; O and LSE come from attn_fwd on the GPU. The
kernels multiply bf16/fp16 operands (P, dS, Q, K, V, dO) with float32 accumulation and round the
gradients to the input dtype, so each gradient element carries relative errors of about 2^-9 from
its operands' rounding, partly averaged over the key / query sums: the bound is a relative RMSE
of 1e-2 (about four times the measured error) and a max-abs error of 3 % of the largest
reference element, per gradient tensor.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_47_amd import inputs

pytestmark = pytest.mark.gpu

REL_RMSE, REL_MAX = 1e-2, 3e-2


def note(msg):
    print(f"[case] {msg}", flush=True)


def check(name, got, ref):
    g = got.float().cpu().numpy().astype(np.float64)
    d = g - ref
    rms = float(np.sqrt(np.mean(ref ** 2)))
    rel_rmse = float(np.sqrt(np.mean(d ** 2))) / rms
    rel_max = float(np.abs(d).max()) / float(np.abs(ref).max())
    print(f"    {name}: rel rmse {rel_rmse:.2e}  max/max {rel_max:.2e}")
    assert rel_rmse <= REL_RMSE and rel_max <= REL_MAX, name


def run_case(lib, B, H, S_q, S_k, D, causal, dt, seed):
    q, k, v = inputs.qkv(B, H, S_q, S_k, D, seed=seed, dtype=dt, device="cuda")
    do = inputs.normal((B, H, S_q, D), seed, inputs.TENSOR_OUTLIER, dtype=dt, device="cuda")
    scale = 1 / math.sqrt(D)
    o, lse = lib.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = lib.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return q, k, v, do, scale, dq, dk, dv


CASES = [
    (1, 2, 200, 200, 64, False), (1, 2, 200, 200, 128, True), (1, 2, 100, 333, 128, False),
    (1, 2, 130, 257, 64, True), (2, 1, 1, 70, 128, False), (1, 1, 33, 33, 128, True),
    # several 128-row outer blocks per head: interior (unmasked) tiles, the causal heaviest-first deal,
    # and at D = 64 the fused dK/dV pass over many inner tiles
    (1, 2, 1000, 1000, 64, True), (1, 2, 700, 1100, 64, False), (1, 2, 900, 900, 128, True),
]


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}q{c[2]}k{c[3]}D{c[4]}{'c' if c[5] else 'n'}")
def test_bwd_against_oracle(gpu_lib, case, dt):
    B, H, S_q, S_k, D, causal = case
    note(f"bwd {case} {dt}")
    q, k, v, do, scale, dq, dk, dv = run_case(gpu_lib, B, H, S_q, S_k, D, causal, dt, 3)
    rq, rk, rv = oracle.attention_backward(q.float().cpu().numpy(), k.float().cpu().numpy(),
                                           v.float().cpu().numpy(), do.float().cpu().numpy(), causal, scale)
    check("dQ", dq, rq)
    check("dK", dk, rk)
    check("dV", dv, rv)


def test_bwd_fullsize_two_heads(gpu_lib):
    """B=2, H=16, S=2048, D=128, causal (a training-sized step), two heads against the oracle."""
    note("bwd full size B2 H16 S2048 D128 causal")
    B, H, S, D = 2, 16, 2048, 128
    q, k, v, do, scale, dq, dk, dv = run_case(gpu_lib, B, H, S, S, D, True, torch.bfloat16, 0)
    for b, h in ((0, 0), (1, 15)):
        rq, rk, rv = oracle.attention_backward(q[b:b + 1, h:h + 1].float().cpu().numpy(),
                                               k[b:b + 1, h:h + 1].float().cpu().numpy(),
                                               v[b:b + 1, h:h + 1].float().cpu().numpy(),
                                               do[b:b + 1, h:h + 1].float().cpu().numpy(), True, scale)
        check(f"dQ b{b}h{h}", dq[b:b + 1, h:h + 1], rq)
        check(f"dK b{b}h{h}", dk[b:b + 1, h:h + 1], rk)
        check(f"dV b{b}h{h}", dv[b:b + 1, h:h + 1], rv)


@pytest.mark.parametrize("B,H,S,D,causal", [(2, 16, 8192, 128, False), (2, 16, 8192, 128, True),
                                            (4, 32, 4096, 64, False), (4, 32, 4096, 64, True)],
                         ids=["B2H16S8K_D128_n", "B2H16S8K_D128_c", "B4H32S4K_D64_n", "B4H32S4K_D64_c"])
def test_bwd_bench_workloads_two_heads(gpu_lib, B, H, S, D, causal):
    """The backward workloads the bench times (same seed, inputs and launch), two whole heads against
    the oracle: the first and the last (b, h), which sit on different XCDs and, when causal, take the
    heaviest-first deal's first and last outer blocks."""
    note(f"bwd bench workload B{B} H{H} S{S} D{D} causal={causal}")
    q, k, v, do, scale, dq, dk, dv = run_case(gpu_lib, B, H, S, S, D, causal, torch.bfloat16, 0)
    for b, h in ((0, 0), (B - 1, H - 1)):
        rq, rk, rv = oracle.attention_backward(q[b:b + 1, h:h + 1].float().cpu().numpy(),
                                               k[b:b + 1, h:h + 1].float().cpu().numpy(),
                                               v[b:b + 1, h:h + 1].float().cpu().numpy(),
                                               do[b:b + 1, h:h + 1].float().cpu().numpy(), causal, scale)
        check(f"dQ b{b}h{h}", dq[b:b + 1, h:h + 1], rq)
        check(f"dK b{b}h{h}", dk[b:b + 1, h:h + 1], rk)
        check(f"dV b{b}h{h}", dv[b:b + 1, h:h + 1], rv)


def test_bwd_is_deterministic(gpu_lib):
    note("bwd determinism")
    q, k, v, do, scale, dq, dk, dv = run_case(gpu_lib, 1, 4, 500, 500, 128, True, torch.bfloat16, 5)
    o, lse = gpu_lib.fwd(q, k, v, causal=True, scale=scale)
    dq2, dk2, dv2 = gpu_lib.bwd(q, k, v, o, lse, do, causal=True, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
