"""GPU checks of the roundings where random data almost never lands on a tie.

* E4M3 codes (hadamard_quant without the transform, quant_per_tensor): a block
  whose maximum is exactly 448 has inv = 448 / 448 = 1, so its elements reach
  the conversion unchanged. Such a block holds every finite E4M3 value, every
  midpoint between neighbours (ties go to the even code), and the bf16 / fp16
  neighbours just above and below each midpoint, with both signs. A block
  whose maximum is 0.60546875 maps that maximum to fl32(a * fl32(448 / a)) =
  448.00003, just past the largest finite E4M3 value: it must give 448 (code
  0x7E), never NaN. Codes and scales are compared bit for bit with the oracle.
* Rounding of O to bf16 / fp16: with Q = 0 every probability is 1, so O is the
  mean of V over the keys. V rows 0 and 1 hold a value and its neighbour one
  step up in the output type, every other row is 0, and S_k is a power of two,
  so O = (v0 + v1) / S_k is exactly halfway between two representable values.
  Round to nearest even is the reading of the pages' silence on rounding; a
  truncating or round-half-up conversion gives a different result in half of
  these columns, which the test also asserts.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_attention_47_amd import inputs

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[case] {msg}", flush=True)


def finite_e4m3():
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))      # 0 .. 448, ascending
    return vals


def neighbours(x, dt):
    """The representable values of dtype dt just below and just above x (x representable)."""
    t = torch.tensor(x, dtype=dt)
    up = torch.nextafter(t, torch.tensor(np.inf, dtype=dt))
    dn = torch.nextafter(t, torch.tensor(-np.inf, dtype=dt))
    return dn.float().numpy(), up.float().numpy()


def tie_block(dt):
    """64 x 128 values: the E4M3 grid, its midpoints and their dtype neighbours, both signs; max 448."""
    vals = finite_e4m3()
    mids = (vals[:-1] + vals[1:]) / 2
    dn, up = neighbours(mids, dt)
    pos = np.concatenate([vals, mids, dn[mids > 0], up])
    allv = np.concatenate([pos, -pos])
    blk = np.zeros(64 * 128)
    blk[: allv.size] = allv
    blk[-1] = 448.0
    assert np.array_equal(torch.tensor(blk, dtype=dt).double().numpy(), blk)   # all exactly representable
    return blk.reshape(64, 128)


def edge_block(dt):
    """A block whose maximum maps just past 448: 0.60546875 * fl32(448 / 0.60546875) = 448.00003."""
    a = np.float32(0.60546875)
    assert np.float32(a * np.float32(np.float32(448) / a)) > np.float32(448)
    rng = np.random.default_rng(11)
    blk = rng.uniform(-0.6, 0.6, size=(64, 128))
    blk[0, 0], blk[5, 7] = a, -a
    blk = torch.tensor(blk, dtype=dt).double().numpy()
    return blk


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_e4m3_ties_and_saturation_edge_bitexact(gpu_lib, dt):
    note(f"E4M3 ties and 448 edge, {dt}")
    x = np.stack([tie_block(dt), edge_block(dt)]).reshape(1, 1, 128, 128)
    xt = torch.tensor(x, dtype=dt)
    x8, sc = gpu_lib.hadamard_quant(xt.cuda(), inputs.signs(128, 0).cuda(), block_rows=64,
                                    apply_hadamard=False)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_blocks(xt.float().numpy(), 64)
    assert sc.cpu().numpy()[0, 0, 0] == 1.0                      # 448 / 448: the ties reach the conversion as is
    np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    np.testing.assert_array_equal(x8.cpu().numpy(), rc)
    assert x8[0, 0, 64, 0].item() == 0x7E and x8[0, 0, 69, 7].item() == 0xFE   # 448.00003 -> 448, never NaN
    assert not bool(((x8 & 0x7F) == 0x7F).any())                                 # no NaN code anywhere
    for blk in (x[:, :, :64], x[:, :, 64:]):                     # one scale for the whole tensor
        bt = torch.tensor(blk, dtype=dt)
        p8, ps = gpu_lib.quant_per_tensor(bt.cuda())
        torch.cuda.synchronize()
        pc, pscale = oracle.quantize_per_tensor(bt.float().numpy())
        assert ps.cpu().numpy().view(np.uint32)[0] == np.float32(pscale).view(np.uint32)
        np.testing.assert_array_equal(p8.cpu().numpy(), pc)


def rne_expected(x32, dt):
    """x32 (float32, exactly representable midpoints) rounded to dt by nearest-even and by truncation."""
    bits = x32.view(np.uint32).astype(np.uint64)
    if dt == torch.bfloat16:
        rne = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
        trunc = (bits >> 16).astype(np.uint16)
        return rne, trunc
    # float16: the float32 values here are normal float16 numbers, so the mantissa keeps its top 10 bits
    rne = torch.tensor(x32).to(torch.float16).numpy().view(np.uint16)     # torch's conversion is RNE
    t = torch.tensor(x32).to(torch.float16).float().numpy()
    trunc = np.where(np.abs(t) > np.abs(x32),
                     torch.tensor(x32).to(torch.float16).numpy().view(np.uint16) - 1,
                     torch.tensor(x32).to(torch.float16).numpy().view(np.uint16)).astype(np.uint16)
    return rne, trunc


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("S_k,D,what", [(2, 128, "short-range kernel"), (2048, 128, "main kernel"),
                                        (8192, 64, "split short-range kernel D64"), (256, 256, "D=256 kernel")])
def test_output_rounds_to_nearest_even_at_midpoints(gpu_lib, dt, S_k, D, what):
    note(f"O rounding at midpoints, {what}, S_k={S_k} D={D} {dt}")
    S_q = 64
    rng = np.random.default_rng(D + S_k)
    # column d: v0 = a value of dt with a random exponent, sign and mantissa parity, v1 = its upper neighbour
    mag = np.exp2(rng.integers(0, 4, size=D)) * (1 + rng.integers(0, 128, size=D) / 128.0)   # O stays normal in fp16
    v0 = torch.tensor(mag * rng.choice([-1.0, 1.0], size=D), dtype=dt)
    v1 = torch.nextafter(v0, torch.tensor(np.inf, dtype=dt))
    v = torch.zeros((1, 1, S_k, D), dtype=dt)
    v[0, 0, 0], v[0, 0, 1] = v0, v1
    q = torch.zeros((1, 1, S_q, D), dtype=dt)
    k = inputs.normal((1, 1, S_k, D), 4, inputs.TENSOR_K, dtype=dt)
    o, lse = gpu_lib.fwd(q.cuda(), k.cuda(), v.cuda(), causal=False)
    torch.cuda.synchronize()
    exact = ((v0.double() + v1.double()) / S_k).numpy()
    x32 = exact.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), exact)        # the midpoints are float32 numbers
    rne, trunc = rne_expected(x32, dt)
    got = o[0, 0].cpu().view(torch.int16).numpy().view(np.uint16)
    assert (got == rne[None, :]).all(), np.argwhere(got != rne[None, :])[:5]
    assert int((rne != trunc).sum()) >= D // 4                  # the case tells RNE from truncation
    assert float(np.abs(lse.cpu().numpy() - np.log(S_k)).max()) <= 1e-6
