"""GPU check of attn_mfma_stream, the matrix-core stream that bench.py times beside the attention kernels.

It is a measurement aid, not part of the attention path: the test checks that each kind runs, reports the
floating-point operations the launch performs (2*M*N*K per instruction, 32*iters instructions per wave, two
waves per SIMD on every CU), writes one finite value per thread, and refuses a sink that is too small.
"""

import pytest
import torch

from exact_attention_47_amd import attn

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,mnk", [(0, 32 * 32 * 16), (1, 32 * 32 * 64), (2, 16 * 16 * 32)])
def test_mfma_stream_runs_and_counts(gpu_lib, kind, mnk):
    print(f"[case] mfma stream kind {kind}", flush=True)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.full((2 * n_cu * 256,), float("nan"), dtype=torch.float32, device="cuda")
    iters = 50
    flop = attn.mfma_stream(kind, iters, sink=sink)
    torch.cuda.synchronize()
    assert flop == 2.0 * mnk * 32 * iters * (2 * n_cu * 4)
    assert bool(torch.isfinite(sink).all())
    small = torch.empty(2 * n_cu * 256 - 4, dtype=torch.float32, device="cuda")
    with pytest.raises(attn.AttnError):
        attn.mfma_stream(kind, iters, sink=small)
