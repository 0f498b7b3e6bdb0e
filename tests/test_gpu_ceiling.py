"""The MFMA-only ceiling kernels (cutbce_mfma_ceiling on constant operands, cutbce_mfma_ceiling_random on
random operands) that bench.py reports beside the sweeps: each runs, every
wave records increasing timestamps, and the rate and clock it implies are physically possible (at most the
published dense bf16 peak at the 2.4 GHz peak clock)."""
import pytest
import torch

from vocabulary_label_bce_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("run", [B.mfma_ceiling, B.mfma_ceiling_random], ids=["constant", "random"])
def test_mfma_ceiling_stamps_and_rate(run):
    blocks, waves, iters = 64, 8, 2000
    stamps = torch.zeros(4 * blocks * waves, dtype=torch.int64, device="cuda")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s = torch.cuda.current_stream()
    run(blocks, waves, iters, stamps, s)
    ev0.record(s)
    run(blocks, waves, iters, stamps, s)
    ev1.record(s)
    torch.cuda.synchronize()
    st = stamps.view(-1, 4).cpu()
    assert (st[:, 1] > st[:, 0]).all() and (st[:, 3] > st[:, 2]).all()
    ghz = (0.1 * (st[:, 1] - st[:, 0]).double() / (st[:, 3] - st[:, 2]).double()).median().item()
    assert 0.3 < ghz < 2.6
    ms = ev0.elapsed_time(ev1)
    tflops = blocks * waves * iters * 4 * 32768 / (ms * 1e-3) / 1e12
    # 64 of the 256 CUs: at most a quarter of the 2.5 PFLOP/s peak
    assert 0.0 < tflops <= 2500.0 / 4 * 1.02
