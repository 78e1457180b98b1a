"""The MFMA calibration probe (a measurement aid, not part of the method)
runs in all four modes and reports the flops of its launch."""
import pytest
import torch

from response_replay_attention_amd import ls_calib_mfma

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_calib_probe_runs_and_counts_its_flops(mode):
    wgs, iters = 4, 16
    out = torch.full((wgs * 512,), float("nan"), dtype=torch.float32, device="cuda")
    flops = ls_calib_mfma(mode, wgs, iters, out)
    torch.cuda.synchronize()
    assert flops == wgs * 8 * iters * 4 * 32768
    assert bool(torch.isfinite(out).all())  # every thread stored its sum
