"""The matrix-instruction throughput probe (a measurement aid of bench.py)."""
import pytest
import torch

import particle_grid_mass_amd as mm

pytestmark = pytest.mark.gpu


def test_probe_runs_and_writes_every_thread():
    out = torch.full((8 * 256,), float("nan"), dtype=torch.float64, device="cuda")
    mm.probe_mfma_f64(8, 3, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert (out != 0).all()
    # the same call twice gives the same sums (no state between calls)
    again = mm.probe_mfma_f64(8, 3)
    torch.cuda.synchronize()
    assert torch.equal(out, again)
