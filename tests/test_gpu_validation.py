"""The binding refuses, on the host, buffers that would make a kernel read or
write out of bounds: binning arrays of another grid or too short for the
particles, and record sets smaller than what the deposition reads (records of
another grid, or scalar records deposited as 3x3 ones). Every call here
raises before anything is enqueued."""
import numpy as np
import pytest
import torch

import particle_grid_mass_amd as mm
from tests.gpu_util import require_gpu, to_dev
from workloads import Grid, random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_binding_rejects_mismatched_buffers():
    case = random_case(91, 1, (6, 5, 7), 500, kind="ecsim")
    sp = case.species[0]
    pos, w, B = (to_dev(a, torch.float64) for a in (sp.pos, sp.w, sp.B))
    bs, perm = mm.bin_particles(case.grid, 1, pos)
    other = Grid((7, 5, 7))
    with pytest.raises(ValueError):
        mm.assemble_ecsim(other, 1, pos, w, B, bs, perm, beta=0.5)  # bin_start of another grid
    with pytest.raises(ValueError):
        mm.assemble_ecsim(case.grid, 1, pos, w, B, bs, perm[:-1], beta=0.5)  # perm short by one
    with pytest.raises(ValueError):
        mm.contract_bins(case.grid, 1, pos, w, B, bs[:-1], perm, beta=0.5)
    with pytest.raises(ValueError):
        mm.bin_particles(case.grid, 1, pos, torch.empty(10, dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError):
        mm.deposit_moments(case.grid, 1, pos, torch.ones(500, 4, dtype=torch.float64, device="cuda"), bs,
                           perm[:100])
    rec_s = mm.contract_bins(case.grid, 1, pos, w, None, bs, perm)  # scalar records
    M9 = torch.empty(case.grid.ncells * 27 * 9, dtype=torch.float64, device="cuda")
    with pytest.raises(ValueError):
        mm.deposit_records(case.grid, 1, rec_s, M9, tensorial=True)  # scalar records read as 3x3
    rec_t = mm.contract_bins(case.grid, 1, pos, w, B, bs, perm)
    big = Grid((6, 5, 9))
    Mb = torch.empty(big.ncells * 27 * 9, dtype=torch.float64, device="cuda")
    with pytest.raises(ValueError):
        mm.deposit_records(big, 1, rec_t, Mb, tensorial=True)  # records of a smaller grid
    with pytest.raises(ValueError):
        mm.deposit_records(big, 1, [rec_t, rec_t], Mb, tensorial=True)
    torch.cuda.synchronize()
    # the matching call still works
    mm.deposit_records(case.grid, 1, rec_t, M9, tensorial=True)
    torch.cuda.synchronize()
    assert np.isfinite(M9.cpu().numpy()).all()
