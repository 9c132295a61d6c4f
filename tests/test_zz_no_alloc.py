"""The allocation-free entry point (mm_assemble_ecsim_noalloc) against the
entry point it varies (mm_assemble_ecsim with the matrix-core algorithm),
called through the C ABI: two calls in a row on one GPU, the second with a
smaller input, each equal to the workspace entry point's result and within
the fp64 / fp32 budget of the oracle. The records of the second call overwrite
the fixed scratch left by the first."""
import numpy as np
import pytest
import torch

import particle_grid_mass_amd as mm
from particle_grid_mass_amd import _lib
from tests.gpu_util import TDT, as_numpy_M, assert_match, oracle_assemble, require_gpu, to_dev
from workloads import Grid, random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _both(case):
    dt = TDT[case.dtype]
    sp = case.species[0]
    pos, w, B = to_dev(sp.pos, dt), to_dev(sp.w, dt), to_dev(sp.B, dt)
    bs, perm = mm.bin_particles(case.grid, case.order, pos)
    ref = mm.assemble_ecsim(case.grid, case.order, pos, w, B, bs, perm, beta=sp.beta, sigma=case.sigma)
    # the output buffer is filled with garbage first: the call must overwrite all of it
    M = torch.full_like(ref, float("nan"))
    got = mm.assemble_ecsim_noalloc(case.grid, case.order, pos, w, B, bs, perm, beta=sp.beta, sigma=case.sigma, M=M)
    torch.cuda.synchronize()
    return got, ref


@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("order", [1, 2])
def test_noalloc_matches_workspace_entry_point(order, dtype):
    big = random_case(401 + order, order, (12, 10, 9) if order == 1 else (9, 8, 10), 30000, kind="ecsim",
                      dtype=dtype, beta=0.7, sigma=1.3, origin=(0.25, -2.0, 1.0), h=(0.5, 1.0, 0.75))
    small = random_case(411 + order, order, (7, 6, 5), 3000, kind="ecsim", dtype=dtype, beta=-0.4, sigma=0.9)
    for case in (big, small):  # two calls in a row, the second smaller
        print(f"[case] noalloc {case.name} order={order} {dtype} n={case.grid.n} np={case.np_total}", flush=True)
        got, ref = _both(case)
        assert torch.equal(got, ref), "allocation-free call differs from the workspace entry point"
        assert_match(as_numpy_M(got, case), oracle_assemble(case), dtype)


def test_noalloc_accumulate_and_empty():
    case = random_case(421, 1, (6, 5, 7), 2000, kind="ecsim")
    sp = case.species[0]
    pos, w, B = (to_dev(a, torch.float64) for a in (sp.pos, sp.w, sp.B))
    bs, perm = mm.bin_particles(case.grid, 1, pos)
    M = mm.assemble_ecsim_noalloc(case.grid, 1, pos, w, B, bs, perm, beta=sp.beta)
    M = mm.assemble_ecsim_noalloc(case.grid, 1, pos, w, B, bs, perm, beta=sp.beta, M=M, accumulate=True)
    ref = mm.assemble_ecsim(case.grid, 1, pos, w, B, bs, perm, beta=sp.beta)
    ref = mm.assemble_ecsim(case.grid, 1, pos, w, B, bs, perm, beta=sp.beta, M=ref, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(M, ref)
    e3 = torch.zeros((0, 3), dtype=torch.float64, device="cuda")
    e1 = torch.zeros((0,), dtype=torch.float64, device="cuda")
    ebs, eperm = mm.bin_particles(case.grid, 1, e3)
    M0 = mm.assemble_ecsim_noalloc(case.grid, 1, e3, e1, e3, ebs, eperm, beta=0.5, M=M.clone())
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(M0)) == 0


def test_noalloc_rejects_workloads_beyond_its_scratch():
    g = Grid((40, 40, 40))  # CIC 3x3 fp64 records: 64,000 bins x 2592 B > 64 MiB
    pos = torch.zeros((4, 3), dtype=torch.float64, device="cuda")
    w = torch.ones(4, dtype=torch.float64, device="cuda")
    bs = torch.zeros(g.ncells + 1, dtype=torch.int32, device="cuda")
    perm = torch.zeros(4, dtype=torch.int32, device="cuda")
    M = torch.empty((g.ncells, 27, 9), dtype=torch.float64, device="cuda")
    with pytest.raises(mm.MMError) as ei:
        mm.assemble_ecsim_noalloc(g, 1, pos, w, pos, bs, perm, beta=0.5, M=M)
    assert ei.value.status == _lib.MM_ERR_SCRATCH
