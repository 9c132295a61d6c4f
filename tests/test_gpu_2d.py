"""GPU parity of the 2D problem (a grid with one node plane, n[2] == 1: z
ignored, (R+1)^2 support, (2R+1)^2 offsets) against the oracle: binning bit
for bit, matrices within the fp64 budget, in fp64 and the mixed layout."""
import numpy as np
import pytest
import torch

import oracle
import particle_grid_mass_amd as mm
from particle_grid_mass_amd import _lib
from tests.gpu_util import rel_fro, require_gpu
from workloads import make_2d, random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dt)


def widen(a, mixed):
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float64) if mixed else a


CASES = [(201, 1, (5, 6, 1), 1), (202, 1, (19, 17, 1), 20000), (203, 2, (5, 7, 1), 37), (204, 2, (23, 19, 1), 20000)]


@pytest.mark.parametrize("mixed", [False, True])
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
@pytest.mark.parametrize("seed,order,n,npart", CASES)
def test_2d_assemble(seed, order, n, npart, kind, mixed):
    case = random_case(seed, order, n, npart, kind=kind, beta=0.7, sigma=1.3, origin=(0.25, -2.0, 1.0),
                       h=(0.5, 1.0, 0.75), spread=0.8)
    sp = case.species[0]
    g = case.grid
    print(f"[case] 2d {kind} order={order} n={n} np={npart} mixed={mixed}", flush=True)
    pdt = torch.float32 if mixed else torch.float64
    pos = dev(sp.pos, pdt)
    bs, perm = mm.bin_particles(g, order, pos, mixed=mixed)
    bs_ref, perm_ref = oracle.bin_particles(order, n, g.origin, g.h, widen(sp.pos, mixed))
    w = dev(sp.w, torch.float64)
    if kind == "ecsim":
        M = mm.assemble_ecsim(g, order, pos, w, dev(sp.B, pdt), bs, perm, beta=sp.beta, sigma=case.sigma)
        ref = oracle.assemble(order, n, g.origin, g.h, widen(sp.pos, mixed), sp.w, widen(sp.B, mixed), sp.beta,
                              case.sigma)
    else:
        M = mm.assemble_scalar(g, order, pos, w, bs, perm, sigma=case.sigma)
        ref = oracle.assemble(order, n, g.origin, g.h, widen(sp.pos, mixed), sp.w, None, 0.0, case.sigma)
    torch.cuda.synchronize()
    assert np.array_equal(bs.cpu().numpy(), bs_ref) and np.array_equal(perm.cpu().numpy(), perm_ref)
    assert M.shape[1] == (2 * order + 1) ** 2
    assert rel_fro(M.cpu().numpy().reshape(ref.shape), ref) <= 1e-12


@pytest.mark.parametrize("order", [1, 2])
def test_2d_two_phase_accumulate_and_size(order):
    """The exported phases on a 256 x 256 grid with 16 particles per cell, twice
    into one M (accumulate)."""
    case = make_2d(256, 16, order, "ecsim", seed=210 + order)
    sp = case.species[0]
    g = case.grid
    print(f"[case] 2d two-phase order={order} np={sp.np}", flush=True)
    pos, w, B = dev(sp.pos, torch.float64), dev(sp.w, torch.float64), dev(sp.B, torch.float64)
    bs, perm = mm.bin_particles(g, order, pos)
    rec = mm.contract_bins(g, order, pos, w, B, bs, perm, sp.beta, case.sigma)
    M = torch.empty(g.ncells * mm.noff_grid(order, g) * 9, dtype=torch.float64, device="cuda")
    mm.deposit_records(g, order, rec, M, True)
    mm.deposit_records(g, order, rec, M, True, accumulate=True)
    torch.cuda.synchronize()
    ref = oracle.assemble(order, g.n, g.origin, g.h, sp.pos, sp.w, sp.B, sp.beta, case.sigma)
    assert rel_fro(M.cpu().numpy().reshape(ref.shape), 2 * ref) <= 1e-12


def test_2d_unsupported_combinations():
    case = random_case(220, 1, (6, 6, 1), 100, kind="ecsim")
    sp = case.species[0]
    g = case.grid
    pos, w, B = dev(sp.pos, torch.float64), dev(sp.w, torch.float64), dev(sp.B, torch.float64)
    bs, perm = mm.bin_particles(g, 1, pos)
    for call in (lambda: mm.assemble_ecsim(g, 1, pos, w, B, None, None, beta=0.5, algo="atomic"),
                 lambda: mm.assemble_ecsim(g, 1, pos, w, B, bs, perm, beta=0.5, algo="mfma_atomic"),
                 lambda: mm.assemble_ecsim(g, 1, pos.float(), w.float(), B.float(), bs, perm, beta=0.5),
                 lambda: mm.deposit_moments(g, 1, pos, w.reshape(-1, 1), bs, perm)):
        with pytest.raises(mm.MMError) as ei:
            call()
        assert ei.value.status == _lib.MM_ERR_UNSUPPORTED
