"""GPU parity of the mixed production layout (Sec. 5, "Exactness and
precision": positions and fields stored in fp32; weights, quantities and the
matrix in fp64; every step in fp64 on the fp32 values read exactly). The
oracle takes the same fp32 values widened to fp64, so the fp64 budget of
1e-12 applies and the binning must match bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import particle_grid_mass_amd as mm
from particle_grid_mass_amd import _lib
from tests.gpu_util import as_numpy_M, rel_fro, require_gpu
from workloads import make_config, random_case, grid_field

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def d32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def d64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).cuda()


def widen(a):
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float64)


CASES = [(151, 1, (5, 6, 7), 37), (152, 1, (9, 8, 7), 20000), (153, 2, (7, 6, 5), 1500), (154, 2, (9, 8, 7), 20000),
         (155, 2, (8, 7, 6), 20000)]  # run records (x extent a multiple of 4)


@pytest.mark.parametrize("algo", ["mfma", "mfma_atomic"])
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
@pytest.mark.parametrize("seed,order,n,npart", CASES)
def test_mixed_assemble(seed, order, n, npart, kind, algo):
    case = random_case(seed, order, n, npart, kind=kind, beta=0.7, sigma=1.3, origin=(0.25, -2.0, 1.0),
                       h=(0.5, 1.0, 0.75), spread=0.8)
    sp = case.species[0]
    print(f"[case] mixed {kind}/{algo} order={order} n={n} np={npart}", flush=True)
    pos32 = d32(sp.pos)
    bs, perm = mm.bin_particles(case.grid, order, pos32, mixed=True)
    bs_ref, perm_ref = oracle.bin_particles(order, n, case.grid.origin, case.grid.h, widen(sp.pos))
    torch.cuda.synchronize()
    assert np.array_equal(bs.cpu().numpy(), bs_ref) and np.array_equal(perm.cpu().numpy(), perm_ref)
    w = d64(sp.w)
    if kind == "ecsim":
        M = mm.assemble_ecsim(case.grid, order, pos32, w, d32(sp.B), bs, perm, beta=sp.beta, sigma=case.sigma,
                              algo=algo)
        ref = oracle.assemble(order, n, case.grid.origin, case.grid.h, widen(sp.pos), sp.w, widen(sp.B), sp.beta,
                              case.sigma)
    else:
        M = mm.assemble_scalar(case.grid, order, pos32, w, bs, perm, sigma=case.sigma, algo=algo)
        ref = oracle.assemble(order, n, case.grid.origin, case.grid.h, widen(sp.pos), sp.w, None, 0.0, case.sigma)
    torch.cuda.synchronize()
    assert M.dtype == torch.float64
    assert rel_fro(as_numpy_M(M, case), ref) <= 1e-12


@pytest.mark.parametrize("order", [1, 2])
def test_mixed_grid_field_and_moments(order):
    case = random_case(160 + order, order, (9, 8, 7), 20000, kind="ecsim", beta=0.5)
    sp = case.species[0]
    g = case.grid
    F = grid_field(g, 160 + order)
    pos32 = d32(sp.pos)
    bs, perm = mm.bin_particles(g, order, pos32, mixed=True)
    M = mm.assemble_ecsim_gridB(g, order, pos32, d64(sp.w), d32(F), bs, perm, beta=sp.beta)
    Bp = oracle.interp_field(order, g.n, g.origin, g.h, widen(sp.pos), widen(F))
    ref = oracle.assemble(order, g.n, g.origin, g.h, widen(sp.pos), sp.w, Bp, sp.beta, 1.0)
    Q = np.random.default_rng(order).normal(size=(sp.np, 4))
    m = mm.deposit_moments(g, order, pos32, d64(Q), bs, perm)
    torch.cuda.synchronize()
    assert rel_fro(as_numpy_M(M, case), ref) <= 1e-12
    assert rel_fro(m.cpu().numpy(), oracle.moments(order, g.n, g.origin, g.h, widen(sp.pos), Q)) <= 1e-12


def test_mixed_atomic_is_unsupported():
    case = random_case(170, 1, (5, 5, 5), 100, kind="ecsim")
    sp = case.species[0]
    with pytest.raises(mm.MMError) as ei:
        mm.assemble_ecsim(case.grid, 1, d32(sp.pos), d64(sp.w), d32(sp.B), None, None, beta=0.5, algo="atomic")
    assert ei.value.status == _lib.MM_ERR_UNSUPPORTED


def test_mixed_config2_full():
    case = make_config(2)
    sp = case.species[0]
    print("[case] mixed config 2", flush=True)
    pos32 = d32(sp.pos)
    bs, perm = mm.bin_particles(case.grid, 1, pos32, mixed=True)
    M = mm.assemble_ecsim(case.grid, 1, pos32, d64(sp.w), d32(sp.B), bs, perm, beta=sp.beta)
    torch.cuda.synchronize()
    ref = oracle.assemble(1, case.grid.n, case.grid.origin, case.grid.h, widen(sp.pos), sp.w, widen(sp.B), sp.beta,
                          case.sigma)
    assert rel_fro(as_numpy_M(M, case), ref) <= 1e-12
