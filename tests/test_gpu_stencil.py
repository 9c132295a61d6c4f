"""GPU parity of the canonical-half deposit (Sec. 3.4 compact storage) and of
the stencil matrix-vector product (the mass matrix acting on a grid vector in
the field equation, Sec. 2.1), through the C ABI, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import particle_grid_mass_amd as mm
from tests.gpu_util import TOL, TDT, oracle_assemble, rel_fro, require_gpu, to_dev
from workloads import make_config, random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def records_and_M(case, canonical):
    """Contract and deposit every species (full or canonical stencil)."""
    dt = TDT[case.dtype]
    tens = case.kind == "ecsim"
    nc = 9 if tens else 1
    nof = mm.noff_canonical(case.order) if canonical else mm.noff(case.order)
    M = torch.empty(case.grid.ncells * nof * nc, dtype=dt, device="cuda")
    for si, sp in enumerate(case.species):
        pos, w = to_dev(sp.pos, dt), to_dev(sp.w, dt)
        B = to_dev(sp.B, dt) if tens else None
        bs, perm = mm.bin_particles(case.grid, case.order, pos)
        rec = mm.contract_bins(case.grid, case.order, pos, w, B, bs, perm, sp.beta, case.sigma)
        mm.deposit_records(case.grid, case.order, rec, M, tens, accumulate=si > 0, canonical=canonical)
    torch.cuda.synchronize()
    return M.view(case.grid.ncells, nof, nc)


CASES = [(101, 1, (5, 6, 7), 3000), (102, 2, (7, 6, 5), 3000), (103, 2, (9, 8, 7), 20000),
         (104, 2, (8, 7, 6), 20000)]  # run records (x extent a multiple of 4) for fp64 3x3


@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
@pytest.mark.parametrize("seed,order,n,npart", CASES)
def test_canonical_deposit(seed, order, n, npart, kind, dtype):
    case = random_case(seed, order, n, npart, kind=kind, dtype=dtype, beta=0.6, sigma=1.2,
                       origin=(0.25, -2.0, 1.0), h=(0.5, 1.0, 0.75))
    print(f"[case] canonical order={order} n={n} {kind} {dtype}", flush=True)
    Mf = records_and_M(case, False).cpu().numpy()
    Mc = records_and_M(case, True).cpu().numpy()
    c = (mm.noff(order) - 1) // 2
    assert Mc.shape[1] == mm.noff_canonical(order)
    assert np.array_equal(Mc, Mf[:, c:, :])  # the same sums, bit for bit
    ref = oracle.canonical_half(order, oracle_assemble(case))
    assert rel_fro(Mc, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
@pytest.mark.parametrize("seed,order,n,npart", CASES)
def test_stencil_matvec(seed, order, n, npart, kind, dtype):
    case = random_case(seed + 7, order, n, npart, kind=kind, dtype=dtype, beta=0.6,
                       origin=(0.25, -2.0, 1.0), h=(0.5, 1.0, 0.75))
    print(f"[case] matvec order={order} n={n} {kind} {dtype}", flush=True)
    tens = kind == "ecsim"
    nn = case.grid.ncells
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(nn, 3) if tens else nn)
    if dtype == "f32":
        x = x.astype(np.float32)
    Mo = oracle_assemble(case)
    ref = oracle.stencil_matvec(order, case.grid.n, Mo, x.astype(np.float64))
    xd = to_dev(x, TDT[dtype])
    for canonical in (False, True):
        M = records_and_M(case, canonical)
        y = mm.stencil_matvec(case.grid, order, M, xd, tens, canonical=canonical)
        torch.cuda.synchronize()
        assert rel_fro(y.cpu().numpy(), ref) <= TOL[dtype], canonical


def test_canonical_two_species_and_matvec_config3():
    """Two species with the two-species configuration's makeup (125 particles
    per cell, sorted, on 4^3 cells) accumulated into the canonical half, and the
    product from the canonical half against the oracle's from the full M."""
    case = make_config(3, scale=4)
    print(f"[case] canonical two species np={case.np_total}", flush=True)
    Mc = records_and_M(case, True)
    Mo = oracle_assemble(case)
    assert rel_fro(Mc.cpu().numpy(), oracle.canonical_half(1, Mo)) <= 1e-12
    x = np.random.default_rng(3).normal(size=(case.grid.ncells, 3))
    y = mm.stencil_matvec(case.grid, 1, Mc, to_dev(x, torch.float64), True, canonical=True)
    torch.cuda.synchronize()
    assert rel_fro(y.cpu().numpy(), oracle.stencil_matvec(1, case.grid.n, Mo, x)) <= 1e-12


def test_matvec_config2_full():
    case = make_config(2)
    print("[case] matvec config 2", flush=True)
    M = records_and_M(case, False)
    Mc = records_and_M(case, True)
    x = np.random.default_rng(4).normal(size=(case.grid.ncells, 3))
    xd = to_dev(x, torch.float64)
    y = mm.stencil_matvec(case.grid, 1, M, xd, True)
    yc = mm.stencil_matvec(case.grid, 1, Mc, xd, True, canonical=True)
    torch.cuda.synchronize()
    ref = oracle.stencil_matvec(1, case.grid.n, oracle_assemble(case), x)
    assert rel_fro(y.cpu().numpy(), ref) <= 1e-12
    assert rel_fro(yc.cpu().numpy(), ref) <= 1e-12
