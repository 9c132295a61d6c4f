"""GPU parity of the assembly with the magnetic field on the grid nodes: each
particle's field is gathered with its own support weights before its response
tensor is formed (fused into the fp64 matrix-core contraction; interpolated
to the particles first on the other paths). The oracle gathers the field in
fp64 (oracle.interp_field) and assembles with it; matrices must agree within
the relative Frobenius budget (1e-12 fp64, 1e-5 fp32)."""
import numpy as np
import pytest
import torch

import oracle
import particle_grid_mass_amd as mm
from tests.gpu_util import TOL, TDT, as_numpy_M, rel_fro, require_gpu, species_scalars, to_dev
from workloads import make_config, random_case, grid_field, Case, Species, Grid

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def oracle_gridB(case, F):
    M = None
    for si, sp in enumerate(case.species):
        beta, sigma = species_scalars(case, sp)
        Bp = oracle.interp_field(case.order, case.grid.n, case.grid.origin, case.grid.h, sp.pos, F)
        M = oracle.assemble(case.order, case.grid.n, case.grid.origin, case.grid.h, sp.pos, sp.w, Bp, beta, sigma,
                            M=M, accumulate=si > 0)
    return M


def gpu_gridB(case, F, algo="mfma", two_phase=False):
    dt = TDT[case.dtype]
    Fd = to_dev(F, dt)
    M = None
    for si, sp in enumerate(case.species):
        pos, w = to_dev(sp.pos, dt), to_dev(sp.w, dt)
        bs = perm = None
        if algo != "atomic":
            bs, perm = mm.bin_particles(case.grid, case.order, pos)
        if two_phase:
            if M is None:
                M = torch.empty(case.grid.ncells * mm.noff(case.order) * 9, dtype=dt, device="cuda")
            rec = mm.contract_bins(case.grid, case.order, pos, w, None, bs, perm, sp.beta, case.sigma, Bgrid=Fd)
            mm.deposit_records(case.grid, case.order, rec, M, True, accumulate=si > 0)
        else:
            M = mm.assemble_ecsim_gridB(case.grid, case.order, pos, w, Fd, bs, perm, beta=sp.beta, sigma=case.sigma,
                                        M=M, accumulate=si > 0, algo=algo)
    torch.cuda.synchronize()
    return as_numpy_M(M, case)


SMALL = [
    # seed, order, n, npart
    (51, 1, (5, 6, 7), 1),
    (52, 1, (5, 6, 7), 37),
    (53, 1, (9, 8, 7), 20000),
    (54, 2, (5, 6, 7), 3),
    (55, 2, (7, 6, 5), 1500),
    (56, 2, (9, 8, 7), 20000),
    (57, 2, (8, 6, 7), 15000),  # run records (x extent a multiple of 4) for fp64
    (58, 2, (12, 5, 5), 7),
]


@pytest.mark.parametrize("algo", ["mfma", "mfma_atomic", "atomic"])
@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("seed,order,n,npart", SMALL)
def test_gridB_small(seed, order, n, npart, dtype, algo):
    case = random_case(seed, order, n, npart, kind="ecsim", dtype=dtype, beta=0.7, sigma=1.3,
                       origin=(0.25, -2.0, 1.0), h=(0.5, 1.0, 0.75), spread=0.8)
    F = grid_field(case.grid, seed, dtype)
    print(f"[case] gridB/{algo} order={order} n={n} np={npart} {dtype}", flush=True)
    assert rel_fro(gpu_gridB(case, F, algo), oracle_gridB(case, F)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("order", [1, 2])
def test_gridB_two_phase_and_heavy_bin(order, dtype):
    """The two exported phases with the grid field, on one bin of 5000 particles
    plus a sparse remainder (many chunks, empty bins, ragged groups)."""
    rng = np.random.default_rng(60 + order)
    pos = np.concatenate([np.array([3.0, 2.0, 4.0]) + rng.random((5000, 3)), rng.random((700, 3)) * [6, 6, 7]])
    w = rng.uniform(0.5, 1.5, len(pos))
    cast = (lambda a: a.astype(np.float32)) if dtype == "f32" else (lambda a: a)
    case = Case("heavy-gridB", Grid((6, 6, 7)), order, "ecsim", [Species(cast(pos), cast(w), None, 0.5)], dtype=dtype)
    F = grid_field(case.grid, 3, dtype)
    print(f"[case] gridB two-phase order={order} {dtype}", flush=True)
    assert rel_fro(gpu_gridB(case, F, two_phase=True), oracle_gridB(case, F)) <= TOL[dtype]


def test_gridB_equals_per_particle_path():
    """Gathering on the device equals passing the oracle's gathered field per
    particle, and a constant grid field equals that constant per particle."""
    case = random_case(71, 2, (8, 7, 9), 30000, kind="ecsim", beta=0.4)
    sp = case.species[0]
    F = grid_field(case.grid, 71)
    Bp = oracle.interp_field(2, case.grid.n, case.grid.origin, case.grid.h, sp.pos, F)
    pos, w = to_dev(sp.pos, torch.float64), to_dev(sp.w, torch.float64)
    bs, perm = mm.bin_particles(case.grid, 2, pos)
    Mg = mm.assemble_ecsim_gridB(case.grid, 2, pos, w, to_dev(F, torch.float64), bs, perm, beta=sp.beta)
    Mp = mm.assemble_ecsim(case.grid, 2, pos, w, to_dev(Bp, torch.float64), bs, perm, beta=sp.beta)
    c = np.array([0.3, -1.2, 0.8])
    Mc = mm.assemble_ecsim_gridB(case.grid, 2, pos, w, to_dev(np.tile(c, (case.grid.ncells, 1)), torch.float64),
                                 bs, perm, beta=sp.beta)
    Mcp = mm.assemble_ecsim(case.grid, 2, pos, w, to_dev(np.tile(c, (sp.np, 1)), torch.float64), bs, perm,
                            beta=sp.beta)
    torch.cuda.synchronize()
    assert rel_fro(Mg.cpu().numpy(), Mp.cpu().numpy()) <= 1e-13
    assert rel_fro(Mc.cpu().numpy(), Mcp.cpu().numpy()) <= 1e-13


@pytest.mark.parametrize("cid,kind", [(2, None), (4, "ecsim")])
def test_gridB_config_full(cid, kind):
    case = make_config(cid, kind=kind)
    F = grid_field(case.grid, 1000 + cid)
    print(f"[case] gridB config {cid} full", flush=True)
    assert rel_fro(gpu_gridB(case, F), oracle_gridB(case, F)) <= 1e-12
