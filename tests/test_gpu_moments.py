"""GPU parity of the moment deposition (m[g][k] = sum_p W_pg Q_p[k]: charge,
current and higher moments on the matrix cores) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import particle_grid_mass_amd as mm
from tests.gpu_util import TOL, TDT, rel_fro, require_gpu, to_dev
from workloads import make_config, random_case, Grid

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def quantities(seed, npart, nq, dtype):
    Q = np.random.default_rng(seed).normal(size=(npart, nq))
    return Q.astype(np.float32) if dtype == "f32" else Q


def gpu_moments(grid, order, pos, Q, dtype, m=None, accumulate=False):
    dt = TDT[dtype]
    p = to_dev(pos, dt)
    bs, perm = mm.bin_particles(grid, order, p)
    out = mm.deposit_moments(grid, order, p, to_dev(Q, dt), bs, perm, m=m, accumulate=accumulate)
    torch.cuda.synchronize()
    return out


CASES = [(131, 1, (5, 6, 7), 1), (132, 1, (9, 8, 7), 20000), (133, 2, (5, 6, 7), 37), (134, 2, (9, 8, 7), 20000)]


@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("nq", [1, 4, 10, 16])
@pytest.mark.parametrize("seed,order,n,npart", CASES)
def test_moments_small(seed, order, n, npart, nq, dtype):
    case = random_case(seed, order, n, npart, kind="scalar", dtype=dtype, origin=(0.25, -2.0, 1.0),
                       h=(0.5, 1.0, 0.75), spread=0.8)
    pos = case.species[0].pos
    Q = quantities(seed, npart, nq, dtype)
    print(f"[case] moments order={order} n={n} np={npart} nq={nq} {dtype}", flush=True)
    got = gpu_moments(case.grid, order, pos, Q, dtype).double().cpu().numpy()
    ref = oracle.moments(order, n, case.grid.origin, case.grid.h, pos, Q)
    assert rel_fro(got, ref) <= TOL[dtype]


@pytest.mark.parametrize("order", [1, 2])
def test_moments_accumulate_empty_heavy_deterministic(order):
    """One bin of 5000 particles; accumulate adds; np = 0 zeroes or keeps;
    two runs agree bit for bit."""
    rng = np.random.default_rng(140 + order)
    pos = np.array([3.0, 2.0, 4.0]) + rng.random((5000, 3))
    grid = Grid((6, 6, 7))
    Q = quantities(7, 5000, 4, "f64")
    m1 = gpu_moments(grid, order, pos, Q, "f64")
    m2 = gpu_moments(grid, order, pos, Q, "f64")
    assert torch.equal(m1, m2)
    ref = oracle.moments(order, grid.n, grid.origin, grid.h, pos, Q)
    assert rel_fro(m1.cpu().numpy(), ref) <= 1e-12
    m3 = gpu_moments(grid, order, pos, Q, "f64", m=m1.clone(), accumulate=True)
    assert rel_fro(m3.cpu().numpy(), 2 * ref) <= 1e-12
    e3 = torch.zeros((0, 3), dtype=torch.float64, device="cuda")
    eq = torch.zeros((0, 4), dtype=torch.float64, device="cuda")
    bs, perm = mm.bin_particles(grid, order, e3)
    keep = mm.deposit_moments(grid, order, e3, eq, bs, perm, m=m1.clone(), accumulate=True)
    zero = mm.deposit_moments(grid, order, e3, eq, bs, perm, m=m1.clone(), accumulate=False)
    torch.cuda.synchronize()
    assert torch.equal(keep, m1) and int(torch.count_nonzero(zero)) == 0


@pytest.mark.parametrize("cid,kind,nq", [(2, None, 4), (4, "ecsim", 10)])
def test_moments_config_full(cid, kind, nq):
    """Charge and current (q, q v) on config 2, ten moments on config 4."""
    case = make_config(cid, kind=kind)
    sp = case.species[0]
    rng = np.random.default_rng(cid)
    v = rng.normal(size=(sp.np, 3))
    q = sp.w[:, None]
    cols = [q, q * v]
    if nq == 10:
        cols.append(np.stack([q[:, 0] * v[:, i] * v[:, j] for i in range(3) for j in range(i, 3)], axis=1))
    Q = np.ascontiguousarray(np.concatenate(cols, axis=1))
    assert Q.shape[1] == nq
    print(f"[case] moments config {cid} nq={nq}", flush=True)
    got = gpu_moments(case.grid, case.order, sp.pos, Q, "f64").cpu().numpy()
    ref = oracle.moments(case.order, case.grid.n, case.grid.origin, case.grid.h, sp.pos, Q)
    assert rel_fro(got, ref) <= 1e-12
