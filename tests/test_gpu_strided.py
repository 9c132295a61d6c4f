"""GPU parity of strided particle arrays (the *_strided entry points).

The pages state the problem per particle (position, weight, field; Pennati &
Markidis, Sec. 2.1 Eq. 6) and leave the storage open. The strided entry
points read the three arrays with any element stride, e.g. one record of
position, weight and field per particle. Binning must match the oracle bit
for bit, matrices the oracle to the fp64 budget, and both must be bit for bit
what the dense arrays give, since only the addressing differs.

Storage columns that no array covers hold NaN, so that a read of a wrong
element shows in the result.
"""
import numpy as np
import pytest
import torch

import oracle
import particle_grid_mass_amd as mm
from tests.gpu_util import as_numpy_M, assert_match, oracle_assemble, require_gpu, to_dev
from tests.test_gpu_edges import edge_case
from workloads import make_config, random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


# name: (columns per record, first column of pos, of w, of B) for one shared
# storage, or None for three storages of their own strides
LAYOUTS = {
    "record8": (8, 0, 3, 4),    # x y z w Bx By Bz and one unused value: 64 bytes
    "record11": (11, 5, 1, 8),  # interleaved with values the assembly does not read
    "apart": None,              # pos every 5, w every 2, B every 4 doubles, three storages
}


def strided_views(sp, layout):
    """(pos, w, B) device views of storage laid out as `layout` (float64)."""
    n = sp.pos.shape[0]
    spec = LAYOUTS[layout]
    if spec is None:
        sp_pos, sp_w, sp_B = np.full((n, 5), np.nan), np.full((n, 2), np.nan), np.full((n, 4), np.nan)
        sp_pos[:, 1:4], sp_w[:, 1], sp_B[:, 0:3] = sp.pos, sp.w, sp.B
        P, W, Bt = (to_dev(a, torch.float64) for a in (sp_pos, sp_w, sp_B))
        return P[:, 1:4], W[:, 1], Bt[:, 0:3]
    cols, cp, cw, cb = spec
    rec = np.full((n, cols), np.nan)
    rec[:, cp:cp + 3], rec[:, cw], rec[:, cb:cb + 3] = sp.pos, sp.w, sp.B
    R = to_dev(rec, torch.float64)
    return R[:, cp:cp + 3], R[:, cw], R[:, cb:cb + 3]


def dense(sp):
    return to_dev(sp.pos, torch.float64), to_dev(sp.w, torch.float64), to_dev(sp.B, torch.float64)


def assemble(case, views_of, algo="mfma"):
    M = None
    for si, sp in enumerate(case.species):
        pos, w, B = views_of(sp)
        bs, perm = mm.bin_particles(case.grid, case.order, pos)
        M = mm.assemble_ecsim(case.grid, case.order, pos, w, B, bs, perm, beta=sp.beta, sigma=case.sigma, M=M,
                              accumulate=si > 0, algo=algo)
    torch.cuda.synchronize()
    return M


def check_bins(case, pos_view, order):
    sp = case.species[0]
    bs_ref, perm_ref = oracle.bin_particles(order, case.grid.n, case.grid.origin, case.grid.h, sp.pos)
    bs, perm = mm.bin_particles(case.grid, order, pos_view)
    torch.cuda.synchronize()
    assert np.array_equal(bs.cpu().numpy(), bs_ref)
    assert np.array_equal(perm.cpu().numpy(), perm_ref)


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("seed,n,npart,srt", [(1, (5, 6, 7), 1, False), (2, (9, 8, 7), 5000, False),
                                             (3, (9, 8, 7), 5000, True), (4, (40, 33, 17), 300000, False)])
def test_strided_binning(seed, n, npart, srt, order, layout):
    """Positions read through a stride: the same bins as the oracle on the
    dense positions (key-ordered input takes the kernels' short cut)."""
    case = random_case(seed, order, n, npart, kind="ecsim", sorted_by_cell=srt, origin=(-1.5, 0.25, 3.0),
                       h=(0.5, 0.75, 1.25))
    print(f"[case] strided binning {layout} order={order} n={n} np={npart} sorted={srt}", flush=True)
    pos, _, _ = strided_views(case.species[0], layout)
    assert not pos.is_contiguous() or npart <= 1
    check_bins(case, pos, order)


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("spacing", ["pow2", "dyadic", "inexact"])
@pytest.mark.parametrize("order", [1, 2])
def test_strided_edge_binning(order, spacing, layout):
    case = edge_case(300 + order, order, "ecsim", "f64", spacing)
    print(f"[case] strided edge binning {case.name} {layout}", flush=True)
    check_bins(case, strided_views(case.species[0], layout)[0], order)


SMALL = [
    # seed, n, npart
    (11, (5, 6, 7), 1),
    (12, (5, 6, 7), 37),
    (13, (9, 8, 7), 20000),
    (14, (16, 12, 10), 120000),
]


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("seed,n,npart", SMALL)
def test_strided_assembly(seed, n, npart, layout):
    case = random_case(seed, 1, n, npart, kind="ecsim", beta=0.7, sigma=1.3, origin=(0.25, -2.0, 1.0),
                       h=(0.5, 1.0, 0.75), spread=0.8)
    print(f"[case] strided assembly {layout} n={n} np={npart}", flush=True)
    M = assemble(case, lambda sp: strided_views(sp, layout))
    assert_match(as_numpy_M(M, case), oracle_assemble(case), "f64")
    Md = assemble(case, dense)
    assert torch.equal(M, Md)


SMALL2 = [
    # seed, n, npart: an x extent of 8 or 12 gives run records, 7 per-bin records
    (51, (8, 6, 5), 3),
    (52, (7, 6, 5), 1500),
    (53, (12, 7, 6), 20000),
    (54, (9, 8, 7), 20000),
]


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("seed,n,npart", SMALL2)
def test_strided_assembly_tsc(seed, n, npart, layout):
    """Second order: the fp64 TSC contraction reads the strides (run records
    and per-bin records), matching the oracle and the dense path bit for bit."""
    case = random_case(seed, 2, n, npart, kind="ecsim", beta=0.7, sigma=1.3, origin=(0.25, -2.0, 1.0),
                       h=(0.5, 1.0, 0.75), spread=0.8)
    print(f"[case] strided TSC assembly {layout} n={n} np={npart}", flush=True)
    M = assemble(case, lambda sp: strided_views(sp, layout))
    assert_match(as_numpy_M(M, case), oracle_assemble(case), "f64")
    Md = assemble(case, dense)
    assert torch.equal(M, Md)


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("n", [(8, 6, 8), (7, 6, 8)])
def test_strided_edge_assembly_tsc(n, layout):
    """Particles on nodes, at the TSC tie and on the periodic boundary."""
    case = edge_case(410, 2, "ecsim", "f64", "dyadic", n=n)
    print(f"[case] strided TSC edge assembly {case.name} n={n} {layout}", flush=True)
    M = assemble(case, lambda sp: strided_views(sp, layout))
    assert_match(as_numpy_M(M, case), oracle_assemble(case), "f64")


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("spacing", ["pow2", "dyadic", "inexact"])
def test_strided_edge_assembly(spacing, layout):
    """Particles on nodes, faces and the periodic boundary, several periods out."""
    case = edge_case(400, 1, "ecsim", "f64", spacing)
    print(f"[case] strided edge assembly {case.name} {layout}", flush=True)
    M = assemble(case, lambda sp: strided_views(sp, layout))
    assert_match(as_numpy_M(M, case), oracle_assemble(case), "f64")


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_strided_records_bitwise(layout):
    """The two phases: the records of the strided views equal the dense ones
    bit for bit, and their deposit matches the oracle."""
    case = random_case(21, 1, (12, 10, 9), 30000, kind="ecsim", beta=0.4, sigma=0.9)
    sp = case.species[0]
    print(f"[case] strided records {layout}", flush=True)
    pos, w, B = strided_views(sp, layout)
    bs, perm = mm.bin_particles(case.grid, 1, pos)
    rec = mm.contract_bins(case.grid, 1, pos, w, B, bs, perm, sp.beta, case.sigma)
    pd, wd, Bd = dense(sp)
    rec_d = mm.contract_bins(case.grid, 1, pd, wd, Bd, bs, perm, sp.beta, case.sigma)
    M = torch.empty(case.grid.ncells * 27 * 9, dtype=torch.float64, device="cuda")
    mm.deposit_records(case.grid, 1, rec, M, True)
    torch.cuda.synchronize()
    assert torch.equal(rec, rec_d)
    assert_match(as_numpy_M(M, case), oracle_assemble(case), "f64")
    # second order, run records
    case2 = random_case(22, 2, (12, 10, 9), 30000, kind="ecsim", beta=0.4, sigma=0.9)
    sp2 = case2.species[0]
    pos, w, B = strided_views(sp2, layout)
    bs, perm = mm.bin_particles(case2.grid, 2, pos)
    nrec = mm.record_bytes(case2.grid, 2, torch.float64, True)
    # zero-filled buffers: the padding slots of run records are never written
    rec = mm.contract_bins(case2.grid, 2, pos, w, B, bs, perm, sp2.beta, case2.sigma,
                           rec=torch.zeros(nrec, dtype=torch.uint8, device="cuda"))
    pd, wd, Bd = dense(sp2)
    rec_d = mm.contract_bins(case2.grid, 2, pd, wd, Bd, bs, perm, sp2.beta, case2.sigma,
                             rec=torch.zeros(nrec, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(rec, rec_d)


def test_strided_two_species_and_empty():
    """Two species accumulated into one M, and a species without particles."""
    case = make_config(2, scale=12)  # 12^3 cells, 64 per cell
    other = random_case(31, 1, case.grid.n, 5000, kind="ecsim", beta=-0.3).species[0]
    case.species.append(other)
    print("[case] strided two species", flush=True)
    M = assemble(case, lambda sp: strided_views(sp, "record8"))
    assert_match(as_numpy_M(M, case), oracle_assemble(case), "f64")
    empty = torch.empty((0, 8), dtype=torch.float64, device="cuda")
    bs, perm = mm.bin_particles(case.grid, 1, empty[:, 0:3])
    M0 = mm.assemble_ecsim(case.grid, 1, empty[:, 0:3], empty[:, 3], empty[:, 4:7], bs, perm, beta=0.5)
    M1 = mm.assemble_ecsim(case.grid, 1, empty[:, 0:3], empty[:, 3], empty[:, 4:7], bs, perm, beta=0.5, M=M.clone(),
                           accumulate=True)
    torch.cuda.synchronize()
    assert int(bs.abs().sum()) == 0 and float(M0.abs().max()) == 0.0
    assert torch.equal(M1, M)


def test_strided_config3_shuffled():
    """Config 3 (64^3 cells, 125 per cell, two species) in shuffled order,
    each species one 64-byte record per particle."""
    case = make_config(3, shuffled=True)
    print(f"[case] strided c3 shuffled np={case.np_total}", flush=True)
    M = assemble(case, lambda sp: strided_views(sp, "record8"))
    assert_match(as_numpy_M(M, case), oracle_assemble(case), "f64")
    sp = case.species[0]
    bs, perm = mm.bin_particles(case.grid, 1, strided_views(sp, "record8")[0])
    bs_ref, perm_ref = oracle.bin_particles(1, case.grid.n, case.grid.origin, case.grid.h, sp.pos)
    assert np.array_equal(bs.cpu().numpy(), bs_ref)
    assert np.array_equal(perm.cpu().numpy(), perm_ref)
    del M
    Md = assemble(case, dense)
    M = assemble(case, lambda sp: strided_views(sp, "record8"))
    assert torch.equal(M, Md)


def test_strided_unsupported():
    """Strides reach the fp64 matrix-core path only; fp32 storage must be dense."""
    case = random_case(41, 2, (8, 6, 5), 100, kind="ecsim")
    sp = case.species[0]
    pos, w, B = strided_views(sp, "record8")
    bs, perm = mm.bin_particles(case.grid, 2, pos)
    with pytest.raises(mm.MMError):
        mm.assemble_ecsim(case.grid, 2, pos, w, B, bs, perm, beta=0.5, algo="atomic")
    case1 = random_case(42, 1, (8, 6, 5), 100, kind="ecsim")
    pos, w, B = strided_views(case1.species[0], "record8")
    bs, perm = mm.bin_particles(case1.grid, 1, pos)
    for algo in ("mfma_atomic", "atomic", "valu"):
        with pytest.raises(mm.MMError):
            mm.assemble_ecsim(case1.grid, 1, pos, w, B, bs, perm, beta=0.5, algo=algo)
    rec32 = torch.zeros((100, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        mm.bin_particles(case1.grid, 1, rec32[:, 0:3])
    torch.cuda.synchronize()
