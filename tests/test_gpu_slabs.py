"""Slabs of planes: the plane-range contraction and deposition of run records,
and the assembly that overlaps the two phases by slabs.

The split by planes changes only which launch computes a record or a
stencil entry, never the kernels' arithmetic or order of summation: every
result is compared bit for bit with the unsplit two-phase path, which the
other parity tests compare with the oracle; the overlapped assembly is also
checked against the oracle directly on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import particle_grid_mass_amd as mm
from tests.gpu_util import assert_match, species_scalars
from workloads import grid_field, random_case

pytestmark = pytest.mark.gpu

RUNREC = 9360  # values per run record (999 union entries of 9 components, planes padded to 16)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"


def _dev(case, sp, mode):
    """Device arrays of one species: (pos, w, B) in the storage of `mode`
    (f64, f32, or mix: fp32 positions and field, fp64 weights)."""
    pdt = torch.float64 if mode == "f64" else torch.float32
    wdt = torch.float32 if mode == "f32" else torch.float64
    pos = torch.from_numpy(np.ascontiguousarray(sp.pos)).to("cuda", pdt)
    w = torch.from_numpy(np.ascontiguousarray(sp.w)).to("cuda", wdt)
    B = torch.from_numpy(np.ascontiguousarray(sp.B)).to("cuda", pdt)
    return pos, w, B


def _case(seed, n, npart, mode, spread=1.0):
    case = random_case(seed, 2, n, npart, kind="ecsim", dtype="f32" if mode == "f32" else "f64", spread=spread)
    if mode == "mix":  # the stored fp32 values, seen by the oracle in fp64
        for sp in case.species:
            sp.pos = sp.pos.astype(np.float32).astype(np.float64)
            sp.B = sp.B.astype(np.float32).astype(np.float64)
    return case


def _print(tag, case, mode):
    print(f"[slabs] {tag} grid={case.grid.n} np={case.np_total} mode={mode}", flush=True)


PARTS = {7: [(0, 3), (3, 5), (5, 5), (5, 7)], 10: [(0, 1), (1, 4), (4, 9), (9, 10)]}


@pytest.mark.parametrize("mode", ["f64", "f32", "mix"])
@pytest.mark.parametrize("n,npart", [((12, 5, 7), 9000), ((16, 12, 10), 30000)])
def test_contract_planes_bit_identical(n, npart, mode):
    """Records written plane range by plane range (odd and even ranges, an
    empty one) deposit to the same M as the records of one contraction, and a
    range writes only its own runs' records."""
    case = _case(41, n, npart, mode)
    _print("contract planes", case, mode)
    sp = case.species[0]
    beta, sigma = species_scalars(case, sp)
    pos, w, B = _dev(case, sp, mode)
    bs, perm = mm.bin_particles(case.grid, 2, pos, mixed=mode == "mix")
    rec = mm.contract_bins(case.grid, 2, pos, w, B, bs, perm, beta, sigma)
    mdt = torch.float32 if mode == "f32" else torch.float64
    nn = case.grid.ncells
    M_full = torch.empty(nn * 125 * 9, dtype=mdt, device="cuda")
    mm.deposit_records(case.grid, 2, rec, M_full, True)
    rec_p = torch.full_like(rec, 0x5A)
    for z0, z1 in PARTS[n[2]]:
        mm.contract_bins_planes(case.grid, 2, pos, w, B, bs, perm, beta, sigma, z0, z1, rec_p)
    M_p = torch.full_like(M_full, float("nan"))
    mm.deposit_records(case.grid, 2, rec_p, M_p, True)
    torch.cuda.synchronize()
    assert torch.equal(M_p, M_full)
    # one range leaves every other run's record untouched
    esz = 4 if mode == "f32" else 8
    runs_per_plane = (n[0] // 4) * n[1]
    lo, hi = 2 * runs_per_plane * RUNREC * esz, 4 * runs_per_plane * RUNREC * esz
    rec_q = torch.full_like(rec, 0x5A)
    mm.contract_bins_planes(case.grid, 2, pos, w, B, bs, perm, beta, sigma, 2, 4, rec_q)
    nrb = mm.record_bytes(case.grid, 2, mdt, True)
    torch.cuda.synchronize()
    assert bool((rec_q[:lo] == 0x5A).all()) and bool((rec_q[hi:nrb] == 0x5A).all())
    assert not bool((rec_q[lo:hi] == 0x5A).all())
    # ... and its runs' records deposit as the full contraction's: copy them in
    rec_m = rec.clone()
    rec_m[lo:hi] = rec_q[lo:hi]
    M_q = torch.empty_like(M_full)
    mm.deposit_records(case.grid, 2, rec_m, M_q, True)
    torch.cuda.synchronize()
    assert torch.equal(M_q, M_full)


@pytest.mark.parametrize("canonical", [False, True])
@pytest.mark.parametrize("mode", ["f64", "f32"])
def test_deposit_planes_bit_identical(mode, canonical):
    """Deposits by node-plane ranges that partition the grid write every entry
    once, equal to one deposition: one and two record sets, overwrite and
    accumulate, full stencil (with mirrored entries across ranges) and the
    canonical half."""
    case = _case(42, (16, 12, 10), 30000, mode)
    other = _case(43, (16, 12, 10), 12000, mode, spread=0.6)
    _print("deposit planes", case, mode)
    mdt = torch.float32 if mode == "f32" else torch.float64
    recs = []
    for c in (case, other):
        sp = c.species[0]
        beta, sigma = species_scalars(c, sp)
        pos, w, B = _dev(c, sp, mode)
        bs, perm = mm.bin_particles(c.grid, 2, pos)
        recs.append(mm.contract_bins(c.grid, 2, pos, w, B, bs, perm, beta, sigma))
    nn = case.grid.ncells
    nof = mm.noff_canonical(2) if canonical else 125
    g = torch.Generator(device="cpu").manual_seed(7)
    M0 = torch.randn(nn * nof * 9, generator=g, dtype=torch.float64).to("cuda", mdt)
    for sets in (recs[:1], recs):
        for acc in (False, True):
            M_full = M0.clone()
            mm.deposit_records(case.grid, 2, sets if len(sets) > 1 else sets[0], M_full, True, accumulate=acc,
                               canonical=canonical)
            M_p = M0.clone() if acc else torch.full_like(M0, float("nan"))
            for z0, z1 in PARTS[10]:
                mm.deposit_records_planes(case.grid, 2, sets, M_p, z0, z1, accumulate=acc, canonical=canonical)
            torch.cuda.synchronize()
            assert torch.equal(M_p, M_full), (len(sets), acc)


def _sampled_rows_check(case, sp, M, mode, nodes):
    beta, sigma = species_scalars(case, sp)
    B = sp.B
    ref = oracle.rows(2, case.grid.n, case.grid.origin, case.grid.h, sp.pos, sp.w, nodes, B, beta, sigma)
    got = M.view(case.grid.ncells, -1)[torch.from_numpy(nodes).cuda()].double().cpu().numpy().reshape(ref.shape)
    assert_match(got, ref, "f32" if mode == "f32" else "f64")


@pytest.mark.parametrize("mode", ["f64", "f32", "mix"])
@pytest.mark.parametrize("n", [(96, 96, 18), (96, 88, 17)])
def test_assemble_overlapped(mode, n):
    """mm_assemble_ecsim on a grid the library splits into slabs (96 x 96 x 18:
    five slabs, the last of two planes; 96 x 88 x 17: the last of one plane,
    visited in plain order) equals the two phases in turn bit for bit,
    overwriting and accumulating, and matches the oracle on sampled rows."""
    case = _case(44, n, 400000, mode, spread=0.7)
    assert mm.slab_planes(case.grid, 2) == 4
    _print("assemble overlapped", case, mode)
    sp = case.species[0]
    beta, sigma = species_scalars(case, sp)
    pos, w, B = _dev(case, sp, mode)
    bs, perm = mm.bin_particles(case.grid, 2, pos, mixed=mode == "mix")
    mdt = torch.float32 if mode == "f32" else torch.float64
    nn = case.grid.ncells
    rec = mm.contract_bins(case.grid, 2, pos, w, B, bs, perm, beta, sigma)
    M_two = torch.empty(nn * 125 * 9, dtype=mdt, device="cuda")
    mm.deposit_records(case.grid, 2, rec, M_two, True)
    M = torch.full_like(M_two, float("nan"))
    mm.assemble_ecsim(case.grid, 2, pos, w, B, bs, perm, beta, sigma, M=M, algo="mfma")
    torch.cuda.synchronize()
    assert torch.equal(M, M_two)
    # accumulate: M + the same species again
    mm.deposit_records(case.grid, 2, rec, M_two, True, accumulate=True)
    mm.assemble_ecsim(case.grid, 2, pos, w, B, bs, perm, beta, sigma, M=M, accumulate=True, algo="mfma")
    torch.cuda.synchronize()
    assert torch.equal(M, M_two)
    del rec, M_two
    # against the oracle: a fresh assembly, rows of nodes in every slab and on
    # the periodic seam (planes 0, 1, 16, 17)
    mm.assemble_ecsim(case.grid, 2, pos, w, B, bs, perm, beta, sigma, M=M, algo="mfma")
    rng = np.random.default_rng(5)
    nx, ny, nz = n
    zs = np.array([0, 1, 3, 4, 8, 12, 15, 16, n[2] - 1])
    nodes = (rng.integers(0, nx, zs.size) + nx * (rng.integers(0, ny, zs.size) + ny * zs)).astype(np.int64)
    _sampled_rows_check(case, sp, M, mode, nodes)


@pytest.mark.parametrize("mode", ["f64", "mix"])
def test_contract_planes_grid_field(mode):
    """With the field on the grid nodes (gathered inside the fp64 contraction),
    records written plane range by plane range deposit to the same M as one
    contraction, bit for bit."""
    case = _case(46, (16, 12, 10), 30000, mode)
    _print("contract planes gridB", case, mode)
    sp = case.species[0]
    beta, sigma = species_scalars(case, sp)
    pos, w, _ = _dev(case, sp, mode)
    Fg = torch.from_numpy(grid_field(case.grid, 11, "f64")).to("cuda", torch.float32 if mode == "mix" else torch.float64)
    bs, perm = mm.bin_particles(case.grid, 2, pos, mixed=mode == "mix")
    rec = mm.contract_bins(case.grid, 2, pos, w, None, bs, perm, beta, sigma, Bgrid=Fg)
    M_full = torch.empty(case.grid.ncells * 125 * 9, dtype=torch.float64, device="cuda")
    mm.deposit_records(case.grid, 2, rec, M_full, True)
    rec_p = torch.full_like(rec, 0x5A)
    for z0, z1 in PARTS[10]:
        mm.contract_bins_planes(case.grid, 2, pos, w, None, bs, perm, beta, sigma, z0, z1, rec_p, Bgrid=Fg)
    M_p = torch.full_like(M_full, float("nan"))
    mm.deposit_records(case.grid, 2, rec_p, M_p, True)
    torch.cuda.synchronize()
    assert torch.equal(M_p, M_full)


@pytest.mark.parametrize("mode", ["f64", "f32", "mix"])
def test_assemble_overlapped_grid_field(mode):
    """The overlapped assembly with the field on the grid nodes (gathered in
    the fp64 contraction, interpolated first for fp32) equals the two phases."""
    n = (96, 96, 16)
    case = _case(45, n, 200000, mode)
    assert mm.slab_planes(case.grid, 2) == 4
    _print("assemble overlapped gridB", case, mode)
    sp = case.species[0]
    beta, sigma = species_scalars(case, sp)
    pos, w, _ = _dev(case, sp, mode)
    dt = torch.float32 if mode == "f32" else torch.float64
    Fg = torch.from_numpy(grid_field(case.grid, 9, case.dtype)).to("cuda", torch.float32 if mode == "mix" else dt)
    bs, perm = mm.bin_particles(case.grid, 2, pos, mixed=mode == "mix")
    rec = mm.contract_bins(case.grid, 2, pos, w, None, bs, perm, beta, sigma, Bgrid=Fg)
    M_two = torch.empty(case.grid.ncells * 125 * 9, dtype=dt, device="cuda")
    mm.deposit_records(case.grid, 2, rec, M_two, True)
    M = torch.full_like(M_two, float("nan"))
    mm.assemble_ecsim_gridB(case.grid, 2, pos, w, Fg, bs, perm, beta, sigma, M=M, algo="mfma")
    torch.cuda.synchronize()
    assert torch.equal(M, M_two)


def test_assemble_overlapped_stream_order():
    """The overlapped assembly is ordered on the caller's stream: on a user
    stream, work enqueued after the call on that stream sees the finished M;
    two calls issued back to back on two streams (sharing the library's second
    stream and its events) both finish correct, with no synchronisation
    between them."""
    n = (96, 96, 16)
    case = _case(47, n, 150000, "f64")
    sp = case.species[0]
    beta, sigma = species_scalars(case, sp)
    pos, w, B = _dev(case, sp, "f64")
    bs, perm = mm.bin_particles(case.grid, 2, pos)
    rec = mm.contract_bins(case.grid, 2, pos, w, B, bs, perm, beta, sigma)
    ref = torch.empty(case.grid.ncells * 125 * 9, dtype=torch.float64, device="cuda")
    mm.deposit_records(case.grid, 2, rec, ref, True)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    M1 = torch.full_like(ref, float("nan"))
    M2 = torch.full_like(ref, float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        mm.assemble_ecsim(case.grid, 2, pos, w, B, bs, perm, beta, sigma, M=M1, algo="mfma")
        c1 = M1.clone()  # enqueued on s1 after the call
    with torch.cuda.stream(s2):
        mm.assemble_ecsim(case.grid, 2, pos, w, B, bs, perm, beta, sigma, M=M2, algo="mfma")
        c2 = M2.sum()
    s1.synchronize()
    assert torch.equal(c1, ref)
    s2.synchronize()
    assert torch.equal(M2, ref)
    assert torch.isfinite(c2).item()
