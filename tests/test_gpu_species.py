"""GPU parity of the several-species deposition (mm_deposit_records_multi):
every species contracted into a record set of its own, one pass over M for
all of them (the mass matrices of all species enter the one field operator,
Sec. 2.1), through the C ABI, against the oracle of all species."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import particle_grid_mass_amd as mm
from tests.gpu_util import TOL, TDT, assert_match, oracle_assemble, rel_fro, require_gpu, to_dev
from workloads import make_config, random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def species_case(seed, order, n, counts, kind, dtype):
    """One grid, len(counts) species with their own particles, weights, fields and beta."""
    sp = []
    for k, npart in enumerate(counts):
        c = random_case(seed + 17 * k, order, n, npart, kind=kind, dtype=dtype, beta=0.6 - 0.45 * k,
                        sigma=1.2, origin=(0.25, -2.0, 1.0), h=(0.5, 1.0, 0.75), spread=1.0 if k != 1 else 0.5)
        sp += c.species
    return dataclasses.replace(c, species=sp, name=f"species{len(counts)}")


def record_sets(case):
    dt = TDT[case.dtype]
    tens = case.kind == "ecsim"
    recs = []
    for sp in case.species:
        pos, w = to_dev(sp.pos, dt), to_dev(sp.w, dt)
        B = to_dev(sp.B, dt) if tens else None
        bs, perm = mm.bin_particles(case.grid, case.order, pos)
        recs.append(mm.contract_bins(case.grid, case.order, pos, w, B, bs, perm, sp.beta, case.sigma))
    return recs


def new_M(case, canonical, fill=None):
    nc = 9 if case.kind == "ecsim" else 1
    nof = mm.noff_canonical(case.order) if canonical else mm.noff(case.order)
    M = torch.empty(case.grid.ncells * nof * nc, dtype=TDT[case.dtype], device="cuda")
    if fill is not None:
        M.copy_(torch.from_numpy(fill.reshape(-1)).to(M.dtype))
    return M, (case.grid.ncells, nof, nc)


CASES = [(201, 1, (5, 6, 7), (3000, 1200)), (202, 2, (7, 6, 5), (2500, 900, 40)),
         (203, 2, (9, 8, 7), (20000, 7000, 3, 500)), (204, 1, (6, 5, 5), (0, 800)),
         # x extent a multiple of 4: second-order fp64 3x3 records are run records
         (205, 2, (8, 6, 5), (6000, 2000, 0)), (206, 2, (12, 5, 7), (9000, 31))]


@pytest.mark.parametrize("canonical", [False, True])
@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
@pytest.mark.parametrize("seed,order,n,counts", CASES)
def test_deposit_multi(seed, order, n, counts, kind, dtype, canonical):
    case = species_case(seed, order, n, counts, kind, dtype)
    print(f"[case] multi order={order} n={n} counts={counts} {kind} {dtype} canonical={canonical}", flush=True)
    tens = kind == "ecsim"
    recs = record_sets(case)
    M, shape = new_M(case, canonical)
    mm.deposit_records(case.grid, order, recs, M, tens, canonical=canonical)
    # the same sets deposited one after the other (accumulating)
    Ms, _ = new_M(case, canonical)
    for k, r in enumerate(recs):
        mm.deposit_records(case.grid, order, r, Ms, tens, accumulate=k > 0, canonical=canonical)
    # one set through the several-set entry is the single-set deposit, bit for bit
    M1, _ = new_M(case, canonical)
    mm.deposit_records(case.grid, order, recs[:1], M1, tens, canonical=canonical)
    Ms1, _ = new_M(case, canonical)
    mm.deposit_records(case.grid, order, recs[0], Ms1, tens, canonical=canonical)
    torch.cuda.synchronize()
    ref = oracle_assemble(case).reshape(case.grid.ncells, mm.noff(order), -1)
    if canonical:
        ref = oracle.canonical_half(order, ref)
    got = M.view(shape).double().cpu().numpy()
    assert rel_fro(got, ref) <= TOL[dtype]
    assert rel_fro(got, Ms.view(shape).double().cpu().numpy()) <= TOL[dtype]
    assert torch.equal(M1, Ms1)


@pytest.mark.parametrize("order", [1, 2])
def test_deposit_multi_accumulate(order):
    case = species_case(300 + order, order, (7, 7, 6), (4000, 2500), "ecsim", "f64")
    recs = record_sets(case)
    rng = np.random.default_rng(7)
    nc, nof = 9, mm.noff(order)
    base = rng.standard_normal((case.grid.ncells, nof, nc))
    M, shape = new_M(case, False, fill=base)
    mm.deposit_records(case.grid, order, recs, M, True, accumulate=True)
    torch.cuda.synchronize()
    ref = base + oracle_assemble(case).reshape(shape)
    assert rel_fro(M.view(shape).cpu().numpy(), ref) <= 1e-12


def test_config3_multi():
    """Both species of the 64^3, 125-particle-per-cell workload in one deposition."""
    case = make_config(3)
    print("[case] c3 multi", flush=True)
    recs = record_sets(case)
    M, shape = new_M(case, False)
    mm.deposit_records(case.grid, 1, recs, M, True)
    torch.cuda.synchronize()
    assert rel_fro(M.view(shape).cpu().numpy(), oracle_assemble(case).reshape(shape)) <= 1e-12


def mirror_equal(M, order, n):
    """M[g][o] == M[g + d(o)][-o] bit for bit, for every node and offset."""
    R, NO = order, 2 * order + 1
    nx, ny, nz = n
    g = np.arange(nx * ny * nz)
    gx, gy, gz = g % nx, (g // nx) % ny, g // (nx * ny)
    for o in range(NO ** 3):
        ox, oy, oz = o % NO - R, (o // NO) % NO - R, o // (NO * NO) - R
        g2 = (gx + ox) % nx + nx * (((gy + oy) % ny) + ny * ((gz + oz) % nz))
        o2 = NO ** 3 - 1 - o
        if not np.array_equal(M[g, o], M[g2, o2]):
            return False
    return True


@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
def test_mirrored_deposit_exact_symmetry(kind, dtype):
    """The full-stencil deposit that stores each sum at both mirrored entries
    (order 2, and order 1 with several record sets) gives an exactly
    symmetric matrix, and its computed half equals the canonical deposit bit
    for bit."""
    for order, counts in ((2, (6000,)), (2, (3000, 2000)), (1, (4000, 2500))):
        case = species_case(400 + order, order, (7, 6, 8), counts, kind, dtype)
        recs = record_sets(case)
        M, shape = new_M(case, False)
        Mc, cshape = new_M(case, True)
        arg = recs if len(recs) > 1 or order == 2 else recs[0]
        mm.deposit_records(case.grid, order, arg, M, kind == "ecsim")
        mm.deposit_records(case.grid, order, arg, Mc, kind == "ecsim", canonical=True)
        torch.cuda.synchronize()
        Mn = M.view(shape).cpu().numpy()
        assert mirror_equal(Mn, order, case.grid.n), (order, counts)
        c = (mm.noff(order) - 1) // 2
        assert np.array_equal(Mn[:, c:, :], Mc.view(cshape).cpu().numpy()), (order, counts)
        ref = oracle_assemble(case).reshape(shape)
        assert rel_fro(Mn, ref) <= TOL[dtype]


# ------------------------------------------------ every species in one record set
def _widen32(case):
    """The case with positions and fields rounded to fp32 (the mixed layout's
    stored values), as the oracle must see them."""
    sp = [dataclasses.replace(s, pos=s.pos.astype(np.float32).astype(np.float64),
                              B=None if s.B is None else s.B.astype(np.float32).astype(np.float64))
          for s in case.species]
    return dataclasses.replace(case, species=sp)


def species_tuples(case, layout="dense", mixed=False):
    """(pos, w, B, bin_start, perm, beta) per species on the device: dense
    arrays, fp32 positions and fields (mixed), or for layout "record8" one
    64-byte float64 record per particle on every other species."""
    out = []
    for k, sp in enumerate(case.species):
        tens = sp.B is not None and case.kind == "ecsim"
        if mixed:
            pos, w = to_dev(sp.pos, torch.float32), to_dev(sp.w, torch.float64)
            B = to_dev(sp.B, torch.float32) if tens else None
        elif layout == "record8" and k % 2 == 0 and tens:
            R = torch.full((sp.pos.shape[0], 8), float("nan"), dtype=torch.float64, device="cuda")
            R[:, 0:3], R[:, 3], R[:, 4:7] = to_dev(sp.pos, torch.float64), to_dev(sp.w, torch.float64), \
                to_dev(sp.B, torch.float64)
            pos, w, B = R[:, 0:3], R[:, 3], R[:, 4:7]
        else:
            pos, w = to_dev(sp.pos, torch.float64), to_dev(sp.w, torch.float64)
            B = to_dev(sp.B, torch.float64) if tens else None
        bs, perm = mm.bin_particles(case.grid, case.order, pos, mixed=mixed)
        out.append((pos, w, B, bs, perm, sp.beta))
    return out


SET_CASES = [(401, (5, 6, 7), (3000, 1200)), (402, (6, 5, 5), (0, 800)), (403, (9, 8, 7), (20000, 7000, 3, 500)),
             (404, (7, 6, 8), (900, 0, 1, 2000, 37, 4000, 5, 800)),  # the most species a set takes
             (405, (16, 12, 10), (60000, 60000))]


# (kind, storage): strided records are read by the tensorial path only
SET_MODES = [("scalar", "dense"), ("scalar", "mixed"), ("ecsim", "dense"), ("ecsim", "record8"), ("ecsim", "mixed")]


@pytest.mark.parametrize("kind,mode", SET_MODES)
@pytest.mark.parametrize("seed,n,counts", SET_CASES)
def test_contract_species_one_set(seed, n, counts, kind, mode):
    """First order: one contraction launch for every species, one record set,
    one deposit; the oracle sums the species' matrices."""
    case = species_case(seed, 1, n, counts, kind, "f64")
    if mode == "mixed":
        case = _widen32(case)
    print(f"[case] species set n={n} counts={counts} {kind} {mode}", flush=True)
    tens = kind == "ecsim"
    rec = mm.contract_bins_species(case.grid, 1, species_tuples(case, mode, mode == "mixed"), case.sigma)
    M, shape = new_M(case, False)
    mm.deposit_records(case.grid, 1, rec, M, tens)
    torch.cuda.synchronize()
    assert rec.numel() == mm.record_bytes(case.grid, 1, torch.float64, tens)
    assert_match(M.view(shape).cpu().numpy(), oracle_assemble(case).reshape(shape), "f64")


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("algo", ["mfma", "atomic"])
@pytest.mark.parametrize("order,n", [(1, (7, 6, 5)), (2, (7, 6, 5)), (2, (8, 6, 5))])
def test_assemble_ecsim_species(order, n, algo, accumulate):
    """The whole set in one call: one record set (first order, matrix cores)
    or species after species (otherwise), into M or added to it."""
    case = species_case(500 + order, order, n, (5000, 2100, 0), "ecsim", "f64")
    print(f"[case] assemble species order={order} n={n} {algo} accumulate={accumulate}", flush=True)
    shape = (case.grid.ncells, mm.noff(order), 9)
    base = np.random.default_rng(9).standard_normal(shape) if accumulate else np.zeros(shape)
    M = torch.from_numpy(base).cuda()
    mm.assemble_ecsim_species(case.grid, order, species_tuples(case), case.sigma, M=M, accumulate=accumulate,
                              algo=algo)
    torch.cuda.synchronize()
    assert_match(M.cpu().numpy() - base, oracle_assemble(case).reshape(shape), "f64")


def test_config3_one_set():
    """Config 3 (64^3 cells, 125 per cell, two species) as one record set,
    sorted and shuffled, with one 64-byte record per particle."""
    for shuffled in (False, True):
        case = make_config(3, shuffled=shuffled)
        print(f"[case] c3 one set shuffled={shuffled}", flush=True)
        M = mm.assemble_ecsim_species(case.grid, 1, species_tuples(case, "record8" if shuffled else "dense"),
                                      case.sigma)
        torch.cuda.synchronize()
        shape = (case.grid.ncells, 27, 9)
        assert_match(M.cpu().numpy().reshape(shape), oracle_assemble(case).reshape(shape), "f64")
        del M
