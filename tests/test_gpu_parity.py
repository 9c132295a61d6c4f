"""GPU parity: every HIP path (binning, matrix-core assembly, atomic scatter)
against the CPU oracle on the same seeded inputs.

Integer work (bin_start, perm) must match bit for bit; matrices must match
within the relative Frobenius budget (1e-12 fp64, 1e-5 fp32). Sizes run
from single particles and ragged tiles to the full named configurations;
the 134M-particle clustered configuration is checked on sampled stencil
rows computed exactly by the oracle plus a matrix-free bilinear form.
"""
import numpy as np
import pytest
import torch

import oracle
import particle_grid_mass_amd as mm
from tests import dense_ref
from tests.gpu_util import (TOL, TDT, as_numpy_M, assert_match, gpu_assemble, oracle_assemble, rel_fro,
                            require_gpu, to_dev, species_scalars)
from workloads import make_config, random_case, Case, Species, Grid

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    print(f"[gpu] {torch.cuda.get_device_name(0)}", flush=True)


def _print_case(tag, case):
    print(f"[case] {tag} {case.name} order={case.order} kind={case.kind} dtype={case.dtype} np={case.np_total} "
          f"n={case.grid.n}", flush=True)


# ------------------------------------------------------------------ binning
BIN_CASES = [
    # seed, order, n, npart, spread, sorted
    (1, 1, (5, 6, 7), 1, 1.0, False),
    (2, 1, (9, 8, 7), 5000, 1.0, False),
    (3, 1, (9, 8, 7), 5000, 0.4, True),
    (4, 2, (5, 6, 7), 3000, 1.0, False),
    (5, 2, (11, 9, 8), 40000, 0.5, False),
    (6, 1, (40, 33, 17), 300000, 1.0, False),   # > 2^16 bins would need 3 digits: 22440 bins, 2 digits
    (7, 2, (70, 70, 70), 200000, 1.0, False),   # 343000 bins: three 8-bit digit passes
]


@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("seed,order,n,npart,spread,srt", BIN_CASES)
def test_bin_parity(seed, order, n, npart, spread, srt, dtype):
    case = random_case(seed, order, n, npart, kind="scalar", dtype=dtype, spread=spread, sorted_by_cell=srt,
                       origin=(-1.5, 0.25, 3.0), h=(0.5, 0.75, 1.25))
    _print_case("bin", case)
    sp = case.species[0]
    bs_ref, perm_ref = oracle.bin_particles(order, n, case.grid.origin, case.grid.h, sp.pos)
    bs, perm = mm.bin_particles(case.grid, order, to_dev(sp.pos, TDT[dtype]))
    torch.cuda.synchronize()
    assert np.array_equal(bs.cpu().numpy(), bs_ref)
    assert np.array_equal(perm.cpu().numpy(), perm_ref)


def _one_descent(srt, keys, t):
    """``srt`` (keys non-decreasing) with exactly one descent, between t-1 and
    t: the first particle of the next bin after t-1's is moved to t-1."""
    t = t % len(srt)
    j = int(np.searchsorted(keys, keys[t - 1], side="right"))
    assert j < len(srt), "t-1 must not be in the last bin"
    out = np.concatenate([srt[:t - 1], srt[j:j + 1], srt[t - 1:j], srt[j + 1:]])
    k = np.concatenate([keys[:t - 1], keys[j:j + 1], keys[t - 1:j], keys[j + 1:]])
    assert np.count_nonzero(k[1:] < k[:-1]) == 1 and k[t] < k[t - 1]
    return np.ascontiguousarray(out)


# descent positions: wave (64), item row (256) and tile (2048, 4096) boundaries, inside a wave of the
# ragged last tile (5000)
DESCENT_AT = [None, 64, 256, 2048, 4096, 5000]


@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("t", DESCENT_AT)
def test_bin_key_ordered_input(order, t):
    """Input already in key order (the device short cut), and the same input
    with exactly one descent at a wave, item-row or tile boundary or in the
    ragged last tile (the full radix path); three calls in a row so that state
    left in a reused workspace would show."""
    case = random_case(31 + order, order, (9, 8, 7), 6100, kind="scalar", spread=0.6,
                       origin=(-1.5, 0.25, 3.0), h=(0.5, 0.75, 1.25))
    g = case.grid
    pos0 = case.species[0].pos + np.array([0.0, 0.0, 2 * g.h[2]])  # two empty z-planes of bins first
    bs0, perm0 = oracle.bin_particles(order, g.n, g.origin, g.h, pos0)
    srt = np.ascontiguousarray(pos0[perm0])  # keys non-decreasing
    keys = np.searchsorted(bs0, np.arange(len(srt)), side="right") - 1
    mixed = srt if t is None else _one_descent(srt, keys, t)
    for arr in (srt, mixed, srt):
        print(f"[case] key-ordered order={order} descent at {t}", flush=True)
        bs_ref, perm_ref = oracle.bin_particles(order, g.n, g.origin, g.h, arr)
        bs, perm = mm.bin_particles(g, order, to_dev(arr, torch.float64))
        torch.cuda.synchronize()
        assert np.array_equal(bs.cpu().numpy(), bs_ref)
        assert np.array_equal(perm.cpu().numpy(), perm_ref)


def test_bin_empty():
    g = Grid((5, 5, 5))
    bs, perm = mm.bin_particles(g, 1, torch.zeros((0, 3), dtype=torch.float64, device="cuda"))
    torch.cuda.synchronize()
    assert bs.shape[0] == 126 and int(bs.abs().sum()) == 0 and perm.numel() == 0


def test_bin_positions_outside_domain():
    """Periodic wrap of positions several periods away, both signs."""
    case = random_case(17, 2, (6, 7, 5), 3000, kind="scalar")
    pos = case.species[0].pos.copy()
    pos[::3] += np.array([12.0, -14.0, 25.0])
    pos[1::3] -= np.array([30.0, 7.0, 5.0])
    bs_ref, perm_ref = oracle.bin_particles(2, case.grid.n, case.grid.origin, case.grid.h, pos)
    bs, perm = mm.bin_particles(case.grid, 2, to_dev(pos, torch.float64))
    torch.cuda.synchronize()
    assert np.array_equal(bs.cpu().numpy(), bs_ref)
    assert np.array_equal(perm.cpu().numpy(), perm_ref)


# ------------------------------------------------------------------ assembly, small and ragged
SMALL = [
    # seed, order, n, npart
    (11, 1, (5, 6, 7), 1),
    (12, 1, (5, 6, 7), 37),
    (13, 1, (9, 8, 7), 20000),
    (14, 2, (5, 6, 7), 3),
    (15, 2, (7, 6, 5), 1500),
    (16, 2, (9, 8, 7), 20000),
    # x extent a multiple of 4: the second-order fp64 3x3 path writes run records
    (17, 2, (8, 6, 5), 3),
    (18, 2, (12, 7, 6), 20000),
    (19, 2, (16, 5, 5), 1),
    # an odd number of runs (105): a wave of the run-record contraction that takes
    # consecutive runs is left with one
    (20, 2, (12, 5, 7), 9000),
]


@pytest.mark.parametrize("algo", ["mfma", "mfma_atomic", "atomic"])
@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
@pytest.mark.parametrize("seed,order,n,npart", SMALL)
def test_assemble_small(seed, order, n, npart, kind, dtype, algo):
    case = random_case(seed, order, n, npart, kind=kind, dtype=dtype, beta=0.7, sigma=1.3,
                       origin=(0.25, -2.0, 1.0), h=(0.5, 1.0, 0.75), spread=0.8)
    _print_case(f"small/{algo}", case)
    M = as_numpy_M(gpu_assemble(case, algo), case)
    ref = oracle_assemble(case)
    assert_match(M, ref, dtype)


@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_one_heavy_bin(order, dtype):
    """All particles in one cell: one bin far longer than a batch or a round."""
    rng = np.random.default_rng(5 + order)
    npart = 5000
    pos = np.array([3.0, 2.0, 4.0]) + rng.random((npart, 3))
    pos = pos.astype(np.float32) if dtype == "f32" else pos
    w = rng.uniform(0.5, 1.5, npart)
    B = rng.standard_normal((npart, 3))
    if dtype == "f32":
        w, B = w.astype(np.float32), B.astype(np.float32)
    case = Case("heavy", Grid((6, 6, 7)), order, "ecsim", [Species(pos, w, B, 0.5)], dtype=dtype)
    _print_case("heavy", case)
    M = as_numpy_M(gpu_assemble(case, "mfma"), case)
    assert_match(M, oracle_assemble(case), dtype)


def test_accumulate_and_empty():
    case = random_case(21, 1, (6, 5, 7), 2000, kind="ecsim")
    sp = case.species[0]
    pos, w, B = (to_dev(a, torch.float64) for a in (sp.pos, sp.w, sp.B))
    bs, perm = mm.bin_particles(case.grid, 1, pos)
    M = mm.assemble_ecsim(case.grid, 1, pos, w, B, bs, perm, beta=sp.beta)
    M = mm.assemble_ecsim(case.grid, 1, pos, w, B, bs, perm, beta=sp.beta, M=M, accumulate=True)
    ref = oracle_assemble(case)
    assert rel_fro(as_numpy_M(M, case), 2 * ref) <= 1e-12
    # np == 0: overwrite zeroes, accumulate leaves M alone
    e3 = torch.zeros((0, 3), dtype=torch.float64, device="cuda")
    e1 = torch.zeros((0,), dtype=torch.float64, device="cuda")
    ebs, eperm = mm.bin_particles(case.grid, 1, e3)
    M2 = mm.assemble_ecsim(case.grid, 1, e3, e1, e3, ebs, eperm, beta=0.5, M=M.clone(), accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(M2, M)
    M3 = mm.assemble_ecsim(case.grid, 1, e3, e1, e3, ebs, eperm, beta=0.5, M=M.clone(), accumulate=False)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(M3)) == 0


def test_gpu_symmetry_and_partition_of_unity():
    case = random_case(31, 2, (8, 7, 9), 30000, kind="ecsim")
    sp = case.species[0]
    M = as_numpy_M(gpu_assemble(case, "mfma"), case)
    R, NO = 2, 5
    nx, ny, nz = case.grid.n
    g = np.arange(case.grid.ncells)
    gx, gy, gz = g % nx, (g // nx) % ny, g // (nx * ny)
    scale = np.abs(M).max()
    for o in range(NO ** 3):
        ox, oy, oz = o % NO - R, (o // NO) % NO - R, o // (NO * NO) - R
        g2 = (gx + ox) % nx + nx * (((gy + oy) % ny) + ny * ((gz + oz) % nz))
        o2 = (-ox + R) + NO * ((-oy + R) + NO * (-oz + R))
        assert np.abs(M[g, o] - M[g2, o2]).max() <= 1e-13 * scale
    W = dense_ref.dense_W(2, case.grid.n, case.grid.origin, case.grid.h, sp.pos)
    S = np.stack([sp.w[p] * oracle.alpha(sp.B[p], sp.beta).reshape(-1) for p in range(sp.np)])
    assert rel_fro(M.sum(axis=1), W.T @ S) <= 1e-12


# ------------------------------------------------------------------ named configurations, full size
@pytest.mark.parametrize("algo", ["mfma", "atomic"])
def test_config1_full(algo):
    case = make_config(1)
    _print_case(f"c1/{algo}", case)
    assert_match(as_numpy_M(gpu_assemble(case, algo), case), oracle_assemble(case), "f64")


@pytest.mark.parametrize("algo", ["mfma", "atomic"])
def test_config2_full(algo):
    case = make_config(2)
    _print_case(f"c2/{algo}", case)
    assert_match(as_numpy_M(gpu_assemble(case, algo), case), oracle_assemble(case), "f64")


@pytest.mark.parametrize("shuffled", [False, True])
def test_config3_full(shuffled):
    case = make_config(3, shuffled=shuffled)
    _print_case("c3/mfma", case)
    M, bins = gpu_assemble(case, "mfma", return_bins=True)
    ref = oracle_assemble(case)
    assert_match(as_numpy_M(M, case), ref, "f64")
    for (bs, perm), sp in zip(bins, case.species):  # binning of each species, bit-exact
        bs_ref, perm_ref = oracle.bin_particles(1, case.grid.n, case.grid.origin, case.grid.h, sp.pos)
        assert np.array_equal(bs.cpu().numpy(), bs_ref)
        assert np.array_equal(perm.cpu().numpy(), perm_ref)


@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
def test_config4_full(kind):
    case = make_config(4, kind=kind)
    _print_case("c4/mfma", case)
    assert_match(as_numpy_M(gpu_assemble(case, "mfma"), case), oracle_assemble(case), "f64")


@pytest.fixture(scope="module")
def config5_f64():
    return make_config(5, dtype="f64")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dtype", ["f64", "f32"])
def test_config5_sampled(dtype, config5_f64):
    """134M particles, clustered: exact rows for sampled nodes and a bilinear form."""
    case = config5_f64
    if dtype == "f32":
        sp0 = case.species[0]
        case = Case(case.name.replace("f64", "f32"), case.grid, case.order, case.kind,
                    [Species(sp0.pos.astype(np.float32), sp0.w.astype(np.float32), sp0.B.astype(np.float32),
                             sp0.beta, sp0.name)], sigma=case.sigma, dtype="f32", seed=case.seed)
    _print_case("c5/mfma", case)
    sp = case.species[0]
    M = gpu_assemble(case, "mfma")
    nn = case.grid.ncells
    n = case.grid.n[0]
    rng = np.random.default_rng(55)
    centres = [(32, 32, 32), (96, 96, 32), (96, 32, 96), (32, 96, 96)]  # cluster centres: densest bins
    nodes = np.concatenate([rng.integers(0, nn, 44), [0, nn - 1],
                            [x + n * (y + n * z) for (x, y, z) in centres]]).astype(np.int64)
    beta, sigma = species_scalars(case, sp)
    rows_ref = oracle.rows(2, case.grid.n, case.grid.origin, case.grid.h, sp.pos, sp.w, nodes, sp.B, beta, sigma)
    rows = M[torch.from_numpy(nodes).cuda()].double().cpu().numpy().reshape(rows_ref.shape)
    assert_match(rows, rows_ref, dtype)
    # bilinear form u^T M v over the whole matrix (stencil contraction with torch on the GPU
    # output) against the oracle's O(np N) evaluation from the particles.
    u = rng.standard_normal((nn, 3))
    v = rng.standard_normal((nn, 3))
    ref = oracle.bilinear(2, case.grid.n, case.grid.origin, case.grid.h, sp.pos, sp.w, u, v, sp.B, beta, sigma)
    got = _stencil_bilinear_torch(M, case, u, v)
    del M
    torch.cuda.empty_cache()
    assert abs(got - ref) <= (1e-11 if dtype == "f64" else 1e-5) * abs(ref) + 1e-9


def _stencil_bilinear_torch(M, case, u, v):
    n = case.grid.n
    R, NO = case.order, 2 * case.order + 1
    nx, ny, nz = n
    ud = torch.from_numpy(u).cuda()
    vd = torch.from_numpy(v).cuda().reshape(nz, ny, nx, 3)
    Md = M.reshape(nz, ny, nx, NO ** 3, 3, 3)
    total = torch.zeros((), dtype=torch.float64, device="cuda")
    for o in range(NO ** 3):
        ox, oy, oz = o % NO - R, (o // NO) % NO - R, o // (NO * NO) - R
        vs = torch.roll(vd, shifts=(-oz, -oy, -ox), dims=(0, 1, 2)).reshape(-1, 3)
        blk = Md[:, :, :, o].reshape(-1, 3, 3).double()
        total += torch.einsum("gi,gij,gj->", ud, blk, vs)
    return float(total)


# ------------------------------------------------------------------ vector-FMA comparison contraction
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
@pytest.mark.parametrize("seed,order,n,npart", [c for c in SMALL if c[1] == 1])
def test_valu_contraction_small(seed, order, n, npart, kind):
    """MM_ALGO_VALU: the binned CIC contraction on vector FMAs, same records
    and deposit as the matrix-core path."""
    case = random_case(seed, order, n, npart, kind=kind, dtype="f64", beta=0.7, sigma=1.3,
                       origin=(0.25, -2.0, 1.0), h=(0.5, 1.0, 0.75), spread=0.8)
    _print_case("small/valu", case)
    assert_match(as_numpy_M(gpu_assemble(case, "valu"), case), oracle_assemble(case), "f64")


@pytest.mark.parametrize("algo", ["mfma", "valu"])
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
def test_split_k_many_chunks(algo, kind):
    """A grid of few bins (210) holding about 250 particles per occupied bin
    takes the split-K contraction of either algorithm (one bin per wave on the
    matrix cores, four per wave on vector FMAs); the bins are ragged and span
    several chunks of the slices."""
    case = random_case(21, 1, (6, 5, 7), 42000, kind=kind, dtype="f64", beta=0.7, sigma=1.3,
                       origin=(0.25, -2.0, 1.0), h=(0.5, 1.0, 0.75), spread=0.8)
    nb = 6 * 5 * 7
    assert (nb + 3) // 4 < 3072 and (nb + 15) // 16 < 2048 and 42000 >= 16 * nb  # both split-K rules hold
    _print_case(f"splitk/{algo}", case)
    assert_match(as_numpy_M(gpu_assemble(case, algo), case), oracle_assemble(case), "f64")


def test_valu_contraction_config2():
    case = make_config(2)
    _print_case("c2/valu", case)
    assert_match(as_numpy_M(gpu_assemble(case, "valu"), case), oracle_assemble(case), "f64")


def test_valu_unsupported_combinations():
    from particle_grid_mass_amd import _lib
    case = random_case(61, 2, (6, 6, 6), 100, kind="ecsim")
    sp = case.species[0]
    pos, w, B = (to_dev(a, torch.float64) for a in (sp.pos, sp.w, sp.B))
    bs, perm = mm.bin_particles(case.grid, 2, pos)
    with pytest.raises(mm.MMError) as ei:  # second order
        mm.assemble_ecsim(case.grid, 2, pos, w, B, bs, perm, beta=0.5, algo="valu")
    assert ei.value.status == _lib.MM_ERR_UNSUPPORTED
    c1 = random_case(62, 1, (6, 6, 6), 100, kind="ecsim", dtype="f32")
    s1 = c1.species[0]
    p1, w1, B1 = (to_dev(a, torch.float32) for a in (s1.pos, s1.w, s1.B))
    b1, q1 = mm.bin_particles(c1.grid, 1, p1)
    with pytest.raises(mm.MMError) as ei:  # fp32
        mm.assemble_ecsim(c1.grid, 1, p1, w1, B1, b1, q1, beta=0.5, algo="valu")
    assert ei.value.status == _lib.MM_ERR_UNSUPPORTED
