"""Pins for the CPU oracle against what the method and mathematics fix.

Each test ties the oracle (direct scatter of Eq. 6, Pennati & Markidis,
Sec. 2.1) to something other than itself: a dense brute-force contraction
with an independently evaluated B-spline, closed forms that are exact in
binary, the spatial symmetry of Sec. 3.4 / Table 1's footnote, partition of
unity of the B-splines, alpha as a matrix inverse, translation, linearity and
a matrix-free bilinear form.
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests import dense_ref
from workloads import random_case, make_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def rel(a, b):
    d = np.linalg.norm((np.asarray(a) - np.asarray(b)).ravel())
    s = np.linalg.norm(np.asarray(b).ravel())
    return d / s if s > 0 else d


def run_oracle(case, **kw):
    sp = case.species[0]
    return oracle.assemble(case.order, case.grid.n, case.grid.origin, case.grid.h, sp.pos, sp.w,
                           sp.B if case.kind == "ecsim" else None, sp.beta, case.sigma, **kw)


# ---------------------------------------------------------------- dense brute force
@pytest.mark.parametrize("order,n", [(1, (3, 3, 3)), (1, (4, 5, 3)), (1, (5, 4, 6)), (2, (5, 5, 5)),
                                     (2, (6, 5, 7)), (2, (7, 6, 5))])
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
@pytest.mark.parametrize("npart", [1, 2, 3, 4, 97])
def test_dense_bruteforce(order, n, kind, npart):
    seed = 7 + 13 * order + 31 * npart + (0 if kind == "scalar" else 5) + n[0] * 101 + n[1] * 7
    case = random_case(seed, order, n, npart, kind=kind, beta=0.7, sigma=1.3,
                       origin=(-0.25, 0.5, 1.0), h=(0.5, 1.25, 2.0))
    sp = case.species[0]
    # shift some particles by whole periods to exercise the periodic wrap
    pos = sp.pos.copy()
    pos[::2, 0] += 2 * case.grid.n[0] * case.grid.h[0]
    pos[1::3, 2] -= case.grid.n[2] * case.grid.h[2]
    M = oracle.assemble(order, n, case.grid.origin, case.grid.h, pos, sp.w, sp.B, sp.beta, case.sigma)
    Md = dense_ref.dense_M(order, n, case.grid.origin, case.grid.h, pos, sp.w, sp.B, sp.beta, case.sigma)
    ref = dense_ref.dense_to_stencil(order, n, Md)
    assert M.shape == ref.shape
    assert rel(M, ref) < 1e-14


def test_dense_bruteforce_catches_transpose():
    """A transposed alpha (or [B]x sign flip) must fail the dense comparison."""
    case = random_case(3, 1, (4, 4, 4), 5, kind="ecsim", beta=0.9)
    sp = case.species[0]
    M = run_oracle(case)
    Md = dense_ref.dense_M(1, case.grid.n, case.grid.origin, case.grid.h, sp.pos, sp.w, sp.B, sp.beta)
    bad = Md.reshape(3, 3, *Md.shape[1:]).transpose(1, 0, 2, 3).reshape(Md.shape)
    assert rel(M, dense_ref.dense_to_stencil(1, case.grid.n, Md)) < 1e-14
    assert rel(M, dense_ref.dense_to_stencil(1, case.grid.n, bad)) > 1e-3


# ---------------------------------------------------------------- closed forms (golden)
def _golden():
    with open(GOLDEN) as f:
        return {c["name"]: c for c in json.load(f)["cases"]}


def test_golden_cic_on_node():
    c = _golden()["cic_particle_on_node"]
    M = oracle.assemble(c["order"], c["n"], c["origin"], c["h"], np.array(c["pos"]), np.array(c["w"]),
                        None, 0.0, c["sigma"])
    n = c["n"]
    (e,) = c["expect_nonzero"]
    g = e["node"][0] + n[0] * (e["node"][1] + n[1] * e["node"][2])
    o = (e["offset"][0] + 1) + 3 * ((e["offset"][1] + 1) + 3 * (e["offset"][2] + 1))
    assert M[g, o, 0] == e["value"]
    M[g, o, 0] = 0.0
    assert np.count_nonzero(M) == 0


def test_golden_cic_cell_centre():
    c = _golden()["cic_particle_at_cell_centre"]
    M = oracle.assemble(c["order"], c["n"], c["origin"], c["h"], np.array(c["pos"]), np.array(c["w"]),
                        None, 0.0, c["sigma"])
    nz = M[M != 0]
    assert nz.size == c["nonzero_count"]
    assert np.all(nz == c["pair_value"])
    # the 8 corner nodes of cell (0,0,0) each hold 8 offsets
    nodes = np.nonzero(M.any(axis=(1, 2)))[0]
    n = c["n"]
    expect = sorted(ax + n[0] * (ay + n[1] * az) for ax in (0, 1) for ay in (0, 1) for az in (0, 1))
    assert list(nodes) == expect


def test_golden_tsc_on_node():
    c = _golden()["tsc_particle_on_node"]
    M = oracle.assemble(c["order"], c["n"], c["origin"], c["h"], np.array(c["pos"]), np.array(c["w"]),
                        None, 0.0, c["sigma"])
    cw = np.array(c["w1d"])
    n = c["n"]
    m = c["centre_node"]
    expect = np.zeros_like(M)
    for az in range(3):
        for ay in range(3):
            for ax in range(3):
                g = (m[0] - 1 + ax) + n[0] * ((m[1] - 1 + ay) + n[1] * (m[2] - 1 + az))
                for bz in range(3):
                    for by in range(3):
                        for bx in range(3):
                            o = (bx - ax + 2) + 5 * ((by - ay + 2) + 5 * (bz - az + 2))
                            expect[g, o, 0] += (cw[ax] * cw[bx]) * (cw[ay] * cw[by]) * (cw[az] * cw[bz])
    assert np.array_equal(M, expect)
    first, w1d = oracle.support(2, n, c["origin"], c["h"], np.array(c["pos"][0]))
    assert list(first) == [m[0] - 1, m[1] - 1, m[2] - 1]
    assert np.array_equal(w1d, np.tile(cw, (3, 1)))


@pytest.mark.parametrize("name", ["alpha_unit_field", "alpha_half_field_x"])
def test_golden_alpha(name):
    c = _golden()[name]
    a = oracle.alpha(np.array(c["B"]), c["beta"])
    assert np.array_equal(a, np.array(c["alpha"]))


# ---------------------------------------------------------------- alpha identities
def test_alpha_identities():
    rng = np.random.default_rng(5)
    for _ in range(200):
        B = rng.standard_normal(3) * rng.uniform(0.1, 5)
        beta = rng.uniform(-2, 2)
        a = oracle.alpha(B, beta)
        assert np.allclose(a, dense_ref.alpha_inv(B, beta), rtol=0, atol=1e-14)
        u = rng.standard_normal(3)
        # alpha undoes u -> u + beta * B x u
        assert np.allclose(a @ (u + beta * np.cross(B, u)), u, atol=1e-13)
        assert np.allclose(a @ B, B, atol=1e-13)
        assert np.allclose(a.T @ B, B, atol=1e-13)
    assert np.array_equal(oracle.alpha(np.zeros(3), 0.5), np.eye(3))


def test_ecsim_zero_field_is_scalar_bitwise():
    case = random_case(11, 2, (5, 6, 5), 60, kind="ecsim")
    sp = case.species[0]
    Ms = oracle.assemble(2, case.grid.n, case.grid.origin, case.grid.h, sp.pos, sp.w, None, 0.0, 1.5)
    Me = oracle.assemble(2, case.grid.n, case.grid.origin, case.grid.h, sp.pos, sp.w, np.zeros_like(sp.B), 0.8, 1.5)
    for c in range(9):
        i, j = divmod(c, 3)
        if i == j:
            assert np.array_equal(Me[:, :, c], Ms[:, :, 0])
        else:
            assert not np.any(Me[:, :, c])


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
def test_symmetry_bitwise(order, kind):
    n = (6, 5, 7) if order == 2 else (4, 5, 3)
    case = random_case(21 + order, order, n, 300, kind=kind)
    M = run_oracle(case)
    R = order
    NO = 2 * R + 1
    nx, ny, nz = n
    for g in range(nx * ny * nz):
        gx, gy, gz = g % nx, (g // nx) % ny, g // (nx * ny)
        for o in range(NO ** 3):
            ox, oy, oz = o % NO - R, (o // NO) % NO - R, o // (NO * NO) - R
            g2 = (gx + ox) % nx + nx * (((gy + oy) % ny) + ny * ((gz + oz) % nz))
            o2 = (-ox + R) + NO * ((-oy + R) + NO * (-oz + R))
            assert np.array_equal(M[g, o], M[g2, o2])


@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
def test_partition_of_unity(order, kind):
    n = (7, 6, 5)
    case = random_case(40 + order, order, n, 500, kind=kind, sigma=0.75, origin=(1.0, -2.0, 0.5), h=(0.3, 0.4, 0.5))
    sp = case.species[0]
    M = run_oracle(case)
    W = dense_ref.dense_W(order, n, case.grid.origin, case.grid.h, sp.pos)
    assert np.allclose(W.sum(axis=1), 1.0, atol=1e-14)
    if kind == "scalar":
        S = (case.sigma * sp.w)[:, None]
    else:
        S = np.stack([case.sigma * sp.w[p] * oracle.alpha(sp.B[p], sp.beta).reshape(-1) for p in range(sp.np)])
    rows = M.sum(axis=1)                      # [nnodes, ncomp]
    expect = W.T @ S                           # sigma sum_p s_p W_pg
    assert rel(rows, expect) < 1e-13
    assert rel(M.sum(axis=(0, 1)), S.sum(axis=0)) < 1e-13


def test_translation_by_whole_cells():
    n = (6, 5, 7)
    rng = np.random.default_rng(3)
    pos = np.floor(rng.random((200, 3)) * np.array(n) * 1024) / 1024  # exact under integer shifts
    w = rng.uniform(0.5, 1.5, 200)
    B = rng.standard_normal((200, 3))
    for order in (1, 2):
        M0 = oracle.assemble(order, n, (0, 0, 0), (1, 1, 1), pos, w, B, 0.5, 1.0)
        shift = np.array([2, 3, 0])
        M1 = oracle.assemble(order, n, (0, 0, 0), (1, 1, 1), pos + shift, w, B, 0.5, 1.0)
        nx, ny, nz = n
        M0g = M0.reshape(nz, ny, nx, *M0.shape[1:])
        M1g = M1.reshape(nz, ny, nx, *M1.shape[1:])
        assert np.array_equal(np.roll(M0g, shift=(0, 3, 2), axis=(0, 1, 2)), M1g)
        M2 = oracle.assemble(order, n, (0, 0, 0), (1, 1, 1), pos + np.array([0, 0, 4]), w, B, 0.5, 1.0)
        M2g = M2.reshape(nz, ny, nx, *M2.shape[1:])
        assert rel(np.roll(M0g, shift=4, axis=0), M2g) < 1e-15


def test_linearity_additivity_permutation():
    case = random_case(77, 2, (6, 6, 5), 400, kind="ecsim")
    sp = case.species[0]
    args = (2, case.grid.n, case.grid.origin, case.grid.h)
    M = oracle.assemble(*args, sp.pos, sp.w, sp.B, 0.5, 1.0)
    M1 = oracle.assemble(*args, sp.pos[:150], sp.w[:150], sp.B[:150], 0.5, 1.0)
    M2 = oracle.assemble(*args, sp.pos[150:], sp.w[150:], sp.B[150:], 0.5, 1.0, M=M1.copy(), accumulate=True)
    assert rel(M2, M) < 1e-14
    Mc = oracle.assemble(*args, sp.pos, 3.0 * sp.w, sp.B, 0.5, 1.0)
    assert rel(Mc, 3.0 * M) < 1e-15
    perm = np.random.default_rng(1).permutation(sp.np)
    Mp = oracle.assemble(*args, sp.pos[perm], sp.w[perm], sp.B[perm], 0.5, 1.0)
    assert rel(Mp, M) < 1e-14


def test_empty_and_accumulate_semantics():
    n = (5, 5, 5)
    M = oracle.assemble(1, n, (0, 0, 0), (1, 1, 1), np.zeros((0, 3)), np.zeros(0))
    assert M.shape == (125, 27, 1) and not M.any()
    M = np.full((125, 27, 9), 2.0)
    oracle.assemble(1, n, (0, 0, 0), (1, 1, 1), np.zeros((0, 3)), np.zeros(0), np.zeros((0, 3)), 0.5, 1.0,
                    M=M, accumulate=True)
    assert np.all(M == 2.0)


def test_thread_count_determinism():
    case = random_case(5, 1, (8, 8, 8), 4000, kind="ecsim")
    a = run_oracle(case, nthreads=1)
    b = run_oracle(case, nthreads=5)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- bilinear form and rows
@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
def test_bilinear_form(order, kind):
    n = (6, 7, 5)
    case = random_case(90 + order, order, n, 700, kind=kind)
    sp = case.species[0]
    M = run_oracle(case)
    rng = np.random.default_rng(9)
    nn = case.grid.ncells
    shp = (nn, 3) if kind == "ecsim" else (nn,)
    u, v = rng.standard_normal(shp), rng.standard_normal(shp)
    lhs = dense_ref.stencil_bilinear(order, n, M, u, v)
    rhs = oracle.bilinear(order, n, case.grid.origin, case.grid.h, sp.pos, sp.w, u, v,
                          sp.B if kind == "ecsim" else None, sp.beta, case.sigma)
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(rhs))
    if kind == "scalar":
        assert dense_ref.stencil_bilinear(order, n, M, u, u) >= 0.0


def test_rows_match_full():
    case = random_case(123, 2, (6, 6, 6), 900, kind="ecsim")
    sp = case.species[0]
    M = run_oracle(case)
    nodes = np.array([0, 5, 17, 100, 215, 17])
    r = oracle.rows(2, case.grid.n, case.grid.origin, case.grid.h, sp.pos, sp.w, nodes, sp.B, sp.beta, case.sigma)
    assert rel(r, M[nodes]) < 1e-14


# ---------------------------------------------------------------- binning
@pytest.mark.parametrize("order", [1, 2])
def test_binning_stable_and_supports(order):
    n = (7, 5, 6)
    case = random_case(300 + order, order, n, 2000, kind="scalar", origin=(0.5, -1.0, 2.0), h=(0.7, 1.1, 0.9))
    pos = case.species[0].pos
    bs, perm = oracle.bin_particles(order, n, case.grid.origin, case.grid.h, pos)
    nb = case.grid.ncells
    assert bs[0] == 0 and bs[nb] == len(pos) and np.all(np.diff(bs) >= 0)
    assert sorted(perm) == list(range(len(pos)))
    W = dense_ref.dense_W(order, n, case.grid.origin, case.grid.h, pos)
    nx, ny, nz = n
    for k in range(nb):
        mem = perm[bs[k]:bs[k + 1]]
        assert np.all(np.diff(mem) > 0)  # stable: ascending particle index within a bin
        kx, ky, kz = k % nx, (k // nx) % ny, k // (nx * ny)
        allowed = set()
        for az in range(order + 1):
            for ay in range(order + 1):
                for ax in range(order + 1):
                    allowed.add((kx + ax) % nx + nx * (((ky + ay) % ny) + ny * ((kz + az) % nz)))
        for p in mem:
            supp = set(np.nonzero(W[p] > 0)[0])
            assert supp <= allowed


def _fp32_faces():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "fp32_faces.json")) as f:
        return json.load(f)


def test_fp32_positions_decided_exactly():
    """fp32 positions are placed as their exact values are (Sec. 2.3 support
    rule on the stored value): next to a cell face or a TSC half-cell tie,
    where fp32 arithmetic on the quotient would land on the face or the tie,
    the oracle's cell, fraction and TSC centre equal the exact rational ones
    (tests/golden/fp32_faces.json, written by make_fp32_faces.py with
    fractions.Fraction, never by the oracle), and each case contradicts the
    fp32-arithmetic reading."""
    from fractions import Fraction
    d = _fp32_faces()
    assert len(d["faces"]) >= 4 and len(d["ties"]) >= 4
    for c in d["faces"]:
        n = (c["n"],) * 3
        x = np.array([float.fromhex(c["x_hex"]), 0.0, 0.0], dtype=np.float64)
        assert np.float32(x[0]) == x[0]  # an fp32 value
        first, w1d = oracle.support(1, n, (c["origin"],) * 3, (c["h"],) * 3, x)
        assert first[0] == c["exact_cell"] != c["fp32_cell"]
        xi = Fraction(c["exact_xi"])
        assert abs(Fraction(w1d[0, 1]) - xi) <= Fraction(1, 2 ** 50)
        assert abs(Fraction(w1d[0, 0]) - (1 - xi)) <= Fraction(1, 2 ** 50)
    for c in d["ties"]:
        n = (c["n"],) * 3
        x = np.array([float.fromhex(c["x_hex"]), 0.0, 0.0], dtype=np.float64)
        first, w1d = oracle.support(2, n, (c["origin"],) * 3, (c["h"],) * 3, x)
        assert c["exact_tsc_centre"] != c["fp32_tsc_centre"]
        assert first[0] == (c["exact_tsc_centre"] - 1) % c["n"]
        # centred on j (xi just below 1/2): delta = xi, so the upper weight 1/2 (1/2 + delta)^2 is just below 1/2
        delta = Fraction(c["exact_xi"])
        assert abs(Fraction(w1d[0, 2]) - Fraction(1, 2) * (Fraction(1, 2) + delta) ** 2) <= Fraction(1, 2 ** 50)
        # binning keys follow the same decision
        bs, perm = oracle.bin_particles(2, n, (c["origin"],) * 3, (c["h"],) * 3, x[None, :])
        key = int(np.searchsorted(bs, 0, side="right") - 1)
        assert key % c["n"] == (c["exact_tsc_centre"] - 1) % c["n"]


def test_config_generators_shapes():
    c1 = make_config(1)
    assert c1.np_total == 32768 and c1.order == 1 and c1.kind == "scalar"
    assert np.all(c1.species[0].w >= 0.5) and np.all(c1.species[0].w < 1.5)
    c4 = make_config(4, kind="scalar", scale=8)
    assert c4.order == 2 and c4.np_total == 64 * 512
    c3 = make_config(3, scale=8, shuffled=True)
    assert len(c3.species) == 2 and c3.species[0].beta == -0.5
    assert abs(c3.species[1].beta - 0.5 / 1836) < 1e-18
    assert c3.np_total == 125 * 512


# ---------------------------------------------------------------- grid field gathered at the particles
def _field(seed, n):
    return np.random.default_rng(seed).normal(size=(int(np.prod(n)), 3))


@pytest.mark.parametrize("order,n", [(1, (3, 4, 5)), (1, (6, 5, 4)), (2, (5, 5, 5)), (2, (7, 6, 5))])
def test_interp_field_dense(order, n):
    """B_p = sum_a W_pa F[g_a] against the dense interpolation matrix (wrapped
    distances, no first-support-node logic), with particles shifted by whole
    periods."""
    case = random_case(41 + order + n[0], order, n, 60, kind="scalar", origin=(-0.25, 0.5, 1.0), h=(0.5, 1.25, 2.0))
    pos = case.species[0].pos.copy()
    pos[::2, 1] += 3 * n[1] * case.grid.h[1]
    pos[1::4, 0] -= 2 * n[0] * case.grid.h[0]
    F = _field(5 + order, n)
    got = oracle.interp_field(order, n, case.grid.origin, case.grid.h, pos, F)
    ref = dense_ref.dense_W(order, n, case.grid.origin, case.grid.h, pos) @ F
    assert rel(got, ref) < 1e-14
    # a swapped pair of field components or a node shifted by one fails it
    assert rel(got, dense_ref.dense_W(order, n, case.grid.origin, case.grid.h, pos) @ F[:, [1, 0, 2]]) > 1e-2
    assert rel(got, dense_ref.dense_W(order, n, case.grid.origin, case.grid.h, pos) @ np.roll(F, 1, axis=0)) > 1e-2


@pytest.mark.parametrize("order", [1, 2])
def test_interp_field_constant_and_linear(order):
    """Partition of unity: a constant field comes back unchanged. Linear
    reproduction: both B-splines reproduce a + G x for particles whose support
    does not cross the periodic boundary."""
    n = (9, 8, 10)
    origin, h = (1.0, -2.0, 0.5), (0.5, 0.25, 2.0)
    rng = np.random.default_rng(11 + order)
    u = 2.0 + rng.random((200, 3)) * (np.array(n) - 5.0)  # grid units, away from the wrap
    pos = np.asarray(origin) + u * np.asarray(h)
    c = np.array([0.3, -1.7, 2.5])
    got = oracle.interp_field(order, n, origin, h, pos, np.tile(c, (int(np.prod(n)), 1)))
    assert np.max(np.abs(got - c)) < 1e-14
    k = np.arange(int(np.prod(n)))
    xn = np.stack([origin[0] + h[0] * (k % n[0]), origin[1] + h[1] * ((k // n[0]) % n[1]),
                   origin[2] + h[2] * (k // (n[0] * n[1]))], axis=1)
    G = rng.normal(size=(3, 3))
    got = oracle.interp_field(order, n, origin, h, pos, c + xn @ G.T)
    assert np.max(np.abs(got - (c + pos @ G.T))) < 1e-12


def test_interp_field_cic_on_node_exact():
    """A CIC particle on a node takes that node's value exactly."""
    n = (4, 5, 6)
    F = _field(3, n)
    pos = np.array([[2.0, 3.0, 1.0], [0.0, 0.0, 0.0]])
    got = oracle.interp_field(1, n, (0, 0, 0), (1, 1, 1), pos, F)
    assert np.array_equal(got[0], F[2 + 4 * (3 + 5 * 1)]) and np.array_equal(got[1], F[0])


@pytest.mark.parametrize("order,n", [(1, (4, 5, 3)), (2, (6, 5, 7))])
def test_grid_field_assembly_dense(order, n):
    """Tensorial assembly with the field gathered from the grid: the oracle
    (gather, then Eq. 6) against the dense form W^T diag(sigma w alpha(W F)) W."""
    case = random_case(71 + order, order, n, 40, kind="ecsim", beta=0.6, sigma=0.9,
                       origin=(-0.25, 0.5, 1.0), h=(0.5, 1.25, 2.0))
    sp = case.species[0]
    F = _field(9, n)
    Bp = oracle.interp_field(order, n, case.grid.origin, case.grid.h, sp.pos, F)
    M = oracle.assemble(order, n, case.grid.origin, case.grid.h, sp.pos, sp.w, Bp, sp.beta, case.sigma)
    Wd = dense_ref.dense_W(order, n, case.grid.origin, case.grid.h, sp.pos)
    Md = dense_ref.dense_M(order, n, case.grid.origin, case.grid.h, sp.pos, sp.w, Wd @ F, sp.beta, case.sigma)
    assert rel(M, dense_ref.dense_to_stencil(order, n, Md)) < 1e-14


# ---------------------------------------------------------------- canonical half and stencil product
@pytest.mark.parametrize("order,n", [(1, (3, 4, 5)), (2, (5, 6, 7))])
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
def test_stencil_matvec_dense(order, n, kind):
    """y = M x read off the stencil storage equals the dense product built by
    brute force (tests/dense_ref.py), for scalar and 3x3 blocks."""
    case = random_case(81 + order, order, n, 50, kind=kind, beta=0.6, sigma=1.1,
                       origin=(-0.25, 0.5, 1.0), h=(0.5, 1.25, 2.0))
    sp = case.species[0]
    M = run_oracle(case)
    Md = dense_ref.dense_M(order, n, case.grid.origin, case.grid.h, sp.pos, sp.w,
                           sp.B if kind == "ecsim" else None, sp.beta, case.sigma)
    nn = case.grid.ncells
    rng = np.random.default_rng(5)
    if kind == "ecsim":
        x = rng.normal(size=(nn, 3))
        # dense [3 nn, 3 nn] operator with block (g, g') = M^{ij}_{g g'}
        D = Md.reshape(3, 3, nn, nn).transpose(2, 0, 3, 1).reshape(3 * nn, 3 * nn)
        ref = (D @ x.reshape(-1)).reshape(nn, 3)
    else:
        x = rng.normal(size=nn)
        ref = Md[0] @ x
    got = oracle.stencil_matvec(order, n, M, x)
    assert rel(got, ref) < 1e-14
    # the (i, j) blocks transposed give another product
    if kind == "ecsim":
        Mt = M.reshape(nn, -1, 3, 3).transpose(0, 1, 3, 2).reshape(M.shape)
        assert rel(oracle.stencil_matvec(order, n, Mt, x), ref) > 1e-3


@pytest.mark.parametrize("order,n", [(1, (4, 5, 3)), (2, (6, 5, 7))])
def test_canonical_half_roundtrip(order, n):
    """The canonical half holds (noff + 1) / 2 offsets (14 or 63) and, with the
    spatial symmetry M[g][-o] = M[g-o][o], gives back the full stencil bitwise."""
    case = random_case(91 + order, order, n, 300, kind="ecsim", beta=0.5)
    M = run_oracle(case)
    Mc = oracle.canonical_half(order, M)
    assert Mc.shape[1] == {1: 14, 2: 63}[order]
    assert np.array_equal(oracle.full_from_canonical(order, n, Mc), M)
    # a canonical half from the wrong side of the centre does not round-trip
    bad = np.ascontiguousarray(M[:, :Mc.shape[1], :])
    assert not np.allclose(oracle.full_from_canonical(order, n, bad), M)


# ---------------------------------------------------------------- moment deposition
@pytest.mark.parametrize("order,n", [(1, (3, 4, 5)), (2, (5, 6, 7))])
@pytest.mark.parametrize("nq", [1, 4, 10])
def test_moments_dense(order, n, nq):
    """m = W^T Q against the dense interpolation matrix (wrapped distances),
    particles shifted by whole periods; a swapped pair of quantities or nodes
    shifted by one fail it."""
    case = random_case(111 + order + nq, order, n, 70, kind="scalar", origin=(-0.25, 0.5, 1.0), h=(0.5, 1.25, 2.0))
    pos = case.species[0].pos.copy()
    pos[::3, 2] += 2 * n[2] * case.grid.h[2]
    Q = np.random.default_rng(nq).normal(size=(len(pos), nq))
    got = oracle.moments(order, n, case.grid.origin, case.grid.h, pos, Q)
    W = dense_ref.dense_W(order, n, case.grid.origin, case.grid.h, pos)
    assert rel(got, W.T @ Q) < 1e-14
    if nq > 1:
        assert rel(got, W.T @ Q[:, ::-1]) > 1e-2
    assert rel(got, np.roll(W.T @ Q, 1, axis=0)) > 1e-2


@pytest.mark.parametrize("order", [1, 2])
def test_moments_charge_conservation_and_node(order):
    """Partition of unity: the deposited total of each quantity is the particle
    total; a CIC particle on a node puts its quantities on that node exactly."""
    case = random_case(121 + order, order, (6, 5, 7), 500, kind="scalar")
    Q = np.random.default_rng(2).uniform(0.5, 1.5, size=(500, 4))
    m = oracle.moments(order, case.grid.n, case.grid.origin, case.grid.h, case.species[0].pos, Q)
    assert np.max(np.abs(m.sum(axis=0) - Q.sum(axis=0))) < 1e-12 * Q.sum()
    if order == 1:
        q = np.array([[1.5, -2.0, 0.25, 3.0]])
        m1 = oracle.moments(1, (4, 5, 6), (0, 0, 0), (1, 1, 1), np.array([[2.0, 3.0, 1.0]]), q)
        assert np.array_equal(m1[2 + 4 * (3 + 5 * 1)], q[0]) and np.count_nonzero(m1) == 4


# ---------------------------------------------------------------- 2D (n[2] == 1)
@pytest.mark.parametrize("order,n", [(1, (3, 4, 1)), (1, (5, 4, 1)), (2, (5, 6, 1)), (2, (7, 5, 1))])
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
def test_dense_bruteforce_2d(order, n, kind):
    """The 2D problem (z ignored, (R+1)^2 support, (2R+1)^2 offsets) against
    the dense brute force with one node plane; the 2D stencil has 9 or 25
    offsets and is symmetric, M[g][o] = M[g+o][-o]."""
    case = random_case(181 + order + n[0], order, n, 60, kind=kind, beta=0.6, sigma=1.2,
                       origin=(-0.25, 0.5, 1.0), h=(0.5, 1.25, 2.0))
    sp = case.species[0]
    pos = sp.pos.copy()
    pos[::2, 2] += 17.3  # z is ignored
    M = oracle.assemble(order, n, case.grid.origin, case.grid.h, pos, sp.w, sp.B if kind == "ecsim" else None,
                        sp.beta, case.sigma)
    assert M.shape[1] == (2 * order + 1) ** 2
    Md = dense_ref.dense_M(order, n, case.grid.origin, case.grid.h, pos, sp.w, sp.B if kind == "ecsim" else None,
                           sp.beta, case.sigma)
    assert rel(M, dense_ref.dense_to_stencil(order, n, Md)) < 1e-14
    NO = 2 * order + 1
    g = np.arange(case.grid.ncells)
    gx, gy = g % n[0], g // n[0]
    for o in range(NO * NO):
        ox, oy = o % NO - order, o // NO - order
        g2 = (gx + ox) % n[0] + n[0] * ((gy + oy) % n[1])
        assert np.array_equal(M[g, o], M[g2, (NO * NO - 1) - o])


@pytest.mark.parametrize("order", [1, 2])
def test_binning_2d_keys(order):
    """2D keys ignore z: a particle's bin is its first support node in the plane."""
    case = random_case(191 + order, order, (6, 7, 1), 500, kind="scalar")
    pos = case.species[0].pos.copy()
    pos[:, 2] = np.random.default_rng(1).normal(size=500) * 100
    bs, perm = oracle.bin_particles(order, case.grid.n, case.grid.origin, case.grid.h, pos)
    assert bs[-1] == 500 and len(bs) == 43
    bs0, perm0 = oracle.bin_particles(order, case.grid.n, case.grid.origin, case.grid.h, case.species[0].pos)
    assert np.array_equal(bs, bs0) and np.array_equal(perm, perm0)
