"""GPU parity at the positions where the support rule makes its decisions.

Sec. 2.3 of the page places the CIC support on the two corners of the cell
(j = floor(u)) and centres the TSC support on the nearest node, the tie
xi = 1/2 going up. The random workloads almost never put a particle exactly
on a node, a cell face, the TSC tie or the periodic boundary; these tests do,
on purpose, and several periods outside the box, through every assembly
algorithm, both orders, both kinds and both precisions. Positions are chosen
so that (x - origin)/h is exact in binary (dyadic offsets and spacings), and
also with a spacing that is not, where both sides must take the same IEEE
quotient. A last group puts fp32 positions next to a face or a tie where
fp32 arithmetic would decide otherwise than the exact value
(tests/golden/fp32_faces.json).

Integer results (bins) are compared bit for bit; matrices by relative
Frobenius error and by the largest entry error.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import particle_grid_mass_amd as mm
from tests.gpu_util import TDT, as_numpy_M, assert_match, gpu_assemble, oracle_assemble, require_gpu, to_dev
from workloads import Case, Grid, Species

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


# grid coordinate u = (x - origin)/h per axis, relative to a node k: on the node,
# a quarter, the TSC tie, just below and above it, three quarters, and the
# far face; and the same several periods outside the box
FRACS = [0.0, 0.25, 0.5, 0.5 - 2.0 ** -20, 0.5 + 2.0 ** -20, 0.75, 1.0 - 2.0 ** -30]
PERIODS = [0, 0, 0, 1, -1, 3, -4]

SPACINGS = {
    "pow2": ((-1.5, 0.25, 2.0), (0.5, 2.0, 0.25)),     # (x - o) * (1/h) path, exact
    "dyadic": ((0.25, -2.0, 1.0), (0.75, 1.25, 0.375)),  # IEEE division, exact quotients
    "inexact": ((0.1, -0.7, 0.3), (0.3, 0.7, 1.1)),     # IEEE division, rounded quotients
}


def edge_case(seed, order, kind, dtype, spacing, n=(7, 6, 8), npart=400):
    """Particles at the decision points of the support rule on grid n (an x
    extent of 8 sends second-order fp64 3x3 records through the run records,
    7 through the per-bin ones)."""
    origin, h = SPACINGS[spacing]
    rng = np.random.default_rng(seed)
    pos = np.empty((npart, 3))
    for d in range(3):
        k = rng.integers(0, n[d], npart)
        f = np.array(FRACS)[rng.integers(0, len(FRACS), npart)]
        per = np.array(PERIODS)[rng.integers(0, len(PERIODS), npart)]
        u = k + f + per * n[d]
        u[::37] = n[d]          # exactly on the far boundary: wraps to node 0
        u[5::41] = -n[d]        # one period below the origin, on a node
        pos[:, d] = origin[d] + u * h[d]
    w = rng.uniform(0.5, 1.5, npart)
    B = rng.standard_normal((npart, 3)) if kind == "ecsim" else None
    if dtype == "f32":
        pos, w = pos.astype(np.float32), w.astype(np.float32)
        B = None if B is None else B.astype(np.float32)
    sp = Species(pos, w, B, 0.6, "edges")
    return Case(f"edges_{spacing}_o{order}_{kind}_{dtype}", Grid(n, origin, h), order, kind, [sp], sigma=1.2,
                dtype=dtype)


@pytest.mark.parametrize("spacing", sorted(SPACINGS))
@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("order", [1, 2])
def test_edge_binning(order, dtype, spacing):
    case = edge_case(100 + order, order, "scalar", dtype, spacing)
    sp = case.species[0]
    print(f"[case] {case.name} binning", flush=True)
    bs_ref, perm_ref = oracle.bin_particles(order, case.grid.n, case.grid.origin, case.grid.h, sp.pos)
    bs, perm = mm.bin_particles(case.grid, order, to_dev(sp.pos, TDT[dtype]))
    torch.cuda.synchronize()
    assert np.array_equal(bs.cpu().numpy(), bs_ref)
    assert np.array_equal(perm.cpu().numpy(), perm_ref)


@pytest.mark.parametrize("algo", ["mfma", "mfma_atomic", "atomic"])
@pytest.mark.parametrize("spacing", sorted(SPACINGS))
@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("kind", ["scalar", "ecsim"])
@pytest.mark.parametrize("order,n", [(1, (7, 6, 8)), (2, (7, 6, 8)), (2, (8, 6, 7))])
def test_edge_assembly(order, n, kind, dtype, spacing, algo):
    case = edge_case(200 + order, order, kind, dtype, spacing, n=n)
    print(f"[case] {case.name} {algo}", flush=True)
    M = as_numpy_M(gpu_assemble(case, algo), case)
    assert_match(M, oracle_assemble(case), dtype)


@pytest.mark.parametrize("spacing", sorted(SPACINGS))
@pytest.mark.parametrize("order,n", [(1, (7, 6, 8)), (2, (7, 6, 8)), (2, (8, 6, 7))])
def test_edge_mixed_layout(order, n, spacing):
    """fp32 positions and field with fp64 weights and matrix (the production
    layout): every decision in fp64 on the fp32 values, held to the fp64 budget."""
    case = edge_case(300 + order, order, "ecsim", "f64", spacing, n=n)
    sp = case.species[0]
    p32, b32 = sp.pos.astype(np.float32), sp.B.astype(np.float32)
    print(f"[case] {case.name} mixed", flush=True)
    pos, w, B = to_dev(p32, torch.float32), to_dev(sp.w, torch.float64), to_dev(b32, torch.float32)
    bs, perm = mm.bin_particles(case.grid, order, pos, mixed=True)
    M = mm.assemble_ecsim(case.grid, order, pos, w, B, bs, perm, beta=sp.beta, sigma=case.sigma)
    torch.cuda.synchronize()
    ref = oracle.assemble(order, case.grid.n, case.grid.origin, case.grid.h, p32, sp.w, b32, sp.beta, case.sigma)
    bs_ref, perm_ref = oracle.bin_particles(order, case.grid.n, case.grid.origin, case.grid.h, p32)
    assert np.array_equal(bs.cpu().numpy(), bs_ref) and np.array_equal(perm.cpu().numpy(), perm_ref)
    assert_match(as_numpy_M(M, case), ref, "f64")


def _faces():
    with open(os.path.join(os.path.dirname(__file__), "golden", "fp32_faces.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("algo", ["mfma", "mfma_atomic", "atomic"])
@pytest.mark.parametrize("order", [1, 2])
def test_fp32_faces_and_ties(order, algo):
    """fp32 positions next to a face (CIC) or a tie (TSC) where fp32 arithmetic
    would move the particle to the next cell or centre: the fp32 path places
    them as their exact values are, like the oracle, bin for bin."""
    d = _faces()
    cases = d["faces"] if order == 1 else d["ties"]
    rng = np.random.default_rng(7 + order)
    for c in cases:
        n = (c["n"],) * 3
        g = Grid(n, (c["origin"],) * 3, (c["h"],) * 3)
        npart = 64
        x = np.float32(float.fromhex(c["x_hex"]))
        pos = np.empty((npart, 3), dtype=np.float32)
        pos[:, 0] = x
        pos[:, 1:] = (np.float32(c["origin"]) + rng.integers(0, c["n"], (npart, 2)).astype(np.float32)
                      * np.float32(c["h"]) + np.float32(0.37) * np.float32(c["h"]))
        pos[::2, 1] = x  # the same near-face coordinate on a second axis
        w = rng.uniform(0.5, 1.5, npart).astype(np.float32)
        B = rng.standard_normal((npart, 3)).astype(np.float32)
        case = Case(f"fp32_face_{c['target']}", g, order, "ecsim", [Species(pos, w, B, 0.5)], dtype="f32")
        print(f"[case] fp32 {'face' if order == 1 else 'tie'} x={c['x_hex']} h={c['h']} {algo}", flush=True)
        if algo != "atomic":
            bs_ref, perm_ref = oracle.bin_particles(order, n, g.origin, g.h, pos)
            bs, perm = mm.bin_particles(g, order, to_dev(pos, torch.float32))
            torch.cuda.synchronize()
            assert np.array_equal(bs.cpu().numpy(), bs_ref) and np.array_equal(perm.cpu().numpy(), perm_ref)
        M = as_numpy_M(gpu_assemble(case, algo), case)
        assert_match(M, oracle_assemble(case), "f32")
