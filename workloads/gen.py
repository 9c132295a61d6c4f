"""Seeded input generators (no assembly arithmetic lives here).

Every array is drawn with numpy's PCG64 from ``SeedSequence(seed)``; each
array kind has its own spawned stream so sizes can change without shifting
the other draws. Positions are ``origin + (cell + U[0,1)) * h`` per axis,
cell-major (x fastest), so a uniform workload is sorted by cell.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Grid:
    """Periodic grid: ``n`` cells (= nodes) per axis, nodes at ``origin + k*h``."""
    n: Tuple[int, int, int]
    origin: Tuple[float, float, float] = (0.0, 0.0, 0.0)
    h: Tuple[float, float, float] = (1.0, 1.0, 1.0)

    @property
    def ncells(self) -> int:
        return int(self.n[0]) * int(self.n[1]) * int(self.n[2])


@dataclasses.dataclass
class Species:
    """One particle species: positions ``[np,3]``, weights ``[np]``, field ``[np,3]``."""
    pos: np.ndarray
    w: np.ndarray
    B: Optional[np.ndarray]
    beta: float = 0.0
    name: str = "species"

    @property
    def np(self) -> int:
        return int(self.pos.shape[0])


@dataclasses.dataclass
class Case:
    """A complete workload: grid, interpolation order, kind and species."""
    name: str
    grid: Grid
    order: int                 # 1 = CIC, 2 = TSC
    kind: str                  # "scalar" or "ecsim"
    species: List[Species]
    sigma: float = 1.0
    dtype: str = "f64"         # "f64" or "f32" (fp32 variants round the fp64 draws)
    seed: int = 0
    note: str = ""

    @property
    def np_total(self) -> int:
        return sum(s.np for s in self.species)


def _streams(seed: int, k: int = 6):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(k)]


def _round(a: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    if a is None or dtype == "f64":
        return a
    return a.astype(np.float32)


def positions_f32(pos: np.ndarray, grid: "Grid") -> np.ndarray:
    """Positions rounded to float32 without leaving the cell they were drawn
    in. Rounding to nearest can put a value drawn just below a cell's upper
    face onto that face, i.e. into the next cell (a few particles per
    million), which would break the cell order of a cell-sorted draw; such a
    value takes the float32 just below the face instead."""
    p32 = pos.astype(np.float32)
    for d in range(3):
        o, h = grid.origin[d], grid.h[d]
        face = np.floor((pos[:, d] - o) / h) + 1.0  # upper face of the drawn cell, in cells
        over = (p32[:, d].astype(np.float64) - o) / h >= face
        p32[over, d] = np.nextafter(p32[over, d], np.float32(-np.inf))
    return p32


def species_from_counts(grid: Grid, counts: np.ndarray, rng_pos, rng_w, rng_b, with_B: bool, beta: float,
                        name: str, w_range=(0.5, 1.5)) -> Species:
    """Particles cell by cell with ``counts[cell]`` per cell, uniform inside each cell."""
    counts = np.asarray(counts, dtype=np.int64)
    nx, ny, nz = grid.n
    npart = int(counts.sum())
    cell = np.repeat(np.arange(grid.ncells, dtype=np.int64), counts)
    pos = np.empty((npart, 3), dtype=np.float64)
    u = rng_pos.random((npart, 3))
    ci = (cell % nx, (cell // nx) % ny, cell // (nx * ny))
    for d in range(3):
        pos[:, d] = grid.origin[d] + (ci[d] + u[:, d]) * grid.h[d]
    del u, cell
    w = rng_w.uniform(w_range[0], w_range[1], size=npart)
    B = rng_b.standard_normal((npart, 3)) if with_B else None
    return Species(pos=pos, w=w, B=B, beta=beta, name=name)


def uniform_species(grid: Grid, ppc: int, seed: int, with_B: bool, beta: float = 0.5,
                    name: str = "species") -> Species:
    rp, rw, rb = _streams(seed, 3)
    counts = np.full(grid.ncells, ppc, dtype=np.int64)
    return species_from_counts(grid, counts, rp, rw, rb, with_B, beta, name)


def clustered_counts(n: int, mean: float, seed: int, sigma_cells: float = 16.0, cap_factor: float = 4.0,
                     centres=None) -> np.ndarray:
    """Per-cell counts from a capped sum of periodic Gaussians, drawn multinomially.

    Density lambda(c) = min(A * sum_k exp(-d_k^2 / (2 sigma^2)), cap_factor*mean),
    d_k the periodic minimum-image distance from the cell centre to centre k;
    A is found by bisection so that sum(lambda) = mean * n^3; the counts are
    one multinomial draw of exactly mean * n^3 particles with p ~ lambda.
    """
    if centres is None:
        q = n / 4.0
        centres = [(q, q, q), (3 * q, 3 * q, q), (3 * q, q, 3 * q), (q, 3 * q, 3 * q)]
    c = np.arange(n, dtype=np.float64) + 0.5
    total = np.zeros((n, n, n))  # indexed [z, y, x]
    for (cx, cy, cz) in centres:
        def dd(v, cc):
            d = np.abs(v - cc)
            d = np.minimum(d, n - d)
            return d * d
        dx2, dy2, dz2 = dd(c, cx), dd(c, cy), dd(c, cz)
        total += np.exp(-(dz2[:, None, None] + dy2[None, :, None] + dx2[None, None, :]) / (2 * sigma_cells ** 2))
    target = mean * n ** 3
    cap = cap_factor * mean
    lo, hi = 0.0, 1.0
    while np.minimum(hi * total, cap).sum() < target:
        hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.minimum(mid * total, cap).sum() < target:
            lo = mid
        else:
            hi = mid
    lam = np.minimum(hi * total, cap).reshape(-1)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(8)[7]))
    counts = rng.multinomial(int(round(target)), lam / lam.sum())
    return counts.astype(np.int64)


# Named configurations (sizes, orders and constants of the five workloads).
WORKLOAD_NOTES = {
    1: "CIC scalar fp64, 8^3 cells, 64 ppc uniform (32,768 particles)",
    2: "CIC ECSIM fp64, 32^3 cells, 64 ppc uniform (2,097,152 particles), beta=0.5",
    3: "CIC ECSIM fp64, 64^3 cells, 125 ppc, two species (electrons beta=-0.5, ions beta=+1/3672), "
       "cell-sorted or shuffled",
    4: "TSC scalar or ECSIM fp64, 32^3 cells, 64 ppc uniform (2,097,152 particles), beta=0.5",
    5: "TSC ECSIM, 128^3 cells, mean 64 ppc Gaussian-clustered (134,217,728 particles), beta=0.5, fp64 or fp32",
}


def make_config(cid: int, kind: Optional[str] = None, dtype: str = "f64", shuffled: bool = False,
                scale: Optional[int] = None, ppc: Optional[int] = None) -> Case:
    """Build named configuration ``cid`` (1..5).

    ``kind`` picks scalar/ecsim where a config offers both (config 4);
    ``scale`` replaces the grid edge (same ppc and constants) for reduced runs;
    ``ppc`` replaces the particles per cell of the uniform configurations
    (1, 2 and 4), for sweeps over the particle density.
    """
    if ppc is not None and cid not in (1, 2, 4):
        raise ValueError("ppc applies to the uniform configurations 1, 2 and 4")
    seed = 1000 + cid
    if cid == 1:
        g = Grid((8, 8, 8) if scale is None else (scale,) * 3)
        sp = uniform_species(g, ppc or 64, seed, with_B=False, beta=0.0)
        return Case("c1_cic_scalar", g, 1, "scalar", [sp], dtype="f64", seed=seed, note=WORKLOAD_NOTES[1])
    if cid == 2:
        g = Grid((32, 32, 32) if scale is None else (scale,) * 3)
        sp = uniform_species(g, ppc or 64, seed, with_B=True, beta=0.5)
        sp = Species(sp.pos, sp.w, sp.B, 0.5, "electrons")
        return Case("c2_cic_ecsim", g, 1, "ecsim", [_cast(sp, dtype, g)], dtype=dtype, seed=seed, note=WORKLOAD_NOTES[2])
    if cid == 3:
        g = Grid((64, 64, 64) if scale is None else (scale,) * 3)
        ppc = 125
        rp, rw, rb, rperm, _, _ = _streams(seed, 6)
        counts = np.full(g.ncells, ppc, dtype=np.int64)
        allp = species_from_counts(g, counts, rp, rw, rb, True, 0.0, "all")
        idx = np.arange(allp.np)
        species = []
        for parity, name, beta in ((0, "electrons", -0.5), (1, "ions", 0.5 / 1836.0)):
            sel = idx[idx % 2 == parity]
            if shuffled:
                sel = sel[rperm.permutation(sel.shape[0])]
            species.append(_cast(Species(allp.pos[sel], allp.w[sel], allp.B[sel], beta, name), dtype, g))
        return Case("c3_cic_ecsim_2sp" + ("_shuffled" if shuffled else "_sorted"), g, 1, "ecsim", species,
                    dtype=dtype, seed=seed, note=WORKLOAD_NOTES[3])
    if cid == 4:
        kind = kind or "ecsim"
        g = Grid((32, 32, 32) if scale is None else (scale,) * 3)
        sp = uniform_species(g, ppc or 64, seed, with_B=(kind == "ecsim"), beta=0.5)
        return Case(f"c4_tsc_{kind}", g, 2, kind, [_cast(sp, dtype, g)], dtype=dtype, seed=seed, note=WORKLOAD_NOTES[4])
    if cid == 5:
        n = 128 if scale is None else scale
        g = Grid((n, n, n))
        counts = clustered_counts(n, 64.0, seed, sigma_cells=16.0 * n / 128.0)
        rp, rw, rb = _streams(seed, 3)
        sp = species_from_counts(g, counts, rp, rw, rb, True, 0.5, "electrons")
        return Case(f"c5_tsc_ecsim_clustered_{dtype}", g, 2, "ecsim", [_cast(sp, dtype, g)], dtype=dtype, seed=seed,
                    note=WORKLOAD_NOTES[5])
    raise ValueError(f"unknown config {cid}")


def _cast(sp: Species, dtype: str, grid: Optional["Grid"] = None) -> Species:
    """The species in the storage dtype; with a grid, float32 positions stay
    in the cells they were drawn in (positions_f32)."""
    pos = positions_f32(sp.pos, grid) if (dtype == "f32" and grid is not None) else _round(sp.pos, dtype)
    return Species(pos, _round(sp.w, dtype), _round(sp.B, dtype), sp.beta, sp.name)


def random_case(seed: int, order: int, n: Tuple[int, int, int], npart: int, kind: str = "ecsim",
                beta: float = 0.5, sigma: float = 1.0, dtype: str = "f64",
                origin=(0.0, 0.0, 0.0), h=(1.0, 1.0, 1.0), spread: float = 1.0,
                sorted_by_cell: bool = False) -> Case:
    """Small random case: ``npart`` particles uniform over the box (or over a
    ``spread`` fraction of it, to leave cells empty), optionally cell-sorted."""
    rp, rw, rb, rs = _streams(seed, 4)
    g = Grid(tuple(int(v) for v in n), tuple(float(v) for v in origin), tuple(float(v) for v in h))
    u = rp.random((npart, 3)) * spread
    pos = np.empty((npart, 3))
    for d in range(3):
        pos[:, d] = g.origin[d] + u[:, d] * g.n[d] * g.h[d]
    if sorted_by_cell and npart:
        cell = np.floor(u[:, 0] * g.n[0]) + g.n[0] * (np.floor(u[:, 1] * g.n[1]) + g.n[1] * np.floor(u[:, 2] * g.n[2]))
        pos = pos[np.argsort(cell, kind="stable")]
    w = rw.uniform(0.5, 1.5, size=npart)
    B = rb.standard_normal((npart, 3)) if kind == "ecsim" else None
    sp = _cast(Species(pos, w, B, beta, "random"), dtype)
    return Case(f"random_s{seed}_o{order}_{kind}", g, order, kind, [sp], sigma=sigma, dtype=dtype, seed=seed)


def grid_field(grid: Grid, seed: int, dtype: str = "f64") -> np.ndarray:
    """Magnetic field on the grid nodes, ``[nnodes, 3]``: N(0, 1) per node and
    component (the per-particle field of the configurations, moved to the
    nodes), node index x + nx*(y + ny*z). Drawn from its own seeded stream."""
    (rng,) = _streams(7000 + seed, 1)
    return _round(rng.standard_normal((grid.ncells, 3)), dtype)


def make_2d(n: int = 256, ppc: int = 64, order: int = 1, kind: str = "ecsim", dtype: str = "f64",
            seed: int = 2002) -> Case:
    """The 2D problem (one node plane): an n x n periodic grid with ``ppc``
    particles per cell, cell-major, z of every particle inside the single
    plane (ignored by the assembly); beta = 0.5, sigma = 1."""
    g = Grid((n, n, 1))
    sp = uniform_species(g, ppc, seed, with_B=kind == "ecsim", beta=0.5, name="electrons")
    name = f"2d_{'cic' if order == 1 else 'tsc'}_{kind}_{n}sq_{ppc}ppc"
    return Case(name, g, order, kind, [_cast(sp, dtype)], dtype=dtype, seed=seed,
                note=f"2D {('CIC' if order == 1 else 'TSC')} {kind}, {n}x{n} cells, {ppc} ppc")
