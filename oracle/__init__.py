"""CPU oracle for mass-matrix assembly: ctypes wrapper around ``mm_oracle.c``.

TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the GPU product path must not.

The C library is a plain fp64 direct per-particle scatter of Eq. (6) of
Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for Implicit
Particle-In-Cell Methods" (Sec. 2.1), with the B-spline weights of Sec. 2.3
and the compact stencil storage of Sec. 3.4. See the header of
``mm_oracle.c`` for every reading it takes where the page is silent.

Arrays are numpy float64 (positions ``[np, 3]``, weights ``[np]``, magnetic
field ``[np, 3]`` per particle, or ``[nnodes, 3]`` on the grid for
``interp_field``); the output layout is ``[nnodes, noff, ncomp]`` with
``ncomp`` = 1 (scalar) or 9 (3x3 tensorial, row-major).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mm_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build() -> str:
    """Compile the oracle with gcc (OpenMP, no FP contraction)."""
    tmp = LIB_PATH + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
         "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    I64 = ctypes.c_int64
    D = ctypes.c_double
    lib.oracle_alpha.argtypes = [P, D, P]
    lib.oracle_support.argtypes = [I, P, P, P, P, P, P]
    lib.oracle_assemble.argtypes = [I, P, P, P, I64, P, P, P, D, D, I, P, I]
    lib.oracle_bin.argtypes = [I, P, P, P, I64, P, P, P]
    lib.oracle_bilinear.argtypes = [I, P, P, P, I64, P, P, P, D, D, P, P, P]
    lib.oracle_rows.argtypes = [I, P, P, P, I64, P, P, P, D, D, I64, P, P]
    lib.oracle_interp_field.argtypes = [I, P, P, P, I64, P, P, P]
    lib.oracle_moments.argtypes = [I, P, P, P, I64, P, I, P, I, P]
    lib.oracle_max_threads.argtypes = []
    for f in (lib.oracle_alpha, lib.oracle_support, lib.oracle_assemble, lib.oracle_bin,
              lib.oracle_bilinear, lib.oracle_rows, lib.oracle_interp_field, lib.oracle_moments,
              lib.oracle_max_threads):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _grid_args(n, origin, h):
    return (np.ascontiguousarray(n, dtype=np.int32), np.ascontiguousarray(origin, dtype=np.float64),
            np.ascontiguousarray(h, dtype=np.float64))


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def noff_grid(order: int, n) -> int:
    """Stencil offsets per node: (2R+1)^3, or (2R+1)^2 on a 2D grid (n[2] == 1)."""
    NO = 2 * order + 1
    return NO * NO * (1 if int(n[2]) == 1 else NO)


def noff(order: int) -> int:
    return (2 * order + 1) ** 3


def max_threads() -> int:
    return _load().oracle_max_threads()


def alpha(B, beta: float) -> np.ndarray:
    """3x3 magnetic response tensor of one particle (row-major)."""
    B = _f64(B)
    out = np.empty(9)
    _check(_load().oracle_alpha(_ptr(B), float(beta), _ptr(out)), "alpha")
    return out.reshape(3, 3)


def support(order, n, origin, h, x):
    """First support node (wrapped) and per-dimension 1D weights ``[3, 3]``."""
    n_, o_, h_ = _grid_args(n, origin, h)
    x = _f64(x)
    first = np.empty(3, dtype=np.int32)
    w1d = np.empty(9)
    _check(_load().oracle_support(order, _ptr(n_), _ptr(o_), _ptr(h_), _ptr(x), _ptr(first),
                                  _ptr(w1d)), "support")
    return first, w1d.reshape(3, 3)


def assemble(order, n, origin, h, pos, w, B=None, beta=0.0, sigma=1.0, M=None, accumulate=False,
             nthreads=0) -> np.ndarray:
    """Mass matrix ``[nnodes, noff, ncomp]`` by direct scatter (scalar if ``B is None``)."""
    n_, o_, h_ = _grid_args(n, origin, h)
    pos, w, B = _f64(pos), _f64(w), _f64(B)
    npart = 0 if pos is None else pos.reshape(-1, 3).shape[0]
    ncomp = 1 if B is None else 9
    nnodes = int(np.prod(n_.astype(np.int64)))
    shape = (nnodes, noff_grid(order, n_), ncomp)
    if M is None:
        M = np.zeros(shape)
        accumulate = False
    assert M.shape == shape and M.dtype == np.float64 and M.flags.c_contiguous
    _check(_load().oracle_assemble(order, _ptr(n_), _ptr(o_), _ptr(h_), npart, _ptr(pos), _ptr(w),
                                   _ptr(B), float(beta), float(sigma), int(bool(accumulate)), _ptr(M),
                                   int(nthreads)), "assemble")
    return M


def bin_particles(order, n, origin, h, pos):
    """Stable counting sort by first support node: ``(bin_start[nbins+1], perm[np])``."""
    n_, o_, h_ = _grid_args(n, origin, h)
    pos = _f64(pos)
    npart = pos.reshape(-1, 3).shape[0]
    nbins = int(np.prod(n_.astype(np.int64)))
    bin_start = np.empty(nbins + 1, dtype=np.int32)
    perm = np.empty(max(npart, 1), dtype=np.int32)
    _check(_load().oracle_bin(order, _ptr(n_), _ptr(o_), _ptr(h_), npart, _ptr(pos), _ptr(bin_start),
                              _ptr(perm)), "bin")
    return bin_start, perm[:npart]


def bilinear(order, n, origin, h, pos, w, u, v, B=None, beta=0.0, sigma=1.0) -> float:
    """``sigma * sum_p (W_p u)^T s_p (W_p v)``; u, v are ``[nnodes, 3]`` (tensorial) or ``[nnodes]``."""
    n_, o_, h_ = _grid_args(n, origin, h)
    pos, w, B, u, v = _f64(pos), _f64(w), _f64(B), _f64(u), _f64(v)
    npart = pos.reshape(-1, 3).shape[0]
    out = np.zeros(1)
    _check(_load().oracle_bilinear(order, _ptr(n_), _ptr(o_), _ptr(h_), npart, _ptr(pos), _ptr(w),
                                   _ptr(B), float(beta), float(sigma), _ptr(u), _ptr(v), _ptr(out)), "bilinear")
    return float(out[0])


def rows(order, n, origin, h, pos, w, nodes, B=None, beta=0.0, sigma=1.0) -> np.ndarray:
    """Exact stencil rows ``[len(nodes), noff, ncomp]`` for selected nodes."""
    n_, o_, h_ = _grid_args(n, origin, h)
    pos, w, B = _f64(pos), _f64(w), _f64(B)
    nodes = np.ascontiguousarray(nodes, dtype=np.int64)
    npart = pos.reshape(-1, 3).shape[0]
    ncomp = 1 if B is None else 9
    out = np.zeros((len(nodes), noff_grid(order, n_), ncomp))
    _check(_load().oracle_rows(order, _ptr(n_), _ptr(o_), _ptr(h_), npart, _ptr(pos), _ptr(w), _ptr(B),
                               float(beta), float(sigma), len(nodes), _ptr(nodes), _ptr(out)), "rows")
    return out


def moments(order, n, origin, h, pos, Q, m=None, accumulate=False) -> np.ndarray:
    """Deposit of per-particle quantities ``Q [np, nq]``: ``m[g][k] = sum_p W_pg Q_p[k]``, ``[nnodes, nq]``."""
    n_, o_, h_ = _grid_args(n, origin, h)
    pos, Q = _f64(pos), _f64(Q)
    npart = pos.reshape(-1, 3).shape[0]
    nq = Q.reshape(npart, -1).shape[1] if npart else Q.shape[-1]
    nnodes = int(np.prod(n_.astype(np.int64)))
    if m is None:
        m = np.zeros((nnodes, nq))
        accumulate = False
    assert m.shape == (nnodes, nq) and m.dtype == np.float64 and m.flags.c_contiguous
    _check(_load().oracle_moments(order, _ptr(n_), _ptr(o_), _ptr(h_), npart, _ptr(pos), int(nq),
                                  _ptr(Q), int(bool(accumulate)), _ptr(m)), "moments")
    return m


def interp_field(order, n, origin, h, pos, F) -> np.ndarray:
    """Particle values ``[np, 3]`` of the nodal field ``F[nnodes, 3]``: sum_a W_pa F[g_a]."""
    n_, o_, h_ = _grid_args(n, origin, h)
    pos, F = _f64(pos), _f64(F)
    npart = pos.reshape(-1, 3).shape[0]
    out = np.zeros((npart, 3))
    _check(_load().oracle_interp_field(order, _ptr(n_), _ptr(o_), _ptr(h_), npart, _ptr(pos), _ptr(F),
                                       _ptr(out)), "interp_field")
    return out


# ---------------------------------------------------------------- canonical half and the stencil product
def canonical_offsets(order: int) -> np.ndarray:
    """Full offset indices of the canonical half: the displacements o with
    (dz, dy, dx) >= 0 lexicographically, i.e. full index >= the centre's.
    Sec. 3.4 stores (3^3+1)/2 = 14 (CIC) or (5^3+1)/2 = 63 (TSC) canonical
    offsets, one of each pair o, -o since M[g][o] = M[g+o][-o]; which half is
    not stated, and this one is the reading taken. Canonical index
    k = full index - centre."""
    nof = noff(order)
    return np.arange((nof - 1) // 2, nof)


def canonical_half(order: int, M: np.ndarray) -> np.ndarray:
    """``Mc[g][k] = M[g][centre + k]`` for the full stencil ``M [nnodes, noff, ncomp]``."""
    return np.ascontiguousarray(M[:, canonical_offsets(order), :])


def _offset_vectors(order: int):
    NO = 2 * order + 1
    o = np.arange(NO ** 3)
    return o % NO - order, (o // NO) % NO - order, o // (NO * NO) - order


def _neighbour(n, dx, dy, dz):
    """Node index g + (dx, dy, dz) for every node g (periodic)."""
    nx, ny, nz = (int(v) for v in n)
    g = np.arange(nx * ny * nz)
    gx, gy, gz = g % nx, (g // nx) % ny, g // (nx * ny)
    return ((gx + dx) % nx) + nx * (((gy + dy) % ny) + ny * ((gz + dz) % nz))


def full_from_canonical(order: int, n, Mc: np.ndarray) -> np.ndarray:
    """Rebuild the full stencil from the canonical half with M[g][-o] = M[g-o][o]."""
    nof = noff(order)
    c = (nof - 1) // 2
    nn = Mc.shape[0]
    M = np.empty((nn, nof, Mc.shape[2]))
    M[:, c:, :] = Mc
    ox, oy, oz = _offset_vectors(order)
    for k in range(1, nof - c):
        o = c + k
        src = _neighbour(n, -ox[o], -oy[o], -oz[o])  # g - o
        M[:, c - k, :] = Mc[src, k, :]
    return M


def stencil_matvec(order: int, n, M: np.ndarray, x: np.ndarray) -> np.ndarray:
    """The product of the assembled matrix with a grid vector, as the mass
    matrix acts on the grid electric field in the implicit field equation
    (Sec. 2.1), read off the stencil storage: y[g] = sum_o M[g][o] x[g+o],
    with M[g][o] a 3x3 block
    (row i, column j) acting on the 3-vector x[g+o] in the tensorial case and
    a scalar otherwise. x, y are ``[nnodes, 3]`` (tensorial) or ``[nnodes]``."""
    ox, oy, oz = _offset_vectors(order)
    tens = M.shape[2] == 9
    y = np.zeros_like(np.asarray(x, dtype=np.float64))
    for o in range(noff(order)):
        xo = x[_neighbour(n, ox[o], oy[o], oz[o])]
        if tens:
            y += np.einsum("gij,gj->gi", M[:, o, :].reshape(-1, 3, 3), xo)
        else:
            y += M[:, o, 0] * xo
    return y
