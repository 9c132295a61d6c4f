"""Thin torch-facing binding of the C ABI in ``include/mm.h``.

Argument marshalling only: tensors are checked for device, dtype and
layout, output and workspace buffers are allocated with torch on the
tensors' device, and the call is enqueued on the current torch stream.
Every step of the computation runs in the HIP kernels of ``libmm.so``.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import MMError

_DT = {torch.float64: _lib.MM_F64, torch.float32: _lib.MM_F32}


def _modes(pos: torch.Tensor, other: torch.Tensor):
    """(mm dtype code, field dtype, output dtype) from the position dtype and the
    dtype of the weights / quantities: equal dtypes are MM_F64 or MM_F32;
    float32 positions with float64 weights are the mixed production layout
    MM_MIX (positions and fields fp32; weights, quantities and outputs fp64)."""
    if pos.dtype not in _DT or other.dtype not in _DT:
        raise TypeError(f"unsupported dtypes {pos.dtype}, {other.dtype}")
    if pos.dtype == other.dtype:
        return _DT[pos.dtype], pos.dtype, pos.dtype
    if pos.dtype == torch.float32 and other.dtype == torch.float64:
        return _lib.MM_MIX, torch.float32, torch.float64
    raise TypeError("float64 positions with float32 weights are not a supported layout")


def _grid_of(grid) -> _lib.MMGrid:
    if isinstance(grid, _lib.MMGrid):
        return grid
    if hasattr(grid, "n"):
        return _lib.make_grid(grid.n, getattr(grid, "origin", (0, 0, 0)), getattr(grid, "h", (1, 1, 1)))
    n, origin, h = grid
    return _lib.make_grid(n, origin, h)


def _nnodes(g: _lib.MMGrid) -> int:
    return int(g.n[0]) * int(g.n[1]) * int(g.n[2])


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_tensor(t: torch.Tensor, name: str, dtype, shape_tail=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on a GPU device")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _row_strides(pos: torch.Tensor, w: Optional[torch.Tensor] = None, B: Optional[torch.Tensor] = None):
    """Element strides (pos, w, B) of particle arrays that are views into
    larger storage, such as one float64 record per particle (``part[:, 0:3]``,
    ``part[:, 3]``, ``part[:, 4:7]``), for the ``*_strided`` entry points;
    None when every given array is contiguous (the dense entry points)."""
    arrs = [t for t in (pos, w, B) if t is not None]
    for name, t in zip(("pos", "w", "B"), (pos, w, B)):
        if t is not None and not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
    if all(t.is_contiguous() for t in arrs):
        return None
    for name, t, rows in (("pos", pos, True), ("w", w, False), ("B", B, True)):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must live on a GPU device")
        if t.dtype != torch.float64:
            raise ValueError(f"{name} must be contiguous (strided particle arrays are float64)")
        if rows and (t.dim() != 2 or t.shape[1] != 3 or (t.shape[0] > 1 and t.stride(1) != 1)):
            raise ValueError(f"{name} must be contiguous or a [np, 3] view with unit stride along its rows")
        if not rows and t.dim() != 1:
            raise ValueError(f"{name} must be contiguous or a one-dimensional view")

    def rs(t, dense):
        if t is None or t.shape[0] <= 1:
            return dense
        return int(t.stride(0))
    return rs(pos, 3), rs(w, 1), rs(B, 3)


def _check_bins(bin_start: torch.Tensor, perm: torch.Tensor, nnodes: int, npart: int):
    """The binning arrays must match the grid and the particles they index:
    bin_start holds nnodes + 1 entries and perm at least one per particle
    (the kernels read bin_start[0..nnodes] and perm[bin_start[k] ..])."""
    if bin_start.numel() != nnodes + 1:
        raise ValueError(f"bin_start has {bin_start.numel()} entries, expected nnodes + 1 = {nnodes + 1}")
    if perm.numel() < npart:
        raise ValueError(f"perm has {perm.numel()} entries, fewer than the {npart} particles")


def _call(fn, what, *args):
    st = fn(*args)
    if st != _lib.MM_OK:
        raise MMError(st, what)


def _workspace(fn, what, args_before_ws, device, stream):
    """Query, allocate and return the workspace tensor and its size pointer."""
    nbytes = ctypes.c_size_t(0)
    _call(fn, what + " (workspace query)", *args_before_ws, None, ctypes.byref(nbytes), stream)
    ws = torch.empty(max(int(nbytes.value), 1), dtype=torch.uint8, device=device)
    return ws, nbytes


def noff_grid(order: int, grid) -> int:
    """Stencil offsets per node on this grid: (2R+1)^3, or (2R+1)^2 on a 2D grid (n[2] == 1)."""
    g = _grid_of(grid)
    NO = 2 * order + 1
    return NO * NO * (1 if g.n[2] == 1 else NO)


def noff(order: int) -> int:
    return (2 * order + 1) ** 3


def bin_particles(grid, order: int, pos: torch.Tensor, bin_start: Optional[torch.Tensor] = None,
                  perm: Optional[torch.Tensor] = None, mixed: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Stable counting sort by first support node -> ``(bin_start[nbins+1], perm[np])`` (int32).
    The key is found in fp64 arithmetic for float32 positions too (the
    stored value read exactly), as every assembly path places particles;
    ``mixed`` names the mixed layout (float32 positions, float64 weights)
    and bins the same way."""
    lib = _lib.load()
    g = _grid_of(grid)
    dt = pos.dtype
    if dt not in _DT:
        raise TypeError(f"unsupported dtype {dt}")
    if mixed and dt != torch.float32:
        raise TypeError("mixed binning takes float32 positions")
    strides = _row_strides(pos)
    if strides is None:
        _check_tensor(pos, "pos", dt)
    npart = pos.numel() // 3
    dev = pos.device
    if bin_start is None:
        bin_start = torch.empty(_nnodes(g) + 1, dtype=torch.int32, device=dev)
    if perm is None:
        perm = torch.empty(max(npart, 1), dtype=torch.int32, device=dev)
    _check_tensor(bin_start, "bin_start", torch.int32)
    _check_tensor(perm, "perm", torch.int32)
    _check_bins(bin_start, perm, _nnodes(g), npart)
    s = _stream(dev)
    if strides is not None:
        fn, name = lib.mm_bin_particles_strided, "mm_bin_particles_strided"
        head = (ctypes.byref(g), int(order), npart, _ptr(pos), strides[0], _ptr(bin_start), _ptr(perm))
    else:
        fn, name = lib.mm_bin_particles, "mm_bin_particles"
        head = (ctypes.byref(g), int(order), _lib.MM_MIX if mixed else _DT[dt], npart, _ptr(pos), _ptr(bin_start),
                _ptr(perm))
    ws, nbytes = _workspace(fn, name, head, dev, s)
    _call(fn, name, *head, _ptr(ws), ctypes.byref(nbytes), s)
    return bin_start, perm[:npart]


def _assemble(kind, grid, order, pos, w, B, bin_start, perm, beta, sigma, M, accumulate, algo, Bgrid=None):
    lib = _lib.load()
    g = _grid_of(grid)
    code, fdt, dt = _modes(pos, w)
    strides = _row_strides(pos, w, B) if kind == "ecsim" and Bgrid is None else None
    if strides is None:
        _check_tensor(pos, "pos", fdt)
        _check_tensor(w, "w", dt)
        if B is not None:
            _check_tensor(B, "B", fdt)
    if Bgrid is not None:
        _check_tensor(Bgrid, "Bgrid", fdt)
        if Bgrid.numel() != 3 * _nnodes(g):
            raise ValueError(f"Bgrid has {Bgrid.numel()} elements, expected 3 * nnodes = {3 * _nnodes(g)}")
    npart = pos.numel() // 3
    if w.numel() != npart or (B is not None and B.numel() != 3 * npart):
        raise ValueError("pos, w and B disagree on the particle count")
    if algo not in _lib.ALGOS:
        raise ValueError(f"unknown algo {algo!r}; expected one of {sorted(_lib.ALGOS)}")
    if _lib.ALGOS[algo] != _lib.ALGOS["atomic"]:
        if bin_start is None or perm is None:
            raise ValueError("the matrix-core algorithms need bin_start and perm from bin_particles")
        _check_tensor(bin_start, "bin_start", torch.int32)
        _check_tensor(perm, "perm", torch.int32)
        _check_bins(bin_start, perm, _nnodes(g), npart)
    ncomp = 9 if kind == "ecsim" else 1
    nof = noff_grid(order, g)
    shape = (_nnodes(g), nof, ncomp) if ncomp == 9 else (_nnodes(g), nof)
    dev = pos.device
    if M is None:
        M = torch.empty(shape, dtype=dt, device=dev)
        accumulate = False
    _check_tensor(M, "M", dt)
    if M.numel() != _nnodes(g) * nof * ncomp:
        raise ValueError(f"M has {M.numel()} elements, expected {_nnodes(g) * nof * ncomp}")
    s = _stream(dev)
    a = _lib.ALGOS[algo]
    if kind == "ecsim" and Bgrid is not None:
        fn, name = lib.mm_assemble_ecsim_gridB, "mm_assemble_ecsim_gridB"
        head = (ctypes.byref(g), int(order), code, npart, _ptr(pos), _ptr(w), _ptr(Bgrid), _ptr(bin_start),
                _ptr(perm), float(beta), float(sigma), int(bool(accumulate)), a, _ptr(M))
    elif kind == "ecsim" and strides is not None:
        fn, name = lib.mm_assemble_ecsim_strided, "mm_assemble_ecsim_strided"
        head = (ctypes.byref(g), int(order), npart, _ptr(pos), strides[0], _ptr(w), strides[1], _ptr(B), strides[2],
                _ptr(bin_start), _ptr(perm), float(beta), float(sigma), int(bool(accumulate)), a, _ptr(M))
    elif kind == "ecsim":
        fn, name = lib.mm_assemble_ecsim, "mm_assemble_ecsim"
        head = (ctypes.byref(g), int(order), code, npart, _ptr(pos), _ptr(w), _ptr(B), _ptr(bin_start), _ptr(perm),
                float(beta), float(sigma), int(bool(accumulate)), a, _ptr(M))
    else:
        fn, name = lib.mm_assemble_scalar, "mm_assemble_scalar"
        head = (ctypes.byref(g), int(order), code, npart, _ptr(pos), _ptr(w), _ptr(bin_start), _ptr(perm),
                float(sigma), int(bool(accumulate)), a, _ptr(M))
    ws, nbytes = _workspace(fn, name, head, dev, s)
    _call(fn, name, *head, _ptr(ws), ctypes.byref(nbytes), s)
    return M


def assemble_scalar(grid, order: int, pos, w, bin_start=None, perm=None, sigma: float = 1.0,
                    M: Optional[torch.Tensor] = None, accumulate: bool = False, algo: str = "mfma") -> torch.Tensor:
    """Scalar mass matrix ``[nnodes, noff]``."""
    return _assemble("scalar", grid, order, pos, w, None, bin_start, perm, 0.0, sigma, M, accumulate, algo)


def assemble_ecsim(grid, order: int, pos, w, B, bin_start=None, perm=None, beta: float = 0.0, sigma: float = 1.0,
                   M: Optional[torch.Tensor] = None, accumulate: bool = False, algo: str = "mfma") -> torch.Tensor:
    """3x3 tensorial ECSIM mass matrix ``[nnodes, noff, 9]``."""
    return _assemble("ecsim", grid, order, pos, w, B, bin_start, perm, beta, sigma, M, accumulate, algo)


def assemble_ecsim_gridB(grid, order: int, pos, w, Bgrid, bin_start=None, perm=None, beta: float = 0.0,
                         sigma: float = 1.0, M: Optional[torch.Tensor] = None, accumulate: bool = False,
                         algo: str = "mfma") -> torch.Tensor:
    """3x3 tensorial ECSIM mass matrix with the field on the grid nodes
    (``Bgrid [nnodes, 3]``), gathered at each particle with its support weights."""
    if Bgrid is None:
        raise ValueError("Bgrid is required")
    return _assemble("ecsim", grid, order, pos, w, None, bin_start, perm, beta, sigma, M, accumulate, algo,
                     Bgrid=Bgrid)


def assemble_ecsim_noalloc(grid, order: int, pos, w, B, bin_start, perm, beta: float = 0.0, sigma: float = 1.0,
                           M: Optional[torch.Tensor] = None, accumulate: bool = False) -> torch.Tensor:
    """``assemble_ecsim`` (matrix-core algorithm) through the entry point that
    allocates nothing: the per-bin records live in the library's fixed device
    scratch (``MM_NOALLOC_SCRATCH_BYTES`` per GPU), so no workspace is
    allocated; M is allocated here only when not given. Calls that overlap on
    one GPU race on that scratch."""
    lib = _lib.load()
    g = _grid_of(grid)
    code, fdt, dt = _modes(pos, w)
    _check_tensor(pos, "pos", fdt)
    _check_tensor(w, "w", dt)
    _check_tensor(B, "B", fdt)
    npart = pos.numel() // 3
    if w.numel() != npart or B.numel() != 3 * npart:
        raise ValueError("pos, w and B disagree on the particle count")
    _check_tensor(bin_start, "bin_start", torch.int32)
    _check_tensor(perm, "perm", torch.int32)
    _check_bins(bin_start, perm, _nnodes(g), npart)
    nof = noff_grid(order, g)
    if M is None:
        M = torch.empty((_nnodes(g), nof, 9), dtype=dt, device=pos.device)
        accumulate = False
    _check_tensor(M, "M", dt)
    if M.numel() != _nnodes(g) * nof * 9:
        raise ValueError(f"M has {M.numel()} elements, expected {_nnodes(g) * nof * 9}")
    _call(lib.mm_assemble_ecsim_noalloc, "mm_assemble_ecsim_noalloc", ctypes.byref(g), int(order), code, npart,
          _ptr(pos), _ptr(w), _ptr(B), _ptr(bin_start), _ptr(perm), float(beta), float(sigma),
          int(bool(accumulate)), _ptr(M), _stream(pos.device))
    return M


def contract_bins(grid, order: int, pos, w, B, bin_start, perm, beta: float = 0.0, sigma: float = 1.0,
                  rec: Optional[torch.Tensor] = None, Bgrid: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Phase 1 of the matrix-core assembly: packed per-bin local matrices (uint8
    buffer). The field is per particle (``B``) or on the grid nodes (``Bgrid``
    ``[nnodes, 3]``, gathered at each particle with its support weights)."""
    lib = _lib.load()
    g = _grid_of(grid)
    code, fdt, dt = _modes(pos, w)
    if B is not None and Bgrid is not None:
        raise ValueError("give the field per particle (B) or on the grid (Bgrid), not both")
    strides = _row_strides(pos, w, B) if B is not None else None
    if strides is None:
        _check_tensor(pos, "pos", fdt)
        _check_tensor(w, "w", dt)
        if B is not None:
            _check_tensor(B, "B", fdt)
    if Bgrid is not None:
        _check_tensor(Bgrid, "Bgrid", fdt)
        if Bgrid.numel() != 3 * _nnodes(g):
            raise ValueError(f"Bgrid has {Bgrid.numel()} elements, expected 3 * nnodes = {3 * _nnodes(g)}")
    _check_tensor(bin_start, "bin_start", torch.int32)
    _check_tensor(perm, "perm", torch.int32)
    npart = pos.numel() // 3
    if w.numel() != npart or (B is not None and B.numel() != 3 * npart):
        raise ValueError("pos, w and B disagree on the particle count")
    _check_bins(bin_start, perm, _nnodes(g), npart)
    s = _stream(pos.device)
    if Bgrid is not None:
        fn, name = lib.mm_contract_bins_gridB, "mm_contract_bins_gridB"
        field = Bgrid
    else:
        fn, name = lib.mm_contract_bins, "mm_contract_bins"
        field = B
    if field is not None and field.numel() == 0:
        # no particles: an empty tensor has no device address, but a NULL
        # field would select the scalar records; the library does not read
        # the field when np == 0, so a one-element stand-in marks the call
        # as tensorial
        field = torch.empty(1, dtype=field.dtype, device=field.device)
    if strides is not None:
        fn, name = lib.mm_contract_bins_strided, "mm_contract_bins_strided"
        head = (ctypes.byref(g), int(order), npart, _ptr(pos), strides[0], _ptr(w), strides[1], _ptr(field),
                strides[2], _ptr(bin_start), _ptr(perm), float(beta), float(sigma))
    else:
        head = (ctypes.byref(g), int(order), code, npart, _ptr(pos), _ptr(w), _ptr(field), _ptr(bin_start),
                _ptr(perm), float(beta), float(sigma))
    nbytes = ctypes.c_size_t(0)
    _call(fn, name + " (size query)", *head, None, ctypes.byref(nbytes), s)
    if rec is None:
        rec = torch.empty(max(int(nbytes.value), 1), dtype=torch.uint8, device=pos.device)
    else:
        nbytes = ctypes.c_size_t(rec.numel() * rec.element_size())
    _call(fn, name, *head, _ptr(rec), ctypes.byref(nbytes), s)
    return rec


def _species_array(g, species):
    """ctypes mm_species array for (pos, w, B, bin_start, perm, beta) tuples, one
    per species (dense or strided views as for the single-species calls).
    Returns the array, the dtype code, the output dtype, the device and the
    tensors that must outlive the call."""
    if not 1 <= len(species) <= _lib.MAX_SPECIES:
        raise ValueError(f"between 1 and {_lib.MAX_SPECIES} species, got {len(species)}")
    arr = (_lib.MMSpecies * len(species))()
    keep = []
    code0 = dt0 = dev = None
    for i, sp in enumerate(species):
        pos, w, B, bin_start, perm, beta = sp
        code, fdt, dt = _modes(pos, w)
        if code0 is None:
            code0, dt0, dev = code, dt, pos.device
        elif code != code0:
            raise TypeError("every species must use the same dtypes")
        strides = _row_strides(pos, w, B)
        if strides is None:
            _check_tensor(pos, "pos", fdt)
            _check_tensor(w, "w", dt)
            if B is not None:
                _check_tensor(B, "B", fdt)
            strides = (0, 0, 0)
        npart = pos.numel() // 3
        if w.numel() != npart or (B is not None and B.numel() != 3 * npart):
            raise ValueError(f"species {i}: pos, w and B disagree on the particle count")
        _check_tensor(bin_start, "bin_start", torch.int32)
        _check_tensor(perm, "perm", torch.int32)
        _check_bins(bin_start, perm, _nnodes(g), npart)
        if B is not None and B.numel() == 0:  # no particles: a stand-in address marks the species tensorial
            B = torch.empty(1, dtype=B.dtype, device=B.device)
            keep.append(B)
        arr[i] = _lib.MMSpecies(npart, pos.data_ptr() or None, w.data_ptr() or None,
                                None if B is None else B.data_ptr(), bin_start.data_ptr(), perm.data_ptr() or None,
                                float(beta), strides[0], strides[1], strides[2])
    return arr, code0, dt0, dev, keep


def contract_bins_species(grid, order: int, species, sigma: float = 1.0,
                          rec: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Phase 1 of every species into one record set (``mm_contract_bins_species``):
    each bin's record sums all species' particles in it. ``species`` holds
    ``(pos, w, B, bin_start, perm, beta)`` per species (B None for scalar records)."""
    lib = _lib.load()
    g = _grid_of(grid)
    arr, code, _, dev, keep = _species_array(g, species)
    s = _stream(dev)
    nbytes = ctypes.c_size_t(0)
    head = (ctypes.byref(g), int(order), code, len(species), arr, float(sigma))
    _call(lib.mm_contract_bins_species, "mm_contract_bins_species (size query)", *head, None, ctypes.byref(nbytes),
          s)
    if rec is None:
        rec = torch.empty(max(int(nbytes.value), 1), dtype=torch.uint8, device=dev)
    else:
        nbytes = ctypes.c_size_t(rec.numel() * rec.element_size())
    _call(lib.mm_contract_bins_species, "mm_contract_bins_species", *head, _ptr(rec), ctypes.byref(nbytes), s)
    del keep
    return rec


def assemble_ecsim_species(grid, order: int, species, sigma: float = 1.0, M: Optional[torch.Tensor] = None,
                           accumulate: bool = False, algo: str = "mfma") -> torch.Tensor:
    """3x3 ECSIM mass matrix of several species into one ``M`` (``mm_assemble_ecsim_species``);
    ``species`` holds ``(pos, w, B, bin_start, perm, beta)`` per species."""
    lib = _lib.load()
    g = _grid_of(grid)
    arr, code, dt, dev, keep = _species_array(g, species)
    if algo not in _lib.ALGOS:
        raise ValueError(f"unknown algo {algo!r}; expected one of {sorted(_lib.ALGOS)}")
    nof = noff_grid(order, g)
    if M is None:
        M = torch.empty((_nnodes(g), nof, 9), dtype=dt, device=dev)
        accumulate = False
    _check_tensor(M, "M", dt)
    if M.numel() != _nnodes(g) * nof * 9:
        raise ValueError(f"M has {M.numel()} elements, expected {_nnodes(g) * nof * 9}")
    s = _stream(dev)
    head = (ctypes.byref(g), int(order), code, len(species), arr, float(sigma), int(bool(accumulate)),
            _lib.ALGOS[algo], _ptr(M))
    ws, nbytes = _workspace(lib.mm_assemble_ecsim_species, "mm_assemble_ecsim_species", head, dev, s)
    _call(lib.mm_assemble_ecsim_species, "mm_assemble_ecsim_species", *head, _ptr(ws), ctypes.byref(nbytes), s)
    del keep
    return M


def slab_planes(grid, order: int) -> int:
    """Planes per slab with which the assembly overlaps contraction and
    deposition on this grid (``mm_slab_planes``); 0 when it runs them in turn."""
    lib = _lib.load()
    g = _grid_of(grid)
    out = ctypes.c_int(0)
    _call(lib.mm_slab_planes, "mm_slab_planes", ctypes.byref(g), int(order), ctypes.byref(out))
    return int(out.value)


def contract_bins_planes(grid, order: int, pos, w, B, bin_start, perm, beta: float, sigma: float, z0: int, z1: int,
                         rec: torch.Tensor, Bgrid: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Phase 1 for the bins of planes ``z0 <= z < z1`` only (run records:
    order 2): writes those runs' records into ``rec``, a buffer holding the
    records of the whole grid (``record_bytes``). The field is per particle
    (``B``) or on the grid nodes (``Bgrid`` ``[nnodes, 3]``; float64 or the
    mixed layout)."""
    lib = _lib.load()
    g = _grid_of(grid)
    code, fdt, dt = _modes(pos, w)
    _check_tensor(pos, "pos", fdt)
    _check_tensor(w, "w", dt)
    if (B is None) == (Bgrid is None):
        raise ValueError("give the field per particle (B) or on the grid (Bgrid)")
    npart = pos.numel() // 3
    if B is not None:
        _check_tensor(B, "B", fdt)
        if B.numel() != 3 * npart:
            raise ValueError("pos and B disagree on the particle count")
        field, fn, name = B, lib.mm_contract_bins_planes, "mm_contract_bins_planes"
    else:
        _check_tensor(Bgrid, "Bgrid", fdt)
        if Bgrid.numel() != 3 * _nnodes(g):
            raise ValueError(f"Bgrid has {Bgrid.numel()} elements, expected 3 * nnodes = {3 * _nnodes(g)}")
        field, fn, name = Bgrid, lib.mm_contract_bins_planes_gridB, "mm_contract_bins_planes_gridB"
    _check_tensor(bin_start, "bin_start", torch.int32)
    _check_tensor(perm, "perm", torch.int32)
    if w.numel() != npart:
        raise ValueError("pos and w disagree on the particle count")
    _check_bins(bin_start, perm, _nnodes(g), npart)
    if not isinstance(rec, torch.Tensor) or not rec.is_cuda or not rec.is_contiguous():
        raise ValueError("rec must be a contiguous device tensor")
    if field.numel() == 0:
        field = torch.empty(1, dtype=field.dtype, device=field.device)  # tensorial marker; not read when np == 0
    _call(fn, name, ctypes.byref(g), int(order), code, npart, _ptr(pos), _ptr(w), _ptr(field), _ptr(bin_start),
          _ptr(perm), float(beta), float(sigma), int(z0), int(z1), _ptr(rec), rec.numel() * rec.element_size(),
          _stream(pos.device))
    return rec


def deposit_records_planes(grid, order: int, rec, M: torch.Tensor, z0: int, z1: int, accumulate: bool = False,
                           canonical: bool = False) -> torch.Tensor:
    """Phase 2 for the nodes of planes ``z0 <= z < z1`` (run records): ``rec`` is
    one record buffer or a list of up to four, as for ``deposit_records``."""
    lib = _lib.load()
    recs = list(rec) if isinstance(rec, (list, tuple)) else [rec]
    g = _grid_of(grid)
    _check_tensor(M, "M", None)
    if M.dtype not in _DT:
        raise TypeError(f"unsupported dtype {M.dtype}")
    if not 1 <= len(recs) <= _lib.MM_MAX_RECORD_SETS:
        raise ValueError(f"1 to {_lib.MM_MAX_RECORD_SETS} record sets, got {len(recs)}")
    nof = noff_canonical(order) if canonical else noff_grid(order, g)
    if M.numel() != _nnodes(g) * nof * 9:
        raise ValueError("M has the wrong number of elements")
    for r in recs:
        _check_records(lib, g, order, M.dtype, True, r, M)
    arr = (ctypes.c_void_p * len(recs))(*[r.data_ptr() for r in recs])
    _call(lib.mm_deposit_records_planes, "mm_deposit_records_planes", ctypes.byref(g), int(order), _DT[M.dtype],
          int(bool(canonical)), len(recs), arr, int(bool(accumulate)), int(z0), int(z1), _ptr(M),
          _stream(M.device))
    return M


def record_bytes(grid, order: int, dtype: torch.dtype, tensorial: bool) -> int:
    """Bytes of the per-bin records that a deposition of this grid, order, output
    dtype and kind reads (the records mm_contract_bins writes first)."""
    lib = _lib.load()
    g = _grid_of(grid)
    if dtype not in _DT:
        raise TypeError(f"unsupported dtype {dtype}")
    nbytes = ctypes.c_size_t(0)
    _call(lib.mm_record_bytes, "mm_record_bytes", ctypes.byref(g), int(order), _DT[dtype], int(bool(tensorial)),
          ctypes.byref(nbytes))
    return int(nbytes.value)


def _check_records(lib, g, order, dtype, tensorial, rec, M):
    """A record set must be a device tensor on M's device holding at least the
    bytes the deposition reads (records of another grid, order, dtype or kind
    would be read out of bounds)."""
    if not isinstance(rec, torch.Tensor) or not rec.is_cuda or rec.device != M.device:
        raise ValueError("record sets must be device tensors on M's device")
    if not rec.is_contiguous():
        raise ValueError("record sets must be contiguous")
    need = record_bytes(g, order, dtype, tensorial)
    have = rec.numel() * rec.element_size()
    if have < need:
        raise ValueError(f"record set holds {have} bytes, the deposition reads {need} "
                         f"(records of another grid, order, dtype or kind?)")


def noff_canonical(order: int) -> int:
    """Offsets kept in the canonical half of the stencil: 14 (CIC) or 63 (TSC)."""
    return (noff(order) + 1) // 2


def deposit_records(grid, order: int, rec, M: torch.Tensor, tensorial: bool,
                    accumulate: bool = False, canonical: bool = False) -> torch.Tensor:
    """Phase 2: stencil deposition of the packed records into ``M`` (the full
    stencil, or its canonical half ``[nnodes, 14 | 63, ncomp]``). ``rec`` is
    one record buffer, or a list of up to four (one per species), summed in
    one pass over ``M`` (``mm_deposit_records_multi``)."""
    lib = _lib.load()
    if isinstance(rec, (list, tuple)):
        return _deposit_multi(lib, grid, order, list(rec), M, tensorial, accumulate, canonical)
    g = _grid_of(grid)
    _check_tensor(M, "M", None)
    if M.dtype not in _DT:
        raise TypeError(f"unsupported dtype {M.dtype}")
    ncomp = 9 if tensorial else 1
    nof = noff_canonical(order) if canonical else noff_grid(order, g)
    if M.numel() != _nnodes(g) * nof * ncomp:
        raise ValueError("M has the wrong number of elements")
    _check_records(lib, g, order, M.dtype, tensorial, rec, M)
    fn, name = ((lib.mm_deposit_records_canonical, "mm_deposit_records_canonical") if canonical
                else (lib.mm_deposit_records, "mm_deposit_records"))
    _call(fn, name, ctypes.byref(g), int(order), _DT[M.dtype], int(bool(tensorial)), _ptr(rec),
          int(bool(accumulate)), _ptr(M), _stream(M.device))
    return M


def _deposit_multi(lib, grid, order, recs, M, tensorial, accumulate, canonical):
    g = _grid_of(grid)
    _check_tensor(M, "M", None)
    if M.dtype not in _DT:
        raise TypeError(f"unsupported dtype {M.dtype}")
    if not 1 <= len(recs) <= _lib.MM_MAX_RECORD_SETS:
        raise ValueError(f"1 to {_lib.MM_MAX_RECORD_SETS} record sets, got {len(recs)}")
    ncomp = 9 if tensorial else 1
    nof = noff_canonical(order) if canonical else noff_grid(order, g)
    if M.numel() != _nnodes(g) * nof * ncomp:
        raise ValueError("M has the wrong number of elements")
    for r in recs:
        _check_records(lib, g, order, M.dtype, tensorial, r, M)
    arr = (ctypes.c_void_p * len(recs))(*[r.data_ptr() for r in recs])
    _call(lib.mm_deposit_records_multi, "mm_deposit_records_multi", ctypes.byref(g), int(order), _DT[M.dtype],
          int(bool(tensorial)), int(bool(canonical)), len(recs), arr, int(bool(accumulate)), _ptr(M),
          _stream(M.device))
    return M


def stencil_matvec(grid, order: int, M: torch.Tensor, x: torch.Tensor, tensorial: bool, canonical: bool = False,
                   y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``y[g] = sum_o M[g][o] x[g+o]`` from the full stencil or its canonical
    half; x, y are ``[nnodes, 3]`` (tensorial) or ``[nnodes]``."""
    lib = _lib.load()
    g = _grid_of(grid)
    dt = M.dtype
    if dt not in _DT:
        raise TypeError(f"unsupported dtype {dt}")
    _check_tensor(M, "M", dt)
    _check_tensor(x, "x", dt)
    nn = _nnodes(g)
    nv = 3 if tensorial else 1
    nof = noff_canonical(order) if canonical else noff(order)
    if M.numel() != nn * nof * (9 if tensorial else 1):
        raise ValueError("M has the wrong number of elements")
    if x.numel() != nn * nv:
        raise ValueError(f"x has {x.numel()} elements, expected {nn * nv}")
    if y is None:
        y = torch.empty_like(x)
    _check_tensor(y, "y", dt)
    if y.numel() != nn * nv or y.data_ptr() == x.data_ptr():
        raise ValueError("y must have x's size and not be x")
    _call(lib.mm_stencil_matvec, "mm_stencil_matvec", ctypes.byref(g), int(order), _DT[dt], int(bool(tensorial)),
          int(bool(canonical)), _ptr(M), _ptr(x), _ptr(y), _stream(M.device))
    return y


def deposit_moments(grid, order: int, pos: torch.Tensor, Q: torch.Tensor, bin_start: torch.Tensor,
                    perm: torch.Tensor, m: Optional[torch.Tensor] = None, accumulate: bool = False) -> torch.Tensor:
    """``m[g][k] = sum_p W_pg Q_p[k]`` for per-particle quantities ``Q [np, nq]``
    (nq <= 16), e.g. charge and current; returns ``m [nnodes, nq]``."""
    lib = _lib.load()
    g = _grid_of(grid)
    code, fdt, dt = _modes(pos, Q)
    _check_tensor(pos, "pos", fdt)
    _check_tensor(Q, "Q", dt)
    npart = pos.numel() // 3
    if npart == 0:
        nq = Q.shape[-1] if Q.dim() > 1 else 1
    else:
        if Q.numel() % npart:
            raise ValueError("Q must hold nq values per particle")
        nq = Q.numel() // npart
    _check_tensor(bin_start, "bin_start", torch.int32)
    _check_tensor(perm, "perm", torch.int32)
    nn = _nnodes(g)
    _check_bins(bin_start, perm, nn, npart)
    if m is None:
        m = torch.empty((nn, nq), dtype=dt, device=pos.device)
        accumulate = False
    _check_tensor(m, "m", dt)
    if m.numel() != nn * nq:
        raise ValueError(f"m has {m.numel()} elements, expected {nn * nq}")
    s = _stream(pos.device)
    head = (ctypes.byref(g), int(order), code, npart, _ptr(pos), _ptr(Q), int(nq), _ptr(bin_start), _ptr(perm),
            int(bool(accumulate)), _ptr(m))
    ws, nbytes = _workspace(lib.mm_deposit_moments, "mm_deposit_moments", head, pos.device, s)
    _call(lib.mm_deposit_moments, "mm_deposit_moments", *head, _ptr(ws), ctypes.byref(nbytes), s)
    return m


def probe_mfma_f64(nblocks: int, iters: int, out: Optional[torch.Tensor] = None,
                   device: Optional[torch.device] = None) -> torch.Tensor:
    """Measurement aid: enqueue the fp64 matrix-instruction throughput probe
    (``nblocks`` x 256 threads, ``16 * iters`` v_mfma_f64_4x4x4_4b per wave,
    512 flop each) and return its per-thread output buffer. Time it with
    events on the current stream."""
    lib = _lib.load()
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    if out is None:
        out = torch.empty(int(nblocks) * 256, dtype=torch.float64, device=dev)
    _check_tensor(out, "out", torch.float64)
    if out.numel() < int(nblocks) * 256:
        raise ValueError("out holds fewer than nblocks * 256 doubles")
    _call(lib.mm_probe_mfma_f64, "mm_probe_mfma_f64", int(nblocks), int(iters), _ptr(out), _stream(out.device))
    return out
