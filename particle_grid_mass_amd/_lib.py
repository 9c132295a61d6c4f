"""ctypes loader for ``libmm.so`` (the gfx950 HIP library). Fails loudly if absent."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmm.so")

MM_OK, MM_ERR_NULL, MM_ERR_ARG, MM_ERR_UNSUPPORTED, MM_ERR_WORKSPACE, MM_ERR_HIP, MM_ERR_SCRATCH = range(7)
MM_NOALLOC_SCRATCH_BYTES = 64 << 20
MM_F64, MM_F32, MM_MIX = 0, 1, 2
MM_MAX_RECORD_SETS = 4
ALGOS = {"mfma": 0, "atomic": 1, "mfma_atomic": 2, "valu": 3}

# Every symbol the public header include/mm.h declares.
EXPORTED = ("mm_bin_particles", "mm_assemble_scalar", "mm_assemble_ecsim", "mm_assemble_ecsim_gridB",
            "mm_contract_bins", "mm_contract_bins_gridB", "mm_deposit_records", "mm_deposit_records_canonical",
            "mm_deposit_records_multi", "mm_slab_planes", "mm_contract_bins_planes", "mm_contract_bins_planes_gridB",
            "mm_deposit_records_planes", "mm_bin_particles_strided", "mm_contract_bins_strided",
            "mm_assemble_ecsim_strided", "mm_contract_bins_species", "mm_assemble_ecsim_species",
            "mm_record_bytes", "mm_deposit_moments", "mm_stencil_matvec", "mm_assemble_ecsim_noalloc",
            "mm_probe_mfma_f64", "mm_status_string", "mm_version")


class MMGrid(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32 * 3), ("origin", ctypes.c_double * 3), ("h", ctypes.c_double * 3)]


MAX_SPECIES = 8


class MMSpecies(ctypes.Structure):
    """One species of the multi-species entry points (mm_species)."""
    _fields_ = [("np", ctypes.c_int64), ("pos", ctypes.c_void_p), ("w", ctypes.c_void_p), ("B", ctypes.c_void_p),
                ("bin_start", ctypes.c_void_p), ("perm", ctypes.c_void_p), ("beta", ctypes.c_double),
                ("pos_stride", ctypes.c_int64), ("w_stride", ctypes.c_int64), ("B_stride", ctypes.c_int64)]


class MMError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


_lib = None


def load():
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m particle_grid_mass_amd.build` "
                          "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    I64 = ctypes.c_int64
    D = ctypes.c_double
    SZ = ctypes.POINTER(ctypes.c_size_t)
    G = ctypes.POINTER(MMGrid)
    lib.mm_bin_particles.argtypes = [G, I, I, I64, P, P, P, P, SZ, P]
    lib.mm_assemble_scalar.argtypes = [G, I, I, I64, P, P, P, P, D, I, I, P, P, SZ, P]
    lib.mm_assemble_ecsim.argtypes = [G, I, I, I64, P, P, P, P, P, D, D, I, I, P, P, SZ, P]
    lib.mm_assemble_ecsim_gridB.argtypes = [G, I, I, I64, P, P, P, P, P, D, D, I, I, P, P, SZ, P]
    lib.mm_contract_bins.argtypes = [G, I, I, I64, P, P, P, P, P, D, D, P, SZ, P]
    lib.mm_contract_bins_gridB.argtypes = [G, I, I, I64, P, P, P, P, P, D, D, P, SZ, P]
    lib.mm_deposit_records.argtypes = [G, I, I, I, P, I, P, P]
    lib.mm_deposit_records_canonical.argtypes = [G, I, I, I, P, I, P, P]
    lib.mm_record_bytes.argtypes = [G, I, I, I, SZ]
    lib.mm_deposit_records_multi.argtypes = [G, I, I, I, I, I, ctypes.POINTER(P), I, P, P]
    lib.mm_stencil_matvec.argtypes = [G, I, I, I, I, P, P, P, P]
    lib.mm_deposit_moments.argtypes = [G, I, I, I64, P, P, I, P, P, I, P, P, SZ, P]
    lib.mm_probe_mfma_f64.argtypes = [I, I, P, P]
    lib.mm_assemble_ecsim_noalloc.argtypes = [G, I, I, I64, P, P, P, P, P, D, D, I, P, P]
    lib.mm_slab_planes.argtypes = [G, I, ctypes.POINTER(ctypes.c_int)]
    lib.mm_contract_bins_planes.argtypes = [G, I, I, I64, P, P, P, P, P, D, D, I, I, P, ctypes.c_size_t, P]
    lib.mm_contract_bins_planes_gridB.argtypes = [G, I, I, I64, P, P, P, P, P, D, D, I, I, P, ctypes.c_size_t, P]
    lib.mm_deposit_records_planes.argtypes = [G, I, I, I, I, ctypes.POINTER(P), I, I, I, P, P]
    lib.mm_bin_particles_strided.argtypes = [G, I, I64, P, I64, P, P, P, SZ, P]
    lib.mm_contract_bins_strided.argtypes = [G, I, I64, P, I64, P, I64, P, I64, P, P, D, D, P, SZ, P]
    lib.mm_assemble_ecsim_strided.argtypes = [G, I, I64, P, I64, P, I64, P, I64, P, P, D, D, I, I, P, P, SZ, P]
    SP = ctypes.POINTER(MMSpecies)
    lib.mm_contract_bins_species.argtypes = [G, I, I, I, SP, D, P, SZ, P]
    lib.mm_assemble_ecsim_species.argtypes = [G, I, I, I, SP, D, I, I, P, P, SZ, P]
    for f in (lib.mm_bin_particles, lib.mm_assemble_scalar, lib.mm_assemble_ecsim, lib.mm_assemble_ecsim_gridB,
              lib.mm_contract_bins, lib.mm_contract_bins_gridB, lib.mm_deposit_records,
              lib.mm_deposit_records_canonical, lib.mm_deposit_records_multi, lib.mm_record_bytes,
              lib.mm_stencil_matvec, lib.mm_deposit_moments,
              lib.mm_probe_mfma_f64, lib.mm_assemble_ecsim_noalloc, lib.mm_slab_planes, lib.mm_contract_bins_planes,
              lib.mm_contract_bins_planes_gridB, lib.mm_deposit_records_planes, lib.mm_bin_particles_strided,
              lib.mm_contract_bins_strided, lib.mm_assemble_ecsim_strided, lib.mm_contract_bins_species,
              lib.mm_assemble_ecsim_species):
        f.restype = ctypes.c_int
    lib.mm_status_string.argtypes = [ctypes.c_int]
    lib.mm_status_string.restype = ctypes.c_char_p
    lib.mm_version.argtypes = []
    lib.mm_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load().mm_status_string(int(status)).decode()
    except ImportError:
        return "library not loaded"


def make_grid(n, origin=(0.0, 0.0, 0.0), h=(1.0, 1.0, 1.0)) -> MMGrid:
    g = MMGrid()
    for d in range(3):
        g.n[d] = int(n[d])
        g.origin[d] = float(origin[d])
        g.h[d] = float(h[d])
    return g
