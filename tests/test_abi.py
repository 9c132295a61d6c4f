"""C ABI checks that need no GPU: the library loads, exports every symbol the
public header declares, and rejects bad arguments on the host (before any HIP
call) with the documented status codes. Workspace queries (ws == NULL) also
return without touching the device."""
import ctypes
import os
import re

import pytest

from particle_grid_mass_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mm.h")


def declared_symbols():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mm_status|const char\*)\s+(mm_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_expected_entry_points():
    assert declared_symbols() == sorted(_lib.EXPORTED)


def test_library_exports_all_symbols():
    lib = _lib.load()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert lib.mm_version().decode().startswith("mm ")
    for code in range(7):
        assert lib.mm_status_string(code)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails (or sizes are returned) first


def _bin(grid, order=1, dt=_lib.MM_F64, np_=10, pos=FAKE, bs=FAKE, perm=FAKE, ws=None):
    lib = _lib.load()
    nbytes = ctypes.c_size_t(0)
    st = lib.mm_bin_particles(ctypes.byref(grid) if grid is not None else None, order, dt, np_, pos, bs, perm, ws,
                              ctypes.byref(nbytes), None)
    return st, nbytes.value


def _ecsim(grid, order=1, dt=_lib.MM_F64, np_=10, pos=FAKE, w=FAKE, B=FAKE, bs=FAKE, perm=FAKE, beta=0.5,
           sigma=1.0, algo=0, M=FAKE, ws=None, nbytes=0):
    lib = _lib.load()
    nb = ctypes.c_size_t(nbytes)
    st = lib.mm_assemble_ecsim(ctypes.byref(grid) if grid is not None else None, order, dt, np_, pos, w, B, bs, perm,
                               beta, sigma, 0, algo, M, ws, ctypes.byref(nb), None)
    return st, nb.value


def _scalar(grid, order=1, np_=10, w=FAKE, algo=0, M=FAKE):
    lib = _lib.load()
    nb = ctypes.c_size_t(0)
    return lib.mm_assemble_scalar(ctypes.byref(grid), order, _lib.MM_F64, np_, FAKE, w, FAKE, FAKE, 1.0, 0, algo, M,
                                  None, ctypes.byref(nb), None)


G8 = _lib.make_grid((8, 8, 8))


def test_workspace_queries():
    st, nb = _bin(G8, np_=100000)
    assert st == _lib.MM_OK and nb >= 3 * 100000 * 4
    st, nb0 = _bin(G8, np_=0, pos=None, perm=None)
    assert st == _lib.MM_OK and nb0 == 0
    st, _ = _ecsim(G8)
    assert st == _lib.MM_OK


def test_bin_validation():
    assert _bin(None)[0] == _lib.MM_ERR_NULL
    assert _bin(G8, order=3)[0] == _lib.MM_ERR_ARG
    assert _bin(G8, order=0)[0] == _lib.MM_ERR_ARG
    assert _bin(G8, dt=7)[0] == _lib.MM_ERR_ARG
    assert _bin(_lib.make_grid((2, 8, 8)))[0] == _lib.MM_ERR_ARG          # n < 2R+1 for CIC
    assert _bin(_lib.make_grid((4, 8, 8)), order=2)[0] == _lib.MM_ERR_ARG  # n < 2R+1 for TSC
    assert _bin(_lib.make_grid((8, 8, 8), h=(1, 0, 1)))[0] == _lib.MM_ERR_ARG
    assert _bin(_lib.make_grid((8, 8, 8), h=(1, float("inf"), 1)))[0] == _lib.MM_ERR_ARG
    assert _bin(_lib.make_grid((8, 8, 8), origin=(float("nan"), 0, 0)))[0] == _lib.MM_ERR_ARG
    assert _bin(G8, np_=-1)[0] == _lib.MM_ERR_ARG
    assert _bin(G8, np_=2 ** 31)[0] == _lib.MM_ERR_UNSUPPORTED
    assert _bin(_lib.make_grid((2048, 1024, 1024)))[0] == _lib.MM_ERR_UNSUPPORTED
    assert _bin(G8, pos=None)[0] == _lib.MM_ERR_NULL
    assert _bin(G8, perm=None)[0] == _lib.MM_ERR_NULL
    assert _bin(G8, bs=None)[0] == _lib.MM_ERR_NULL


def test_bin_workspace_too_small():
    lib = _lib.load()
    nbytes = ctypes.c_size_t(16)
    st = lib.mm_bin_particles(ctypes.byref(G8), 1, _lib.MM_F64, 1000, FAKE, FAKE, FAKE, FAKE, ctypes.byref(nbytes),
                              None)
    assert st == _lib.MM_ERR_WORKSPACE


def test_assemble_validation():
    assert _ecsim(None)[0] == _lib.MM_ERR_NULL
    assert _ecsim(G8, order=5)[0] == _lib.MM_ERR_ARG
    assert _ecsim(G8, dt=-1)[0] == _lib.MM_ERR_ARG
    assert _ecsim(G8, algo=9)[0] == _lib.MM_ERR_ARG
    assert _ecsim(G8, beta=float("nan"))[0] == _lib.MM_ERR_ARG
    assert _ecsim(G8, sigma=float("inf"))[0] == _lib.MM_ERR_ARG
    assert _ecsim(G8, np_=2 ** 31)[0] == _lib.MM_ERR_UNSUPPORTED
    assert _ecsim(G8, M=None)[0] == _lib.MM_ERR_NULL
    assert _ecsim(G8, B=None)[0] == _lib.MM_ERR_NULL
    assert _ecsim(G8, pos=None)[0] == _lib.MM_ERR_NULL
    assert _ecsim(G8, bs=None)[0] == _lib.MM_ERR_NULL           # MFMA needs the binning
    assert _ecsim(G8, bs=None, perm=None, algo=1)[0] == _lib.MM_OK  # the atomic scatter does not
    assert _ecsim(G8, np_=0, pos=None, w=None, B=None, bs=None, perm=None)[0] == _lib.MM_OK
    assert _scalar(G8, w=None) == _lib.MM_ERR_NULL
    assert _scalar(G8, order=2) == _lib.MM_OK


def test_scalar_tsc_grid_bounds():
    assert _scalar(_lib.make_grid((5, 5, 5)), order=2) == _lib.MM_OK
    assert _scalar(_lib.make_grid((4, 5, 5)), order=2) == _lib.MM_ERR_ARG


def _gridB(grid, order=1, dt=_lib.MM_F64, np_=10, Bgrid=FAKE, algo=0, bs=FAKE, perm=FAKE):
    lib = _lib.load()
    nb = ctypes.c_size_t(0)
    st = lib.mm_assemble_ecsim_gridB(ctypes.byref(grid), order, dt, np_, FAKE, FAKE, Bgrid, bs, perm, 0.5, 1.0, 0, algo,
                                     FAKE, None, ctypes.byref(nb), None)
    return st, nb.value


def test_grid_field_validation_and_workspace():
    """Workspace query of the grid-field assembly: records only where the fp64
    contraction gathers the field itself, records plus the interpolated field
    (np * 3 values) for fp32, the field alone for the atomic algorithms."""
    st, nb64 = _gridB(G8, np_=1000)
    assert st == _lib.MM_OK
    st, nb_plain = _ecsim(G8, np_=1000)
    assert nb64 == ((nb_plain + 255) & ~255)
    st, nb32 = _gridB(G8, dt=_lib.MM_F32, np_=1000)
    assert st == _lib.MM_OK and nb32 >= 1000 * 3 * 4
    st, nb_at = _gridB(G8, np_=1000, algo=1, bs=None, perm=None)
    assert st == _lib.MM_OK and nb_at == 1000 * 3 * 8
    assert _gridB(G8, Bgrid=None)[0] == _lib.MM_ERR_NULL
    assert _gridB(G8, order=3)[0] == _lib.MM_ERR_ARG
    lib = _lib.load()
    nb = ctypes.c_size_t(0)
    assert lib.mm_contract_bins_gridB(ctypes.byref(G8), 1, _lib.MM_F64, 10, FAKE, FAKE, None, FAKE, FAKE, 0.5, 1.0,
                                      None, ctypes.byref(nb), None) == _lib.MM_ERR_NULL


def test_stencil_matvec_and_canonical_validation():
    lib = _lib.load()
    mv = lambda g, order=1, dt=_lib.MM_F64, M=FAKE, x=FAKE, y=ctypes.c_void_p(0x2000): lib.mm_stencil_matvec(
        ctypes.byref(g) if g is not None else None, order, dt, 1, 0, M, x, y, None)
    assert mv(None) == _lib.MM_ERR_NULL
    assert mv(G8, order=4) == _lib.MM_ERR_ARG
    assert mv(G8, dt=3) == _lib.MM_ERR_ARG
    assert mv(G8, M=None) == _lib.MM_ERR_NULL
    assert mv(G8, y=None) == _lib.MM_ERR_NULL
    assert mv(G8, y=FAKE) == _lib.MM_ERR_ARG  # x == y
    dep = lambda g, rec=FAKE, M=FAKE: lib.mm_deposit_records_canonical(ctypes.byref(g), 2, _lib.MM_F64, 1, rec, 0, M,
                                                                       None)
    assert dep(G8, rec=None) == _lib.MM_ERR_NULL
    assert dep(G8, M=None) == _lib.MM_ERR_NULL
    assert dep(_lib.make_grid((4, 8, 8))) == _lib.MM_ERR_ARG  # n < 2R+1 for TSC


def test_probe_validation():
    """The throughput probe rejects a NULL buffer and counts out of range on the host."""
    lib = _lib.load()
    assert lib.mm_probe_mfma_f64(4, 10, None, None) == _lib.MM_ERR_NULL
    assert lib.mm_probe_mfma_f64(0, 10, FAKE, None) == _lib.MM_ERR_ARG
    assert lib.mm_probe_mfma_f64(4, 0, FAKE, None) == _lib.MM_ERR_ARG
    assert lib.mm_probe_mfma_f64((1 << 20) + 1, 10, FAKE, None) == _lib.MM_ERR_ARG


def test_deposit_records_multi_validation():
    """The several-species deposition rejects a set count outside 1..4, a NULL
    array, NULL entries and 2D grids on the host."""
    lib = _lib.load()
    P = ctypes.c_void_p

    def dep(g, nrec=2, recs="ok", M=FAKE, order=1, dt=_lib.MM_F64):
        arr = (P * 4)(FAKE, ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000))
        if recs == "null_entry":
            arr[1] = None
        a = None if recs is None else arr
        return lib.mm_deposit_records_multi(ctypes.byref(g) if g is not None else None, order, dt, 1, 0, nrec, a, 0,
                                            M, None)

    assert _lib.MM_MAX_RECORD_SETS == 4
    assert dep(None) == _lib.MM_ERR_NULL
    assert dep(G8, nrec=0) == _lib.MM_ERR_ARG
    assert dep(G8, nrec=5) == _lib.MM_ERR_ARG
    assert dep(G8, recs=None) == _lib.MM_ERR_NULL
    assert dep(G8, recs="null_entry") == _lib.MM_ERR_NULL
    assert dep(G8, M=None) == _lib.MM_ERR_NULL
    assert dep(G8, order=3) == _lib.MM_ERR_ARG
    assert dep(G8, dt=7) == _lib.MM_ERR_ARG
    assert dep(_lib.make_grid((8, 8, 1))) == _lib.MM_ERR_UNSUPPORTED


def test_record_bytes_query():
    """mm_record_bytes returns the record size the deposition reads, with the
    usual host-side argument checks, and enqueues nothing."""
    lib = _lib.load()

    def q(g, order=1, dt=_lib.MM_F64, ten=1):
        nb = ctypes.c_size_t(0)
        st = lib.mm_record_bytes(ctypes.byref(g) if g is not None else None, order, dt, ten, ctypes.byref(nb))
        return st, nb.value

    assert q(G8) == (_lib.MM_OK, 512 * 36 * 9 * 8)
    assert q(G8, ten=0) == (_lib.MM_OK, 512 * 36 * 8)
    assert q(G8, dt=_lib.MM_F32) == (_lib.MM_OK, 512 * 36 * 9 * 4)
    # second order, fp64, 3x3: run records of four bins along x (999 canonical
    # entries x 9 components, each slice plane padded to 16 values: 9360 values
    # per run) when n0 % 4 == 0 ...
    assert q(_lib.make_grid((8, 8, 8)), order=2) == (_lib.MM_OK, 512 // 4 * 9360 * 8)
    # ... and one packed triangle per bin (plus the bin order) otherwise
    st, nb2 = q(_lib.make_grid((7, 8, 8)), order=2)
    assert st == _lib.MM_OK and nb2 >= 448 * 378 * 9 * 8
    # fp32 3x3 takes the same run records in fp32 ...
    assert q(_lib.make_grid((8, 8, 8)), order=2, dt=_lib.MM_F32) == (_lib.MM_OK, 512 // 4 * 9360 * 4)
    # ... and one packed triangle per bin otherwise, as the scalar matrix always does
    assert q(_lib.make_grid((7, 8, 8)), order=2, dt=_lib.MM_F32) == (_lib.MM_OK, 448 * 378 * 9 * 4)
    assert q(_lib.make_grid((8, 8, 8)), order=2, dt=_lib.MM_F32, ten=0) == (_lib.MM_OK, 512 * 378 * 4)
    assert q(None)[0] == _lib.MM_ERR_NULL
    assert q(G8, order=3)[0] == _lib.MM_ERR_ARG
    assert q(G8, dt=9)[0] == _lib.MM_ERR_ARG
    assert lib.mm_record_bytes(ctypes.byref(G8), 1, 0, 1, None) == _lib.MM_ERR_NULL
    assert "unsupported" in lib.mm_status_string(_lib.MM_ERR_UNSUPPORTED).decode()


def test_binding_checks_bin_arrays():
    """The binding rejects binning arrays that do not fit the grid or the
    particles before any call reaches the library (host tensors suffice: the
    size check runs on shapes only)."""
    import torch
    from particle_grid_mass_amd import api
    bs = torch.zeros(513, dtype=torch.int32)
    perm = torch.zeros(100, dtype=torch.int32)
    api._check_bins(bs, perm, 512, 100)
    with pytest.raises(ValueError):
        api._check_bins(torch.zeros(512, dtype=torch.int32), perm, 512, 100)  # one short
    with pytest.raises(ValueError):
        api._check_bins(torch.zeros(1001, dtype=torch.int32), perm, 512, 100)  # another grid
    with pytest.raises(ValueError):
        api._check_bins(bs, torch.zeros(99, dtype=torch.int32), 512, 100)  # short perm


def test_noalloc_validation():
    """The allocation-free entry point checks its arguments and the size of the
    records against its fixed scratch on the host, before it looks up the
    scratch or enqueues anything."""
    lib = _lib.load()

    def call(g, order=1, dt=_lib.MM_F64, np_=10, pos=FAKE, B=FAKE, bs=FAKE, M=FAKE):
        return lib.mm_assemble_ecsim_noalloc(ctypes.byref(g) if g is not None else None, order, dt, np_, pos, FAKE,
                                             B, bs, FAKE, 0.5, 1.0, 0, M, None)

    big = _lib.make_grid((64, 64, 64))  # 262,144 nodes: CIC 3x3 fp64 records of 679 MB
    assert call(big) == _lib.MM_ERR_SCRATCH
    assert call(_lib.make_grid((32, 32, 32)), order=2) == _lib.MM_ERR_SCRATCH
    assert call(None) == _lib.MM_ERR_NULL
    assert call(G8, M=None) == _lib.MM_ERR_NULL
    assert call(G8, B=None) == _lib.MM_ERR_NULL
    assert call(G8, bs=None) == _lib.MM_ERR_NULL
    assert call(G8, order=3) == _lib.MM_ERR_ARG
    assert call(G8, dt=9) == _lib.MM_ERR_ARG
    assert call(G8, np_=-1) == _lib.MM_ERR_ARG
    assert _lib.MM_NOALLOC_SCRATCH_BYTES == 64 << 20
    assert "scratch" in lib.mm_status_string(_lib.MM_ERR_SCRATCH).decode()


def test_valu_algo_validation():
    """MM_ALGO_VALU is CIC with fp64 arithmetic, 3D and the field per particle only."""
    assert _ecsim(G8, algo=3)[0] == _lib.MM_OK  # workspace query
    assert _ecsim(G8, order=2, algo=3)[0] == _lib.MM_ERR_UNSUPPORTED
    assert _ecsim(G8, dt=_lib.MM_F32, algo=3)[0] == _lib.MM_ERR_UNSUPPORTED
    assert _ecsim(_lib.make_grid((8, 8, 1)), algo=3)[0] == _lib.MM_ERR_UNSUPPORTED
    assert _ecsim(G8, algo=4)[0] == _lib.MM_ERR_ARG


def test_slab_planes_query():
    """mm_slab_planes: the slab thickness of the overlapped assembly, 0 where
    the two phases run in turn (small planes, few slabs, first order, grids
    without run records)."""
    lib = _lib.load()

    def q(n, order=2):
        out = ctypes.c_int(-1)
        st = lib.mm_slab_planes(ctypes.byref(_lib.make_grid(n)), order, ctypes.byref(out))
        return st, out.value

    assert q((128, 128, 128)) == (_lib.MM_OK, 4)
    assert q((96, 96, 16)) == (_lib.MM_OK, 4)      # 9216 cells per plane, four slabs
    assert q((96, 96, 12)) == (_lib.MM_OK, 0)      # three slabs
    assert q((124, 64, 64)) == (_lib.MM_OK, 0)     # 7936 cells per plane
    assert q((130, 128, 64)) == (_lib.MM_OK, 0)    # n0 not a multiple of 4: per-bin records
    assert q((128, 128, 128), order=1) == (_lib.MM_OK, 0)
    assert q((128, 128, 1)) == (_lib.MM_OK, 0)     # 2D
    assert q((128, 128, 2048)) == (_lib.MM_OK, 8)  # at most 256 slabs
    assert lib.mm_slab_planes(ctypes.byref(G8), 2, None) == _lib.MM_ERR_NULL
    assert lib.mm_slab_planes(None, 2, ctypes.byref(ctypes.c_int())) == _lib.MM_ERR_NULL
    assert q((8, 8, 8), order=3)[0] == _lib.MM_ERR_ARG


def test_planes_validation():
    """The plane-range contraction and deposition check the plane range, the
    record buffer and the kind of records on the host."""
    lib = _lib.load()
    P = ctypes.c_void_p
    g = _lib.make_grid((16, 8, 8))
    need = 16 * 8 * 8 // 4 * 9360 * 8

    def cp(grid=g, order=2, dt=_lib.MM_F64, np_=10, B=FAKE, z0=0, z1=8, rec=FAKE, nbytes=need):
        return lib.mm_contract_bins_planes(ctypes.byref(grid) if grid is not None else None, order, dt, np_, FAKE,
                                           FAKE, B, FAKE, FAKE, 0.5, 1.0, z0, z1, rec, nbytes, None)

    assert cp(None) == _lib.MM_ERR_NULL
    assert cp(rec=None) == _lib.MM_ERR_NULL
    assert cp(z0=-1) == _lib.MM_ERR_ARG
    assert cp(z0=3, z1=2) == _lib.MM_ERR_ARG
    assert cp(z1=9) == _lib.MM_ERR_ARG
    assert cp(dt=5) == _lib.MM_ERR_ARG
    assert cp(np_=-1) == _lib.MM_ERR_ARG
    assert cp(order=1) == _lib.MM_ERR_UNSUPPORTED
    assert cp(B=None) == _lib.MM_ERR_UNSUPPORTED                          # scalar records are per bin
    assert cp(grid=_lib.make_grid((18, 8, 8))) == _lib.MM_ERR_UNSUPPORTED  # n0 % 4 != 0
    assert cp(grid=_lib.make_grid((16, 8, 1)), z1=1) == _lib.MM_ERR_UNSUPPORTED
    assert cp(nbytes=need - 1) == _lib.MM_ERR_WORKSPACE
    assert cp(dt=_lib.MM_F32, nbytes=need // 2 - 1) == _lib.MM_ERR_WORKSPACE
    assert cp(rec=ctypes.c_void_p(0x1008)) == _lib.MM_ERR_ARG

    def cpg(dt=_lib.MM_F64, Bg=FAKE, z1=8):
        return lib.mm_contract_bins_planes_gridB(ctypes.byref(g), 2, dt, 10, FAKE, FAKE, Bg, FAKE, FAKE, 0.5, 1.0, 0,
                                                 z1, FAKE, need, None)

    assert cpg(Bg=None) == _lib.MM_ERR_NULL
    assert cpg(dt=_lib.MM_F32) == _lib.MM_ERR_UNSUPPORTED  # fp32 interpolates the field in a pass of its own
    assert cpg(z1=9) == _lib.MM_ERR_ARG

    def dp(grid=g, order=2, nrec=1, recs="ok", z0=0, z1=8, M=FAKE):
        arr = (P * 4)(FAKE, ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000))
        if recs == "null_entry":
            arr[0] = None
        a = None if recs is None else arr
        return lib.mm_deposit_records_planes(ctypes.byref(grid) if grid is not None else None, order, _lib.MM_F64, 0,
                                             nrec, a, 0, z0, z1, M, None)

    assert dp(None) == _lib.MM_ERR_NULL
    assert dp(nrec=0) == _lib.MM_ERR_ARG
    assert dp(nrec=5) == _lib.MM_ERR_ARG
    assert dp(recs=None) == _lib.MM_ERR_NULL
    assert dp(recs="null_entry") == _lib.MM_ERR_NULL
    assert dp(M=None) == _lib.MM_ERR_NULL
    assert dp(z0=5, z1=4) == _lib.MM_ERR_ARG
    assert dp(z1=9) == _lib.MM_ERR_ARG
    assert dp(order=1) == _lib.MM_ERR_UNSUPPORTED
    assert dp(grid=_lib.make_grid((18, 8, 8))) == _lib.MM_ERR_UNSUPPORTED


def test_strided_validation():
    """The strided entry points check their strides and the combinations that
    read them on the host (size queries only: nothing is launched). Dense
    strides are the dense entry points and answer the same sizes."""
    lib = _lib.load()
    g = _lib.make_grid((8, 8, 8))
    g2 = _lib.make_grid((8, 8, 1))
    sz = ctypes.c_size_t(0)

    def bp(stride=8, np_=10, order=1, pos=FAKE, perm=FAKE, bs=FAKE):
        return lib.mm_bin_particles_strided(ctypes.byref(g), order, np_, pos, stride, bs, perm, None,
                                            ctypes.byref(sz), None)

    assert bp() == _lib.MM_OK
    assert bp(order=2) == _lib.MM_OK
    assert bp(stride=2) == _lib.MM_ERR_ARG
    assert bp(stride=1 << 31) == _lib.MM_ERR_ARG
    assert bp(np_=-1) == _lib.MM_ERR_ARG
    assert bp(pos=None) == _lib.MM_ERR_NULL
    assert bp(bs=None) == _lib.MM_ERR_NULL
    assert bp(np_=0, pos=None, perm=None) == _lib.MM_OK
    want = ctypes.c_size_t(0)
    assert lib.mm_bin_particles(ctypes.byref(g), 1, _lib.MM_F64, 10, FAKE, FAKE, FAKE, None, ctypes.byref(want),
                                None) == _lib.MM_OK
    assert bp() == _lib.MM_OK and sz.value == want.value

    def cb(grid=g, order=1, ps=8, ws_=8, bs_=8, B=FAKE, np_=10):
        return lib.mm_contract_bins_strided(ctypes.byref(grid), order, np_, FAKE, ps, FAKE, ws_, B, bs_, FAKE, FAKE,
                                            0.5, 1.0, None, ctypes.byref(sz), None)

    assert cb() == _lib.MM_OK
    rec_want = ctypes.c_size_t(0)
    assert lib.mm_record_bytes(ctypes.byref(g), 1, _lib.MM_F64, 1, ctypes.byref(rec_want)) == _lib.MM_OK
    assert sz.value == rec_want.value
    assert cb(ps=2) == _lib.MM_ERR_ARG
    assert cb(ws_=0) == _lib.MM_ERR_ARG
    assert cb(bs_=2) == _lib.MM_ERR_ARG
    assert cb(B=None) == _lib.MM_ERR_NULL
    assert cb(B=None, np_=0) == _lib.MM_ERR_NULL  # the records are tensorial
    assert cb(order=2) == _lib.MM_OK                      # the fp64 TSC contraction reads strides too
    assert cb(order=2, ps=3, ws_=1, bs_=3) == _lib.MM_OK  # dense strides: the dense entry point
    assert cb(grid=g2) == _lib.MM_ERR_UNSUPPORTED

    def ae(grid=g, order=1, algo=_lib.ALGOS["mfma"], ps=8, ws_=8, bs_=8):
        return lib.mm_assemble_ecsim_strided(ctypes.byref(grid), order, 10, FAKE, ps, FAKE, ws_, FAKE, bs_, FAKE,
                                             FAKE, 0.5, 1.0, 0, algo, FAKE, None, ctypes.byref(sz), None)

    assert ae() == _lib.MM_OK
    dense = ctypes.c_size_t(0)
    assert lib.mm_assemble_ecsim(ctypes.byref(g), 1, _lib.MM_F64, 10, FAKE, FAKE, FAKE, FAKE, FAKE, 0.5, 1.0, 0,
                                 _lib.ALGOS["mfma"], FAKE, None, ctypes.byref(dense), None) == _lib.MM_OK
    assert ae() == _lib.MM_OK and sz.value == dense.value
    assert ae(ps=2) == _lib.MM_ERR_ARG
    assert ae(ws_=-1) == _lib.MM_ERR_ARG
    for algo in ("atomic", "mfma_atomic", "valu"):
        assert ae(algo=_lib.ALGOS[algo]) == _lib.MM_ERR_UNSUPPORTED
        assert ae(algo=_lib.ALGOS[algo], ps=3, ws_=1, bs_=3) == _lib.MM_OK
    assert ae(order=2) == _lib.MM_OK
    assert ae(order=2, algo=_lib.ALGOS["atomic"]) == _lib.MM_ERR_UNSUPPORTED
    assert ae(grid=g2) == _lib.MM_ERR_UNSUPPORTED


def test_species_validation():
    """The multi-species entry points check the set on the host (size queries
    only: nothing is launched)."""
    lib = _lib.load()
    g = _lib.make_grid((8, 8, 8))
    sz = ctypes.c_size_t(0)
    F = 0x1000

    def sp(np_=10, B=F, beta=0.5, bs=F, perm=F, pos=F, strides=(0, 0, 0)):
        return _lib.MMSpecies(np_, pos, F, B, bs, perm, beta, *strides)

    def arr(*items):
        a = (_lib.MMSpecies * max(len(items), 1))()
        for i, s in enumerate(items):
            a[i] = s
        return a

    def cb(items, order=1, dt=_lib.MM_F64, ns=None, grid=g):
        a = arr(*items)
        return lib.mm_contract_bins_species(ctypes.byref(grid), order, dt, len(items) if ns is None else ns, a, 1.0,
                                            None, ctypes.byref(sz), None)

    rec_t = ctypes.c_size_t(0)
    assert lib.mm_record_bytes(ctypes.byref(g), 1, _lib.MM_F64, 1, ctypes.byref(rec_t)) == _lib.MM_OK
    assert cb([sp(), sp(beta=-0.2)]) == _lib.MM_OK and sz.value == rec_t.value
    assert cb([sp(), sp()], dt=_lib.MM_MIX) == _lib.MM_OK and sz.value == rec_t.value  # fp64 records
    rec_s = ctypes.c_size_t(0)
    assert lib.mm_record_bytes(ctypes.byref(g), 1, _lib.MM_F64, 0, ctypes.byref(rec_s)) == _lib.MM_OK
    assert cb([sp(B=None), sp(B=None)]) == _lib.MM_OK and sz.value == rec_s.value     # scalar records
    assert cb([sp()] * 8) == _lib.MM_OK
    assert cb([sp()] * 2, ns=9) == _lib.MM_ERR_ARG
    assert cb([sp()], ns=0) == _lib.MM_ERR_ARG
    assert cb([sp(), sp(B=None)]) == _lib.MM_ERR_ARG      # a tensorial and a scalar species
    assert cb([sp(np_=-1)]) == _lib.MM_ERR_ARG
    assert cb([sp(beta=float("nan"))]) == _lib.MM_ERR_ARG
    assert cb([sp(bs=None)]) == _lib.MM_ERR_NULL
    assert cb([sp(perm=None)]) == _lib.MM_ERR_NULL
    assert cb([sp(np_=0, perm=None, pos=None)]) == _lib.MM_OK
    assert cb([sp(strides=(8, 8, 8))]) == _lib.MM_OK
    assert cb([sp(strides=(2, 0, 0))]) == _lib.MM_ERR_ARG
    assert cb([sp(strides=(8, 8, 8))], dt=_lib.MM_MIX) == _lib.MM_ERR_UNSUPPORTED
    assert cb([sp()], order=2) == _lib.MM_ERR_UNSUPPORTED
    assert cb([sp()], dt=_lib.MM_F32) == _lib.MM_ERR_UNSUPPORTED
    assert cb([sp()], grid=_lib.make_grid((8, 8, 1))) == _lib.MM_ERR_UNSUPPORTED
    assert lib.mm_contract_bins_species(ctypes.byref(g), 1, _lib.MM_F64, 1, None, 1.0, None, ctypes.byref(sz),
                                        None) == _lib.MM_ERR_NULL

    def ae(items, order=1, dt=_lib.MM_F64, algo="mfma", M=F):
        a = arr(*items)
        return lib.mm_assemble_ecsim_species(ctypes.byref(g), order, dt, len(items), a, 1.0, 0, _lib.ALGOS[algo],
                                             M, None, ctypes.byref(sz), None)

    assert ae([sp(), sp()]) == _lib.MM_OK and sz.value >= rec_t.value     # one record set
    for algo in ("atomic", "mfma_atomic", "valu"):                         # species one by one
        assert ae([sp(), sp()], algo=algo) == _lib.MM_OK
    one = ctypes.c_size_t(0)
    assert lib.mm_assemble_ecsim(ctypes.byref(g), 2, _lib.MM_F64, 10, F, F, F, F, F, 0.5, 1.0, 0, _lib.ALGOS["mfma"],
                                 F, None, ctypes.byref(one), None) == _lib.MM_OK
    assert ae([sp(), sp()], order=2) == _lib.MM_OK and sz.value == one.value
    assert ae([sp(B=None)]) == _lib.MM_ERR_NULL
    assert ae([sp()], M=None) == _lib.MM_ERR_NULL
    assert ae([sp(strides=(8, 8, 8))], algo="atomic") == _lib.MM_ERR_UNSUPPORTED
    assert ae([sp(strides=(8, 8, 8))], order=2) == _lib.MM_OK  # species one by one, each strided
    assert ae([sp(strides=(8, 8, 8))], order=2, dt=_lib.MM_MIX) == _lib.MM_ERR_UNSUPPORTED
