"""Host-side checks of bench.py's bookkeeping (no GPU): every kernel the
roofline may name has a label and a source list, and the source hashes that
tie committed counter runs to kernel versions are computable."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("dtype", ["f64", "f32"])
@pytest.mark.parametrize("tensorial", [False, True])
def test_contract_kernel_named(order, dtype, tensorial):
    k = bench.contract_kernel(order, dtype, tensorial)
    assert k in bench.KERNEL_FILES and k in bench.KERNEL_LABELS


def test_every_kernel_hashable():
    for k in bench.KERNEL_FILES:
        assert k in bench.KERNEL_LABELS
        h = bench.kernel_source_hash(k)
        assert len(h) == 16 and int(h, 16) >= 0


@pytest.mark.parametrize("order", [1, 2])
def test_deposit_bytes_canonical_half(order):
    full = bench.deposit_bytes(order, True, 8, 1000, False)
    half = bench.deposit_bytes(order, True, 8, 1000, False, canonical=True)
    n = (order + 1) ** 3
    rec = 1000 * n * (n + 1) // 2 * 9 * 8
    assert (half - rec) * (2 * order + 1) ** 3 == (full - rec) * ((2 * order + 1) ** 3 + 1) // 2


@pytest.mark.parametrize("order", [1, 2])
def test_deposit_bytes_several_sets(order):
    """One deposition of k record sets reads k sets and writes M once: k - 1
    sets more than one single-set deposit, and less than k single-set deposits
    into one M (the later ones also read M)."""
    n = (order + 1) ** 3
    rec = 1000 * n * (n + 1) // 2 * 9 * 8
    one = bench.deposit_bytes(order, True, 8, 1000, False)
    for k in (2, 3, 4):
        multi = bench.deposit_bytes(order, True, 8, 1000, False, nrec=k)
        assert multi == one + (k - 1) * rec
        seq = one + (k - 1) * bench.deposit_bytes(order, True, 8, 1000, True)
        assert multi < seq


def test_workload_key_names_slab_launches():
    """The counter table keys the slab launches of the overlapped schedule apart
    from the whole-grid launches of the same workload."""
    import argparse
    args = argparse.Namespace(config=5, kind=None, dtype="f64", deposit_per_species=False, shuffled=False,
                              field="particle", canonical=False, dims=3, n2d=256, reorder=False)
    assert bench.workload_key(args) == "config5-f64"
    assert bench.workload_key(args, 4) == "config5-f64-slabs4"
    args.field = "grid"
    assert bench.workload_key(args, 4) == "config5-f64-gridB-slabs4"


def test_traffic_table_entries_name_their_launch_grid():
    """Every committed counter entry records the grid of the launches it was
    averaged over, and the slab entries have smaller grids than the
    whole-grid ones of the same workload."""
    import json
    with open(bench.PMC_FILE) as f:
        d = json.load(f)
    ents = d["kernels"]
    for key, ent in ents.items():
        assert ent["grid"] > 0, key
        if key.endswith("-slabs4"):
            whole = ents.get(key[: -len("-slabs4")])
            if whole is not None:
                assert ent["grid"] < whole["grid"], key


def test_workload_key_names_record_layout():
    """Counters taken on particle records are not read for the dense arrays."""
    import argparse
    args = argparse.Namespace(config=3, kind=None, dtype="f64", deposit_per_species=False, shuffled=True,
                              field="particle", canonical=False, dims=3, n2d=256, reorder=False, layout="records")
    assert bench.workload_key(args) == "config3-f64-shuffled-records"
    args.layout = "arrays"
    assert bench.workload_key(args) == "config3-f64-shuffled"


def test_sweep_options_name_their_workload():
    """--n and --ppc replace the grid edge and the density of a uniform config,
    and the counter table keys such runs apart from the named configs."""
    import argparse
    from workloads import make_config
    case = make_config(2, scale=4, ppc=3)
    assert case.grid.n == (4, 4, 4) and case.np_total == 4 ** 3 * 3
    args = argparse.Namespace(config=2, kind=None, dtype="f64", deposit_per_species=False, shuffled=False,
                              field="particle", canonical=False, dims=3, n2d=256, reorder=False, layout="arrays",
                              n=16, ppc=256)
    assert bench.workload_key(args) == "config2-f64-n16-ppc256"
    try:
        make_config(3, ppc=8)
    except ValueError:
        pass
    else:
        raise AssertionError("config 3 has a fixed density")


def test_positions_f32_keep_their_cells():
    """fp32 positions stay in the cell they were drawn in, and differ from
    plain rounding only where that rounding reached the cell's upper face."""
    import numpy as np
    from workloads import Grid, positions_f32
    g = Grid((4, 4, 4))
    eps = np.finfo(np.float64).eps
    pos = np.array([[0.5, 1.0 - eps, 2.25],          # y rounds up onto the face y = 1 in plain fp32
                    [3.0 - 1e-12, 0.0, 1.5],         # x rounds up onto x = 3
                    [1.25, 2.0, 3.999999999]])       # z rounds onto z = 4, the periodic end
    plain = pos.astype(np.float32)
    got = positions_f32(pos, g)
    assert got.dtype == np.float32
    assert np.array_equal(np.floor(got.astype(np.float64)), np.floor(pos))
    moved = plain != got
    assert moved.sum() == 3 and moved[0, 1] and moved[1, 0] and moved[2, 2]
    assert np.all(got[moved] == np.nextafter(plain[moved], np.float32(-np.inf)))
