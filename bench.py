#!/usr/bin/env python3
"""Benchmark of the mass-matrix hot path on one MI355X.

Metric: particles/s assembled (ECSIM 3x3 mass matrix, fp64), with the
roofline fraction of the dominant kernel. One step is the whole hot path for
every species of the workload: binning (stable counting sort by support
group), per-bin matrix-core contraction, and stencil deposition. Inputs are
seeded synthetic particles already resident in HBM when timing starts.

Default workload: TSC ECSIM fp64 on a 128^3 periodic grid with a clustered
density (134,217,728 particles, mean 64 per cell, four Gaussian clusters),
beta = 0.5, sigma = 1: the largest of the five workloads, one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C] [--kind K]
                    [--dtype f64|f32] [--shuffled] [--algo A] [--no-cpu-baseline]

Timing: W warm-up steps; an untimed pass with events at every phase
boundary (the per-phase breakdown, and which kernel dominates); then K timed
steps between two events, with only the dominant kernel's launches bracketed
by events (its average launch duration feeds the roofline).

Prints one JSON line. ``--gpus`` above 1 is rejected: the path runs on a
single GPU; a multi-GPU decomposition is not implemented.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "particles/s assembled (ECSIM 3x3 mass matrix, fp64) + % MFMA/HBM roofline"
PEAK_FP64_MFMA = 78.6e12
PEAK_FP32_MFMA = 157.3e12
PEAK_HBM = 8.0e12
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
CSRC = os.path.join(ROOT, "particle_grid_mass_amd", "csrc")
HEADERS = ("mm_device.h", "mm_contract.h", "mm_internal.h")
# Source files that define each kernel the roofline may name.
KERNEL_FILES = {
    "k_cic64": ("k_cic64.hip",) + HEADERS,
    "k_cic32": ("k_cic32.hip",) + HEADERS,
    "k_cic64v": ("k_cic64v.hip", "k_contract.hip") + HEADERS,
    "k_cic64_reorder": ("k_cic64.hip",) + HEADERS,
    "k_tsc64": ("k_tsc64.hip", "mm_run.h") + HEADERS,
    "k_tsc32": ("k_tsc32.hip", "mm_run.h") + HEADERS,
    "k_contract": ("k_contract.hip",) + HEADERS,
    "k_gather": ("k_contract.hip",) + HEADERS,
    "k_gather_run": ("k_gather_run.hip", "mm_run.h") + HEADERS,
    "k_mass2d": ("k_mass2d.hip",) + HEADERS,
    "k_gather2d": ("k_mass2d.hip",) + HEADERS,
    "k_atomic_scatter": ("k_scatter.hip",) + HEADERS,
}


KERNEL_LABELS = {
    "k_cic64": "k_cic64 (CIC fp64 per-bin MFMA contraction, 4x4x4 f64, one bin per block)",
    "k_cic32": "k_cic32 (CIC fp32 per-bin MFMA contraction, 4x4x1 f32, one bin per block)",
    "k_cic64_reorder": "torch index_select of pos, w and B into bin order, then k_cic64 through the identity "
                       "permutation (packed-reorder comparison, timed together)",
    "k_cic64v": "k_cic64v + k_gather (CIC fp64 per-bin contraction on vector FMAs and its deposit, "
                "timed together as one MM_ALGO_VALU assembly call)",
    "k_tsc64": "k_tsc64 (TSC fp64 per-bin MFMA contraction, 4x4x4 f64, one bin per block, run records)",
    "k_tsc32": "k_tsc32 (TSC fp32 per-bin MFMA contraction, 4x4x1 f32, one bin and component per block, "
               "run records)",
    "k_contract": "k_contract (per-bin MFMA contraction)",
    "k_gather": "k_gather (stencil deposition of the per-bin records)",
    "k_gather_run": "k_gather_run (stencil deposition of the records of x-runs of four bins)",
    "k_mass2d": "k_mass2d (2D per-bin MFMA contraction, 4x4x4 f64, one bin per block)",
    "k_gather2d": "k_gather2d (2D stencil deposition of the per-bin records)",
    "k_atomic_scatter": "k_atomic_scatter (per-particle atomic scatter, comparison only)",
}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_FILES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def contract_kernel(order: int, dtype: str, tensorial: bool) -> str:
    if dtype == "f64" and order == 1:
        return "k_cic64"
    if dtype == "f32" and order == 1:
        return "k_cic32"
    if dtype == "f64" and tensorial:
        return "k_tsc64"
    return "k_contract"


def flops_per_particle(order: int, tensorial: bool, dims: int = 3) -> int:
    n = (order + 1) ** dims
    return 2 * n * n * (9 if tensorial else 1)


def contract_bytes(order: int, tensorial: bool, elem: int, np_: int, nbins: int, field_on_grid: bool = False,
                   pelem: int = 0, dims: int = 3, rec_elem: int = 0, rec_total: int = 0) -> int:
    """Algorithmic HBM bytes of one contraction launch: each particle's
    position, weight (and field) and permutation entry read once, bin bounds
    read once, one packed upper-triangle record written per bin; a field on
    the grid nodes is read once instead of the per-particle field. pelem: bytes
    of a stored position or field value when it differs from elem (the mixed
    layout's fp32 positions); rec_elem: bytes of a record value (fp64 records
    of the 2D problem); rec_total: the records' total bytes when they are not
    one packed triangle per bin (the run records of second-order fp64 3x3
    assembly, summed over runs of four bins along x)."""
    pelem = pelem or elem
    rec_elem = rec_elem or elem
    n = (order + 1) ** dims
    per_particle = (3 + (3 if tensorial and not field_on_grid else 0)) * pelem + elem + 4
    record = n * (n + 1) // 2 * (9 if tensorial else 1) * rec_elem
    field = nbins * 3 * pelem if tensorial and field_on_grid else 0
    return np_ * per_particle + (nbins + 1) * 4 + (rec_total or nbins * record) + field


def deposit_bytes(order: int, tensorial: bool, elem: int, nbins: int, accumulate: bool,
                  canonical: bool = False, dims: int = 3, rec_elem: int = 0, nrec: int = 1, rec_total: int = 0) -> int:
    """Algorithmic HBM bytes of one deposition launch: every record of the
    nrec record sets (one per species) read once, every stencil entry written
    once (read too when accumulating); the canonical half stores
    (noff + 1) / 2 offsets."""
    rec_elem = rec_elem or elem
    n = (order + 1) ** dims
    noff = (2 * order + 1) ** dims
    if canonical:
        noff = (noff + 1) // 2
    nc = 9 if tensorial else 1
    out = nbins * noff * nc * elem
    rec = rec_total or nbins * n * (n + 1) // 2 * nc * rec_elem
    return nrec * rec + out * (2 if accumulate else 1)


def workload_name(case, field_on_grid: bool = False, mix: bool = False, records: bool = False) -> str:
    n = case.grid.n
    kind = "ECSIM 3x3" if case.kind == "ecsim" else "scalar"
    order = "CIC" if case.order == 1 else "TSC"
    dt = "f64 on fp32 positions and fields" if mix else case.dtype
    return (f"{order} {kind} {dt}, {n[0]}x{n[1]}x{n[2]} periodic cells, {case.np_total:,} particles "
            f"({len(case.species)} species)" + (", magnetic field on the grid nodes" if field_on_grid else "")
            + (", one 64-byte record per particle" if records else "")
            + f", {case.name}" + ("_gridB" if field_on_grid else "") + ("_mix" if mix else "")
            + ("_records" if records else ""))


def workload_key(args, slab: int = 0) -> str:
    """Key of the workload (and launch shape) in the committed counter table:
    slab > 0 names the slab launches of the overlapped schedule."""
    return (f"config{args.config}" + (f"-{args.kind}" if args.kind else "") + f"-{args.dtype}"
            + ("-perspecies" if args.deposit_per_species else "")
            + ("-shuffled" if args.shuffled else "") + ("-gridB" if args.field == "grid" else "")
            + ("-canonical" if args.canonical else "") + (f"-2d{args.n2d}" if args.dims == 2 else "")
            + ("-reorder" if getattr(args, "reorder", False) else "")
            + ("-records" if getattr(args, "layout", "arrays") == "records" else "")
            + (f"-n{args.n}" if getattr(args, "n", 0) else "") + (f"-ppc{args.ppc}" if getattr(args, "ppc", 0) else "")
            + (f"-slabs{slab}" if slab else ""))


def pmc_traffic(kernel: str, khash: str, wkey: str):
    """Measured HBM bytes per launch of `kernel` on workload `wkey` from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs, scaled by the readings of
    a plain copy kernel; None when the counters were taken on other source."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    cal = d.get("calibration", {})
    ent = d.get("kernels", {}).get(f"{kernel}:{wkey}")
    if not ent or ent.get("source_hash") != khash or "fetch_factor" not in cal:
        return None
    return (ent["fetch_kib"] * cal["fetch_factor"] + ent["write_kib"] * cal["write_factor"]) * 1024.0


def onbox_peaks(dev, stream):
    """Peaks measured on this machine, reported beside the published ones: the
    fp64 matrix instruction the contractions issue (v_mfma_f64_4x4x4_4b, the
    library's throughput probe: 2048 workgroups x 4 waves x 16 x iters
    instructions of 512 flop) and a plain 1 GiB device-to-device copy."""
    import torch
    import particle_grid_mass_amd as mm
    nblocks, iters = 2048, 2000
    out = mm.probe_mfma_f64(nblocks, 20, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    mm.probe_mfma_f64(nblocks, iters, out=out)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    t_mfma = e0.elapsed_time(e1) * 1e-3
    mfma = nblocks * 4 * 16 * iters * 512 / t_mfma
    n = (1 << 30) // 8
    a = torch.ones(n, dtype=torch.float64, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    reps = 5
    torch.cuda.synchronize(dev)
    e0.record(stream)
    for _ in range(reps):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    t_copy = e0.elapsed_time(e1) * 1e-3 / reps
    del a, b, out
    return {"mfma_f64_4x4x4_TFLOPs": mfma / 1e12, "copy_GBps": 2 * (1 << 30) / t_copy / 1e9,
            "how": "library probe of v_mfma_f64_4x4x4_4b (2048 x 256 threads, 16 independent accumulators each); "
                   "1 GiB torch copy_, read + write bytes"}


def host_info():
    """Where the CPU baseline ran: logical CPUs of the host, CPUs this process
    may use, and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.lower().startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


def sampled_rows_parity(case, M, nof, ncomp, Fgrid=None, nsample=44, seed=55):
    """Exact oracle rows of the assembled matrix for sampled nodes: random nodes,
    the two corner nodes and, on the clustered workload, the four cluster
    centres (the densest bins). Only particles whose cell lies within three
    cells of a sampled node along every axis (periodically) can reach those
    rows, so only they are passed to the oracle. Single species, field per
    particle."""
    import numpy as np
    import torch
    import oracle
    sp = case.species[0]
    n = [int(v) for v in case.grid.n]
    nn = case.grid.ncells
    rng = np.random.default_rng(seed)
    extra = [0, nn - 1]
    if case.name.startswith("c5"):
        q = n[0] // 4
        extra += [x + n[0] * (y + n[1] * z) for (x, y, z) in
                  ((q, q, q), (3 * q, 3 * q, q), (3 * q, q, 3 * q), (q, 3 * q, 3 * q))]
    nodes = np.unique(np.concatenate([rng.integers(0, nn, nsample), extra]).astype(np.int64))
    near = np.zeros(nn, dtype=bool).reshape(n[2], n[1], n[0])
    span = np.arange(-3, 4)
    for g in nodes:
        gx, gy, gz = g % n[0], (g // n[0]) % n[1], g // (n[0] * n[1])
        near[np.ix_((gz + span) % n[2], (gy + span) % n[1], (gx + span) % n[0])] = True
    pos = np.asarray(sp.pos, dtype=np.float64)
    cell = np.zeros(pos.shape[0], dtype=np.int64)
    for d in (2, 1, 0):
        j = np.floor((pos[:, d] - case.grid.origin[d]) / case.grid.h[d]).astype(np.int64) % n[d]
        cell = cell * n[d] + j
    sel = np.flatnonzero(near.reshape(-1)[cell])
    beta, sigma = sp.beta, case.sigma
    if case.dtype == "f32":
        beta, sigma = float(np.float32(beta)), float(np.float32(sigma))
    B = None
    if case.kind == "ecsim":
        B = sp.B[sel] if Fgrid is None else oracle.interp_field(case.order, n, case.grid.origin, case.grid.h,
                                                                pos[sel], Fgrid)
    ref = oracle.rows(case.order, n, case.grid.origin, case.grid.h, pos[sel], np.asarray(sp.w, np.float64)[sel],
                      nodes, B, beta, sigma)
    got = M.view(nn, nof * ncomp)[torch.from_numpy(nodes).to(M.device)].double().cpu().numpy().reshape(ref.shape)
    err = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    emax = float(np.abs(got - ref).max() / np.abs(ref).max())
    return {"kind": "exact oracle rows of sampled nodes", "nodes": int(nodes.size), "particles_scanned": int(sel.size),
            "rel_fro": err, "max_abs_err_over_max_abs": emax}


def cpu_baseline(case, budget_s: float, Fgrid=None):
    """The oracle as it stands, on the host cores, on a bounded sample. With a
    field on the grid nodes the oracle gathers it at the particles first, and
    that gather is timed with the assembly."""
    import numpy as np
    import oracle
    sp = case.species[0]

    def field(k):
        if case.kind != "ecsim":
            return None
        if Fgrid is None:
            return sp.B[:k]
        return oracle.interp_field(case.order, case.grid.n, case.grid.origin, case.grid.h, sp.pos[:k], Fgrid)
    # whole species if it fits the budget estimate, else a cell-sorted prefix (a slab of cells)
    sample = sp.np
    t0 = time.perf_counter()
    probe = min(sp.np, 200_000)
    oracle.assemble(case.order, case.grid.n, case.grid.origin, case.grid.h, sp.pos[:probe], sp.w[:probe],
                    field(probe), sp.beta, case.sigma)
    rate_guess = probe / max(time.perf_counter() - t0, 1e-6)
    if sp.np / rate_guess > budget_s:
        sample = int(rate_guess * budget_s)
    reps, total_t, Mref = 0, 0.0, None
    while True:
        t0 = time.perf_counter()
        Mref = oracle.assemble(case.order, case.grid.n, case.grid.origin, case.grid.h, sp.pos[:sample],
                               sp.w[:sample], field(sample), sp.beta, case.sigma)
        total_t += time.perf_counter() - t0
        reps += 1
        if total_t >= budget_s or reps >= 100:
            break
    value = sample * reps / total_t
    desc = (f"species 0 of the workload, {'all' if sample == sp.np else 'first'} {sample:,} particles"
            f"{'' if sample == sp.np else ' (cell-sorted prefix: a slab of cells)'}, {reps} run(s)")
    out = {"value": value, "unit": "particles/s", "cores": oracle.max_threads(), "kind": "oracle", "sample": desc}
    out.update(host_info())
    return out, (Mref if sample == sp.np else None)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--kind", default=None, help="scalar|ecsim where the config offers both (config 4)")
    ap.add_argument("--dtype", default="f64", choices=("f64", "f32", "mix"),
                    help="f64, f32, or mix: fp32 positions and fields with fp64 weights, matrix and arithmetic")
    ap.add_argument("--shuffled", action="store_true", help="config 3: randomly shuffled particle order")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mark-every", type=int, default=1,
                    help="bracket the dominant kernel with timing events in every N-th timed step")
    ap.add_argument("--deposit-per-species", action="store_true",
                    help="several species: deposit each species' records on its own (accumulating into M) "
                         "instead of one deposition of all species' records")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work (bounded sample)")
    ap.add_argument("--algo", default="mfma",
                    help="mfma (default) | mfma_atomic | atomic | valu (the CIC contraction on vector FMAs)")
    ap.add_argument("--reorder", action="store_true",
                    help="comparison: after binning, gather pos, w and B into bin order (torch index_select) and "
                         "contract through the identity permutation; the gather is timed with the contraction")
    ap.add_argument("--canonical", action="store_true",
                    help="deposit into the canonical half of the stencil (14 / 63 offsets) instead of the full one")
    ap.add_argument("--matvec", action="store_true",
                    help="also time the stencil matrix-vector product y = M x on the assembled matrix")
    ap.add_argument("--moments", type=int, default=0,
                    help="also time the deposition of this many quantities per particle (e.g. 4: charge and "
                         "current) on the first species")
    ap.add_argument("--dims", type=int, default=3, choices=(2, 3),
                    help="2: the config's order and kind on an n x n grid with one node plane, 64 per cell")
    ap.add_argument("--n2d", type=int, default=256, help="grid edge of the 2D workload")
    ap.add_argument("--field", default="particle", choices=("particle", "grid"),
                    help="ECSIM magnetic field per particle (default) or on the grid nodes, gathered at each "
                         "particle with its support weights")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the on-box peak measurements (matrix-instruction probe and a 1 GiB copy)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the extra pass that times steps with the MALL flushed before each")
    ap.add_argument("--overlap", default="auto", choices=("auto", "off"),
                    help="auto: on grids the library assembles by slabs of planes (mm_slab_planes), contract slab "
                         "by slab and deposit each slab's completed node planes on a second stream meanwhile (the "
                         "schedule of mm_assemble_ecsim, driven here through the plane-range entry points so that "
                         "the contraction launches can be bracketed with events); off: the two phases in turn")
    ap.add_argument("--layout", default="arrays", choices=("arrays", "records"),
                    help="particle storage: arrays (pos, w and B each dense, the default) or records (one 64-byte "
                         "float64 record per particle, x y z w Bx By Bz and one unused value, read through the "
                         "strided entry points; CIC fp64 ECSIM on the matrix-core path)")
    ap.add_argument("--n", type=int, default=0,
                    help="grid edge replacing the config's (a sweep over the grid size)")
    ap.add_argument("--ppc", type=int, default=0,
                    help="particles per cell replacing those of the uniform configs 1, 2 and 4 (a sweep over the "
                         "particle density)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (untimed), the reference kernel that "
                         "scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes")
    args = ap.parse_args()
    if args.mark_every < 1:
        ap.error("--mark-every must be at least 1")

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: --gpus {args.gpus} (WORLD_SIZE={world}) requested, but this build runs on exactly one "
              f"GPU; a multi-GPU decomposition (spatial slabs with a halo sum of ghost stencil rows) is not "
              f"implemented.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import particle_grid_mass_amd as mm
    from workloads import grid_field, make_2d, make_config, positions_f32

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    mix = args.dtype == "mix"
    if args.dims == 2:  # the config's order and kind on a 2D grid (one node plane)
        order2, kind2 = {1: (1, "scalar"), 2: (1, "ecsim"), 3: (1, "ecsim"), 4: (2, args.kind or "scalar"),
                         5: (2, "ecsim")}[args.config]
        case = make_2d(args.n2d, 64, order2, kind2, dtype="f64" if mix else args.dtype, seed=2000 + args.config)
    else:
        if args.ppc and args.config not in (1, 2, 4):
            print("bench.py: --ppc applies to the uniform configs 1, 2 and 4", file=sys.stderr)
            sys.exit(2)
        case = make_config(args.config, kind=args.kind, dtype="f64" if mix else args.dtype, shuffled=args.shuffled,
                           scale=args.n or None, ppc=args.ppc or None)
    if mix:  # the stored fp32 positions and fields, seen by the oracle as the same values in fp64
        for sp in case.species:
            sp.pos = positions_f32(sp.pos, case.grid).astype(np.float64)
            if sp.B is not None:
                sp.B = sp.B.astype(np.float32).astype(np.float64)
    if args.reorder and (args.algo != "mfma" or args.dims != 3 or args.field == "grid"):
        print("bench.py: --reorder compares the matrix-core path with the field per particle (3D)", file=sys.stderr)
        sys.exit(2)
    records = args.layout == "records"
    if records and (case.order != 1 or case.kind != "ecsim" or case.dtype != "f64" or mix or args.algo != "mfma"
                    or args.dims != 3 or args.field == "grid" or args.reorder):
        print("bench.py: --layout records runs CIC fp64 ECSIM with the field per particle on the matrix-core path",
              file=sys.stderr)
        sys.exit(2)
    if args.canonical and args.algo != "mfma":
        print("bench.py: --canonical deposits the records of the matrix-core path (--algo mfma)", file=sys.stderr)
        sys.exit(2)
    on_grid = args.field == "grid"
    if on_grid and case.kind != "ecsim":
        print("bench.py: --field grid needs an ECSIM workload", file=sys.stderr)
        sys.exit(2)
    Fgrid = grid_field(case.grid, 1000 + args.config, case.dtype) if on_grid else None
    if mix and on_grid:
        Fgrid = Fgrid.astype(np.float32).astype(np.float64)
    tdt = torch.float64 if case.dtype == "f64" else torch.float32
    elem = 8 if case.dtype == "f64" else 4
    pdt = torch.float32 if mix else tdt  # stored positions and fields
    pelem = 4 if mix else elem
    tensorial = case.kind == "ecsim"
    order = case.order
    nbins = case.grid.ncells
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=tdt)

    def to_devp(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=pdt)

    spec = []
    for sp in case.species:
        spec.append(dict(pos=to_devp(sp.pos), w=to_dev(sp.w), B=to_devp(sp.B) if tensorial and not on_grid else None,
                         beta=sp.beta,
                         bs=torch.empty(nbins + 1, dtype=torch.int32, device=dev),
                         perm=torch.empty(max(sp.np, 1), dtype=torch.int32, device=dev)))
        if records:  # one record per particle; the step reads it through views
            d = spec[-1]
            R = torch.zeros((sp.np, 8), dtype=torch.float64, device=dev)
            R[:, 0:3], R[:, 3], R[:, 4:7] = d["pos"], d["w"], d["B"]
            d["pos"], d["w"], d["B"] = R[:, 0:3], R[:, 3], R[:, 4:7]
        if args.reorder:  # bin-ordered copies and the identity permutation they are read through
            d = spec[-1]
            d["pos_r"], d["w_r"] = torch.empty_like(d["pos"]), torch.empty_like(d["w"])
            d["B_r"] = torch.empty_like(d["B"]) if d["B"] is not None else None
            d["ident"] = torch.arange(max(sp.np, 1), dtype=torch.int32, device=dev)
    ncomp = 9 if tensorial else 1
    nof = mm.noff_canonical(order) if args.canonical else mm.noff_grid(order, case.grid)
    M = torch.empty(nbins * nof * ncomp, dtype=tdt, device=dev)
    Fd = to_devp(Fgrid) if on_grid else None
    # Several species on the matrix-core path: each species is contracted into
    # a record set of its own and one deposition adds all sets into M (the
    # species' matrices enter one field operator); --deposit-per-species
    # deposits each species' records on its own instead.
    multi = args.algo == "mfma" and len(spec) > 1 and args.dims == 3 and not args.deposit_per_species
    # First order in fp64 arithmetic: the species share one record set, all
    # contracted by one launch (mm_contract_bins_species) and deposited once.
    one_set = multi and order == 1 and case.dtype == "f64" and not on_grid and not args.reorder
    # Slabs of planes: the contraction of slab k on the step's stream, then the
    # node planes it completed deposited on a second stream while slab k + 1
    # contracts (a node plane reads the records of its bin plane and the two
    # before it; planes 0 and 1 wait for the last slab).
    slab = 0
    # (a field on the grid is gathered inside the fp64 contraction; fp32
    # interpolates it in a pass of its own first and keeps the phases in turn)
    if (args.overlap == "auto" and args.algo == "mfma" and args.dims == 3 and tensorial and order == 2
            and not (on_grid and case.dtype == "f32") and not multi and not args.canonical and not args.reorder):
        slab = mm.slab_planes(case.grid, order)
    overlap = slab > 0
    zb = list(range(0, case.grid.n[2], slab)) + [case.grid.n[2]] if overlap else []
    nslab = len(zb) - 1 if overlap else 1
    side = torch.cuda.Stream(dev) if overlap else None
    slab_ev = [torch.cuda.Event() for _ in range(nslab)] if overlap else []
    def species_set():
        return [(s_["pos"], s_["w"], s_["B"], s_["bs"], s_["perm"][:s_["pos"].shape[0]], s_["beta"]) for s_ in spec]

    recs = []
    if overlap:  # the record buffer only: every launch of the timed kernel is a slab launch
        recs.append(torch.empty(mm.record_bytes(case.grid, order, tdt, True), dtype=torch.uint8, device=dev))
    elif one_set:
        for s_ in spec:
            mm.bin_particles(case.grid, order, s_["pos"], s_["bs"], s_["perm"], mixed=mix)
        recs.append(mm.contract_bins_species(case.grid, order, species_set(), case.sigma))
    elif args.algo == "mfma":
        for s_ in (spec if multi else spec[:1]):
            bs_, perm_ = mm.bin_particles(case.grid, order, s_["pos"], s_["bs"], s_["perm"], mixed=mix)
            recs.append(mm.contract_bins(case.grid, order, s_["pos"], s_["w"], s_["B"], bs_, perm_, s_["beta"],
                                         case.sigma, Bgrid=Fd))

    def ecsim(s, bs, perm, si, algo):
        if on_grid:
            mm.assemble_ecsim_gridB(case.grid, order, s["pos"], s["w"], Fd, bs, perm, s["beta"], case.sigma, M=M,
                                    accumulate=si > 0, algo=algo)
        else:
            mm.assemble_ecsim(case.grid, order, s["pos"], s["w"], s["B"], bs, perm, s["beta"], case.sigma, M=M,
                              accumulate=si > 0, algo=algo)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    phases = ("bin", "contract", "deposit")

    def step(evs, marks=(0, 1, 2, 3), ovl=None):
        """One step over every species; records evs[si][k] for k in marks at the
        phase boundaries (0 before binning, 1 after binning, 2 after the
        contraction, 3 after the deposit). With the slab overlap (ovl, default
        as chosen above) mark 2 follows the last slab's contraction on the
        step's stream and mark 3 the join with the second stream."""
        ovl = overlap if ovl is None else ovl
        def mark(si, k):
            if evs is not None and k in marks:
                evs[si][k].record(stream)

        for si, s in enumerate(spec):
            mark(si, 0)
            if args.algo == "atomic":
                if tensorial:
                    ecsim(s, None, None, si, "atomic")
                else:
                    mm.assemble_scalar(case.grid, order, s["pos"], s["w"], None, None, case.sigma, M=M,
                                       accumulate=si > 0, algo="atomic")
                for k in (1, 2, 3):
                    mark(si, k)
                continue
            bs, perm = mm.bin_particles(case.grid, order, s["pos"], s["bs"], s["perm"], mixed=mix)
            mark(si, 1)
            if args.algo == "mfma" and ovl:
                rec = recs[0]
                side.wait_stream(stream)
                for k in range(nslab):
                    mm.contract_bins_planes(case.grid, order, s["pos"], s["w"], s["B"], bs, perm, s["beta"],
                                            case.sigma, zb[k], zb[k + 1], rec, Bgrid=Fd)
                    slab_ev[k].record(stream)
                    side.wait_event(slab_ev[k])
                    with torch.cuda.stream(side):
                        mm.deposit_records_planes(case.grid, order, rec, M, 2 if k == 0 else zb[k], zb[k + 1],
                                                  accumulate=si > 0)
                        if k == nslab - 1:
                            mm.deposit_records_planes(case.grid, order, rec, M, 0, 2, accumulate=si > 0)
                mark(si, 2)
                stream.wait_stream(side)
            elif one_set:  # after the last species' binning: one contraction and one deposit for all
                if si == len(spec) - 1:
                    mm.contract_bins_species(case.grid, order, species_set(), case.sigma, rec=recs[0])
                mark(si, 2)
                if si == len(spec) - 1:
                    mm.deposit_records(case.grid, order, recs[0], M, tensorial, canonical=args.canonical)
            elif args.algo == "mfma":
                rec = recs[si] if multi else recs[0]
                if args.reorder:
                    pidx = perm[:s["pos"].shape[0]]
                    torch.index_select(s["pos"], 0, pidx, out=s["pos_r"])
                    torch.index_select(s["w"], 0, pidx, out=s["w_r"])
                    if s["B"] is not None:
                        torch.index_select(s["B"], 0, pidx, out=s["B_r"])
                    mm.contract_bins(case.grid, order, s["pos_r"], s["w_r"], s["B_r"], bs, s["ident"], s["beta"],
                                     case.sigma, rec=rec)
                else:
                    mm.contract_bins(case.grid, order, s["pos"], s["w"], s["B"], bs, perm, s["beta"], case.sigma,
                                     rec=rec, Bgrid=Fd)
                mark(si, 2)
                if not multi:
                    mm.deposit_records(case.grid, order, rec, M, tensorial, accumulate=si > 0,
                                       canonical=args.canonical)
                elif si == len(spec) - 1:  # one deposition of every species' records
                    mm.deposit_records(case.grid, order, recs, M, tensorial, canonical=args.canonical)
            else:
                if tensorial:
                    ecsim(s, bs, perm, si, args.algo)
                else:
                    mm.assemble_scalar(case.grid, order, s["pos"], s["w"], bs, perm, case.sigma, M=M,
                                       accumulate=si > 0, algo=args.algo)
                mark(si, 2)
            mark(si, 3)

    for _ in range(args.warmup):
        step(None)
    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib * (1 << 20) // 8
        src = torch.ones(n, dtype=torch.float64, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()

    def new_events(nsteps):
        return [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in spec] for _ in range(nsteps)]

    # Phase pass (untimed): events at every phase boundary give the breakdown
    # and name the dominant kernel (the longest single launch of the step).
    psteps = max(1, min(args.steps, 20))
    pev = new_events(psteps)
    for k in range(psteps):
        step(pev[k])
    torch.cuda.synchronize()
    print(f"[bench] phase pass done ({psteps} steps)", file=sys.stderr, flush=True)
    phases = ("bin", "contract", "deposit")
    phase_ms = {p: 0.0 for p in phases}
    for k in range(psteps):
        for si in range(len(spec)):
            for pi, p in enumerate(phases):
                phase_ms[p] += pev[k][si][pi].elapsed_time(pev[k][si][pi + 1])
    nlaunch = {"bin": len(spec), "contract": 1 if one_set else len(spec), "deposit": 1 if multi else len(spec)}
    phase_per_launch_ms = {p: phase_ms[p] / (psteps * nlaunch[p]) for p in phases}
    if args.algo == "mfma":
        dom = max(("contract", "deposit"), key=lambda p: phase_per_launch_ms[p])
    elif args.algo in ("mfma_atomic", "valu"):
        dom = "contract"  # one assembly call: its contraction with the deposit that follows it
    else:  # one kernel per species: the per-particle atomic scatter, bracketed by marks 0 and 1
        dom = "atomic"
        phase_per_launch_ms = {"atomic_scatter": phase_per_launch_ms["bin"]}
    if args.algo in ("mfma_atomic", "valu"):  # the assembly call holds the contraction and its deposit
        phase_per_launch_ms = {"bin": phase_per_launch_ms["bin"], "assemble": phase_per_launch_ms["contract"]}
    bracket = {"contract": (1, 2), "deposit": (2, 3), "atomic": (0, 1)}[dom]

    # Timed pass: whole-step time between t_start and t_end, and the dominant
    # kernel's own launches bracketed by events on its stream (two per species
    # and step, so the timing markers add as little as possible to the step).
    # The dominant kernel is bracketed in every mark_every-th timed step (by
    # default every step). Each event pair adds a few us to its step: on
    # config 2, 127 us per step with a pair in every step and 123-125 us with
    # one in every fifth, where the sampled launches of the denser timeline
    # take 64.6 instead of 62 us.
    ev = new_events(args.steps)
    marked = [k for k in range(args.steps) if k % args.mark_every == 0]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        step(ev[k] if k % args.mark_every == 0 else None, bracket)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    # species whose launches the bracket holds (one deposition per step when
    # the species' records are deposited together)
    dom_species = ([len(spec) - 1] if (multi and dom == "deposit") or (one_set and dom == "contract")
                   else list(range(len(spec))))
    launches = len(marked) * len(dom_species)
    dom_ms = sum(ev[k][si][bracket[0]].elapsed_time(ev[k][si][bracket[1]])
                 for k in marked for si in dom_species)
    np_total = case.np_total
    value = np_total / (ms_step * 1e-3)

    # Cold pass: the same step with the 256 MB MALL (last-level cache) flushed
    # before each step by a 512 MiB device fill outside the timed interval,
    # as when other work runs between two assemblies.
    cold = None
    if not args.no_cold:
        csteps = max(1, min(args.steps, 10))
        scratch = torch.empty((512 << 20) // 8, dtype=torch.float64, device=dev)
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(csteps)]
        torch.cuda.synchronize()
        for k in range(csteps):
            scratch.fill_(float(k))
            cev[k][0].record(stream)
            step(None)
            cev[k][1].record(stream)
        torch.cuda.synchronize()
        del scratch
        cms = sum(a.elapsed_time(b) for a, b in cev) / csteps
        cold = {"ms_per_step": cms, "particles_per_s": np_total / (cms * 1e-3), "steps": csteps,
                "flush": "512 MiB device fill before each step, outside the events around the step"}
        print(f"[bench] cold pass done ({csteps} steps)", file=sys.stderr, flush=True)

    # The contraction once more without the overlap (whole-grid launches, the
    # phases in turn), untimed: the kernel's rate when it has the chip to
    # itself, beside its rate in the overlapped steps.
    solo_ms = None
    if overlap:
        ksteps = max(1, min(args.steps, 10))
        kev = new_events(ksteps)
        torch.cuda.synchronize()
        for k in range(ksteps):
            step(kev[k], (1, 2), ovl=False)
        torch.cuda.synchronize()
        solo_ms = sum(kev[k][si][1].elapsed_time(kev[k][si][2]) for k in range(ksteps)
                      for si in range(len(spec))) / (ksteps * len(spec))
        print(f"[bench] whole-grid contraction pass done ({ksteps} steps)", file=sys.stderr, flush=True)

    np_launch = np_total if one_set else np_total / len(spec)  # particles of one contraction launch
    # with the overlap the bracket holds the step's nslab slab launches
    per = nslab if overlap and dom == "contract" else 1
    launches *= per
    t_dom = dom_ms / launches * 1e-3
    flops = flops_per_particle(order, tensorial, args.dims) * np_launch / per
    # records as the library lays them out for this grid (run records, or one packed triangle per bin)
    rec_total = 0
    if args.algo == "mfma" and args.dims == 3 and order == 2 and tensorial:
        rec_total = mm.record_bytes(case.grid, order, tdt, True)
    run_records = rec_total > 0 and case.grid.n[0] % 4 == 0
    cbytes = contract_bytes(order, tensorial, elem, int(np_launch), nbins, on_grid, pelem, args.dims,
                            8 if args.dims == 2 else 0, rec_total=rec_total) / per
    # one deposition of every species' record sets, or the average over the
    # species' launches: the first overwrites M, the others accumulate into it
    # (read and write)
    if multi:
        dbytes = deposit_bytes(order, tensorial, elem, nbins, accumulate=False, canonical=args.canonical,
                               nrec=1 if one_set else len(spec), rec_total=rec_total)
    else:
        dbytes = sum(deposit_bytes(order, tensorial, elem, nbins, accumulate=si > 0, canonical=args.canonical,
                                   dims=args.dims, rec_elem=8 if args.dims == 2 else 0, rec_total=rec_total)
                     for si in range(len(spec))) / len(spec)
    if dom == "deposit":
        kname = "k_gather2d" if args.dims == 2 else ("k_gather_run" if run_records else "k_gather")
        roof = {"kernel": KERNEL_LABELS[kname], "bound": "hbm",
                "achieved": dbytes / t_dom / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
        roof["algorithmic_bytes_per_launch"] = dbytes
    else:
        kname = contract_kernel(order, case.dtype, tensorial) if dom == "contract" else "k_atomic_scatter"
        if kname == "k_contract" and run_records and case.dtype == "f32":
            kname = "k_tsc32"
        if args.dims == 2 and dom == "contract":
            kname = "k_mass2d"
        if args.algo == "mfma_atomic":
            kname = "k_contract"
        if args.algo == "valu":
            kname = "k_cic64v"
        if args.reorder and dom == "contract":
            kname = "k_cic64_reorder" if kname == "k_cic64" else kname
        peak = PEAK_FP64_MFMA if case.dtype == "f64" else PEAK_FP32_MFMA
        label = KERNEL_LABELS[kname]
        # the binding roof follows the arithmetic intensity: below the ridge
        # (peak flops / peak bytes, 9.8 flop/B for fp64) the launch is bounded
        # by HBM, above it by the matrix cores
        intensity = flops / cbytes if cbytes else float("inf")
        if intensity >= peak / PEAK_HBM:
            roof = {"kernel": label, "bound": "mfma", "achieved": flops / t_dom / 1e12, "peak": peak / 1e12,
                    "unit": "TFLOP/s"}
        else:
            roof = {"kernel": label, "bound": "hbm", "achieved": cbytes / t_dom / 1e9, "peak": PEAK_HBM / 1e9,
                    "unit": "GB/s"}
        roof["arithmetic_intensity_flop_per_B"] = intensity
        roof["algorithmic_flops_per_launch"] = flops
        roof["algorithmic_bytes_per_launch"] = cbytes
        roof["mfma_frac"] = flops / t_dom / peak
        # the same launch against the HBM roof (the CIC ECSIM contraction sits near the ridge)
        roof["hbm_achieved_GBps"] = cbytes / t_dom / 1e9
        roof["hbm_frac"] = cbytes / t_dom / PEAK_HBM
    roof["frac"] = roof["achieved"] / roof["peak"]
    khash = kernel_source_hash(kname)
    traffic = pmc_traffic(kname, khash, workload_key(args, slab if overlap else 0))
    roof["traffic"] = traffic
    roof["traffic_note"] = ("rocprofv3 FETCH_SIZE x fetch_factor + WRITE_SIZE x write_factor per launch "
                            "(profiles/pmc_traffic.json)" if traffic is not None else
                            "no counter run on this kernel source and workload")
    roof["avg_launch_ms"] = t_dom * 1e3
    roof["launches_timed"] = launches  # launches of the timed steps bracketed by events (every mark_every-th step)
    if per > 1:
        roof["launch_note"] = (f"slab launches: the contraction of {slab} bin planes each, {nslab} per step, "
                               f"with the deposition of earlier slabs running beside them on a second stream; "
                               f"per-launch figures are the step's totals / {nslab}")
    if solo_ms is not None and dom == "contract":
        t_solo = solo_ms * 1e-3
        if roof["bound"] == "mfma":
            a_solo = flops * per / t_solo / 1e12
        else:
            a_solo = cbytes * per / t_solo / 1e9
        roof["whole_grid_launch"] = {"avg_launch_ms": solo_ms, "achieved": a_solo, "frac": a_solo / roof["peak"],
                                     "launches": ksteps * len(spec),
                                     "note": "the whole-grid contraction with the chip to itself (phases in turn), "
                                             "untimed pass after the timed one"}
    roof["kernel_source_hash"] = khash
    # the same achieved rate against the peak measured on this machine
    peaks = onbox_peaks(dev, stream) if not args.no_peaks else None
    if peaks is None:
        roof["measured_peak"] = None
    elif roof["bound"] == "hbm":
        roof["measured_peak"] = peaks["copy_GBps"]
    elif case.dtype == "f64":
        roof["measured_peak"] = peaks["mfma_f64_4x4x4_TFLOPs"]
    else:
        roof["measured_peak"] = None  # the probe measures the fp64 instruction only
    roof["frac_of_measured_peak"] = (roof["achieved"] / roof["measured_peak"]) if roof["measured_peak"] else None
    roof["onbox_peaks"] = peaks

    # the assembled matrix applied to a grid vector (the field-equation product),
    # timed on its own after the assembly, from the stencil just assembled
    matvec = None
    if args.matvec:
        nv = 3 if tensorial else 1
        x = torch.randn(nbins * nv, dtype=tdt, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            mm.stencil_matvec(case.grid, order, M, x, tensorial, canonical=args.canonical, y=y)
        reps = 20
        mev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in mev:
            a.record(stream)
            mm.stencil_matvec(case.grid, order, M, x, tensorial, canonical=args.canonical, y=y)
            b.record(stream)
        torch.cuda.synchronize()
        t_mv = sum(a.elapsed_time(b) for a, b in mev) / reps * 1e-3
        mv_bytes = (M.numel() + 2 * x.numel()) * elem  # stencil and x read once, y written once
        matvec = {"kernel": "k_stencil_matvec", "stencil": "canonical half" if args.canonical else "full",
                  "avg_launch_ms": t_mv * 1e3, "algorithmic_bytes": mv_bytes,
                  "achieved_GBps": mv_bytes / t_mv / 1e9, "hbm_frac": mv_bytes / t_mv / PEAK_HBM}

    # moment deposition (charge and current, or nq quantities per particle) on
    # species 0, timed on its own with the binning of the same particles
    moments = None
    if args.moments:
        nq = args.moments
        s0 = spec[0]
        npm = s0["pos"].shape[0]
        Qm = torch.randn(npm, nq, dtype=tdt, device=dev)
        bs_m, perm_m = mm.bin_particles(case.grid, order, s0["pos"], s0["bs"], s0["perm"], mixed=mix)
        mo = mm.deposit_moments(case.grid, order, s0["pos"], Qm, bs_m, perm_m)
        for _ in range(3):
            mm.deposit_moments(case.grid, order, s0["pos"], Qm, bs_m, perm_m, m=mo)
        reps = 20
        mev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in mev:
            a.record(stream)
            mm.deposit_moments(case.grid, order, s0["pos"], Qm, bs_m, perm_m, m=mo)
            b.record(stream)
        torch.cuda.synchronize()
        t_m = sum(a.elapsed_time(b) for a, b in mev) / reps * 1e-3
        nsup = (order + 1) ** 3
        rec_b = nbins * nsup * nq * 8
        m_bytes = npm * (3 * pelem + nq * elem + 4) + (nbins + 1) * 4 + 2 * rec_b + nbins * nq * elem
        moments = {"kernels": "k_moments + k_gather_moments", "nq": nq, "avg_call_ms": t_m * 1e3,
                   "particles_per_s": npm / t_m, "algorithmic_bytes": m_bytes,
                   "achieved_GBps": m_bytes / t_m / 1e9, "hbm_frac": m_bytes / t_m / PEAK_HBM}

    # parity of this run's output against the oracle (and the CPU baseline timing)
    cpu = None
    parity = None
    parity_rows = None
    if not args.no_cpu_baseline:
        cpu, Mref = cpu_baseline(case, args.cpu_budget, Fgrid)
        if Mref is not None and len(spec) == 1:
            got = M.double().cpu().numpy().reshape(nbins, nof, ncomp)
            if args.canonical:
                import oracle
                Mref = oracle.canonical_half(order, Mref)
            parity = float(np.linalg.norm(got - Mref.reshape(got.shape)) / np.linalg.norm(Mref))
        elif len(spec) == 1 and not args.canonical and args.dims == 3:
            parity_rows = sampled_rows_parity(case, M, nof, ncomp, Fgrid)
        print("[bench] cpu baseline and parity done", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "particles/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic",
        "config": {"workload": workload_name(case, on_grid, mix, records), "config_id": args.config,
                   "grid": list(case.grid.n), "layout": args.layout, "order": order, "kind": case.kind,
                   "field": args.field if tensorial else None,
                   "storage": "fp32 positions and fields, fp64 weights and matrix" if mix else case.dtype,
                   "np": np_total,
                   "species": len(spec), "algo": args.algo + ("+reorder" if args.reorder else ""),
                   "stencil": "canonical half" if args.canonical else "full",
                   "step": ("bin per species, one contraction of every species into one record set, one deposit"
                            if one_set else
                            "bin + contract per species, one deposit of all species' records" if multi else
                            (f"bin + contract by slabs of {slab} planes, each slab's completed node planes "
                             f"deposited on a second stream during the next slab's contraction" if overlap else
                             "bin + contract + deposit per species")) if args.algo == "mfma" else
                   ("bin + assemble per species" if args.algo != "atomic" else "atomic scatter per species")},
        "phases_ms_per_launch": phase_per_launch_ms,
        "phases_from": f"untimed pass of {psteps} steps with events at every phase boundary"
                       + (": contract = the slab contractions on the step's stream (the deposits of earlier slabs "
                          "run beside them), deposit = what remains of the deposition after the last slab"
                          if overlap else ""),
        "assembly_only_particles_per_s": np_total / ((phase_ms["contract"] + phase_ms["deposit"]) / psteps * 1e-3)
        if args.algo != "atomic" else value,
        "roofline": roof,
        "stencil_matvec": matvec,
        "moments": moments,
        "cold_mall": cold,
        "cpu_baseline": cpu,
        "parity_rel_fro_vs_oracle": parity,
        "parity_sampled_rows_vs_oracle": parity_rows,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
