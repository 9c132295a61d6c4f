"""Helpers shared by the GPU parity tests (torch device buffers, oracle runs)."""
import numpy as np
import torch

import oracle
import particle_grid_mass_amd as mm

TOL = {"f64": 1e-12, "f32": 1e-5}
TDT = {"f64": torch.float64, "f32": torch.float32}


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / nb if nb > 0 else np.linalg.norm(a)


def max_entry_err(a, b):
    """Largest entry error relative to the largest reference entry."""
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    mb = np.abs(b).max() if b.size else 0.0
    d = np.abs(a - b).max() if a.size else 0.0
    return d / mb if mb > 0 else d


def assert_match(got, ref, dtype):
    """The parity bar: relative Frobenius error within the budget of the dtype,
    and no single entry off by more than that budget times the largest entry
    (a norm alone would let a few large errors hide among millions of
    entries)."""
    e_fro = rel_fro(got, ref)
    e_max = max_entry_err(got, ref)
    assert e_fro <= TOL[dtype], f"relative Frobenius error {e_fro:.3e} > {TOL[dtype]:.0e}"
    assert e_max <= TOL[dtype], f"max entry error {e_max:.3e} of max|ref| > {TOL[dtype]:.0e}"


def species_scalars(case, sp):
    beta, sigma = sp.beta, case.sigma
    if case.dtype == "f32":
        beta, sigma = float(np.float32(beta)), float(np.float32(sigma))
    return beta, sigma


def gpu_assemble(case, algo="mfma", species=None, return_bins=False):
    """Bin + assemble every species of ``case`` into one GPU matrix (torch)."""
    dt = TDT[case.dtype]
    M = None
    bins = []
    for si, sp in enumerate(case.species if species is None else species):
        pos = to_dev(sp.pos, dt)
        w = to_dev(sp.w, dt)
        bs = perm = None
        if algo != "atomic":
            bs, perm = mm.bin_particles(case.grid, case.order, pos)
            bins.append((bs, perm))
        if case.kind == "ecsim":
            B = to_dev(sp.B, dt)
            M = mm.assemble_ecsim(case.grid, case.order, pos, w, B, bs, perm, beta=sp.beta, sigma=case.sigma, M=M,
                                  accumulate=si > 0, algo=algo)
        else:
            M = mm.assemble_scalar(case.grid, case.order, pos, w, bs, perm, sigma=case.sigma, M=M,
                                   accumulate=si > 0, algo=algo)
    torch.cuda.synchronize()
    return (M, bins) if return_bins else M


def oracle_assemble(case, species=None):
    M = None
    for si, sp in enumerate(case.species if species is None else species):
        beta, sigma = species_scalars(case, sp)
        M = oracle.assemble(case.order, case.grid.n, case.grid.origin, case.grid.h, sp.pos, sp.w,
                            sp.B if case.kind == "ecsim" else None, beta, sigma, M=M, accumulate=si > 0)
    return M


def as_numpy_M(M, case):
    ncomp = 9 if case.kind == "ecsim" else 1
    return M.double().cpu().numpy().reshape(case.grid.ncells, mm.noff(case.order), ncomp)
