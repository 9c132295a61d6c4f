"""MI355X (gfx950) particle-to-grid mass-matrix assembly.

The computation lives in ``libmm.so`` (hand-written HIP kernels behind the C
ABI of ``include/mm.h``); this package is its thin torch binding.
"""
from .api import (MMError, assemble_ecsim, assemble_ecsim_gridB, assemble_ecsim_noalloc, assemble_scalar,  # noqa: F401
                  assemble_ecsim_species, bin_particles,
                  contract_bins, contract_bins_species, contract_bins_planes, deposit_moments, deposit_records, deposit_records_planes,
                  noff, noff_canonical, noff_grid,
                  probe_mfma_f64, record_bytes, slab_planes, stencil_matvec)

__all__ = ["bin_particles", "assemble_scalar", "assemble_ecsim", "assemble_ecsim_gridB", "assemble_ecsim_noalloc",
           "assemble_ecsim_species", "contract_bins", "contract_bins_species", "contract_bins_planes", "deposit_records_planes",
           "deposit_records", "deposit_moments", "stencil_matvec", "probe_mfma_f64", "noff", "noff_canonical",
           "noff_grid", "record_bytes", "slab_planes", "MMError"]
