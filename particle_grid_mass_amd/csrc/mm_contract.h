// Launchers of the per-bin matrix-core contraction (phase 1) and the record
// gather (phase 2). Not part of the public API.
#pragma once

#include "mm_internal.h"

namespace mmk {

enum { MODE_RECORD = 0, MODE_ATOMIC = 1 };

// Phase 1: per-bin local matrices. MODE_RECORD writes packed upper-triangle
// records to `out` (record_bytes() long); MODE_ATOMIC adds into the stencil
// matrix `out` with hardware atomics.
hipError_t launch_contract(const GridDev& g, int order, bool f32, const Particles& P, const int32_t* bin_start,
                           const int32_t* perm, double beta, double sigma, int mode, void* out, hipStream_t s);

// Phase 1 for CIC fp64 records: four bins per wave, one per 4x4x4 block.
hipError_t launch_cic64(const GridDev& g, const Particles& P, const int32_t* bin_start, const int32_t* perm,
                        double beta, double sigma, double* rec, hipStream_t s);
// The same for ns (1 .. MAX_SPECIES) species in one launch: each bin's record
// sums the particles of every species (P[i] with bin_start[i], perm[i] and
// beta[i]); all species share the storage type, field placement and kind.
constexpr int MAX_SPECIES = 8;
hipError_t launch_cic64_species(const GridDev& g, int ns, const Particles* P, const int32_t* const* bin_start,
                                const int32_t* const* perm, const double* beta, double sigma, double* rec,
                                hipStream_t s);

// Phase 1 for CIC fp64 records on vector FMAs (the comparison kernel of MM_ALGO_VALU):
// 16 bins per wave, four lanes per bin splitting its 36 pairs.
hipError_t launch_cic64_valu(const GridDev& g, const Particles& P, const int32_t* bin_start, const int32_t* perm,
                             double beta, double sigma, double* rec, hipStream_t s);

// Phase 1 for CIC fp32 records: 16 bins per wave, one per block of v_mfma_f32_4x4x1_16b.
hipError_t launch_cic32(const GridDev& g, const Particles& P, const int32_t* bin_start, const int32_t* perm,
                        double beta, double sigma, float* rec, hipStream_t s);

// Phase 1 for TSC fp64 ECSIM (tensorial) records: 4x4x4 blocks, one bin per block, one wave
// per (group of four bins, row of alpha).
// Run records (tsc_run_records(g)): only the runs of bin planes z0 .. z1 - 1
// (z1 < 0: all planes); other grids take the whole grid only.
hipError_t launch_tsc64(const GridDev& g, const Particles& P, const int32_t* bin_start, const int32_t* perm,
                        double beta, double sigma, double* rec, hipStream_t s, int z0 = 0, int z1 = -1);
// Phase 1 for TSC fp32 ECSIM run records (tsc_run_records(g), field per
// particle): 4x4x1 fp32 blocks, 8 bins and two components per wave; the runs
// of bin planes z0 .. z1 - 1 (z1 < 0: all planes).
hipError_t launch_tsc32(const GridDev& g, const Particles& P, const int32_t* bin_start, const int32_t* perm,
                        double beta, double sigma, float* rec, hipStream_t s, int z0 = 0, int z1 = -1);
// Bytes k_tsc64 uses after its per-bin records (rounded up to 256) for the bin order.
size_t tsc64_order_bytes(int64_t nbins);
// Whether the order-2 tensorial records of this grid (fp64, and fp32 with the
// field per particle) are run records (mm_run.h: x-runs of four bins; 3D
// grids with n0 a multiple of 4) rather than per-bin pair records.
bool tsc_run_records(const GridDev& g);

// Whether launch_contract gathers a grid field itself (Particles::Bgrid) for
// this order, precision and mode; otherwise the field must first be
// interpolated to the particles (launch_interp_field) and passed as B.
bool contract_gathers_field(int order, bool f32, int mode);

// Throughput probe of v_mfma_f64_4x4x4_4b (k_probe.hip): nblocks x 256 threads,
// 16 * iters instructions per wave; out holds nblocks * 256 doubles.
hipError_t launch_probe_mfma_f64(int nblocks, int iters, double* out, hipStream_t s);

// Bytes of the records of this grid: packed per-bin records, nbins * N(N+1)/2 *
// ncomp * sizeof(T) (plus the TSC bin order), or the run records of order-2
// tensorial grids (tsc_run_records), in the precision of the records.
size_t record_bytes(int order, bool f32, bool tensorial, const GridDev& g);

// Phase 2: M[g][o][c] (=|+=) sum of the records of the bins that hold both g and g+o,
// over nrec (1 .. MAX_REC) record sets rec[0..nrec-1] (one per species).
// canonical: only o >= centre, stored at M[g][o - centre][c].
constexpr int MAX_REC = 4;
template <typename T>
struct RecSet {
  const T* r[MAX_REC];
  int n;
};
hipError_t launch_gather(const GridDev& g, int order, bool f32, bool tensorial, const void* const* rec, int nrec,
                         int accumulate, void* M, hipStream_t s, bool canonical = false);

// Phase 2 for run records (order 2, tensorial, tsc_run_records(g)): the same
// sums as launch_gather, read from the records of x-runs of four bins (fp32 or
// fp64 records and output).
// z0, z1: only the node rows of planes z0 .. z1 - 1 (z1 < 0: all), with their
// mirrored entries (full stencil) in planes z .. z + 2; they read the records
// of bin planes z0 - 2 .. z1 - 1 (periodic).
hipError_t launch_gather_run(const GridDev& g, const void* const* rec, int nrec, int accumulate, void* M,
                             hipStream_t s, bool canonical, bool f32, int z0 = 0, int z1 = -1);

// Run records by slabs of planes: whether this contraction takes plane ranges
// (order 2, run records, fp64 or mixed with the field per particle or on the
// grid, fp32 with the field per particle), and the contraction of bin planes
// z0 .. z1 - 1 into rec (the full record layout; only those runs' records
// are written).
bool contract_planes_apply(const GridDev& g, int order, bool f32, const Particles& P);
hipError_t launch_contract_planes(const GridDev& g, bool f32, const Particles& P, const int32_t* bin_start,
                                  const int32_t* perm, double beta, double sigma, void* rec, int z0, int z1,
                                  hipStream_t s);

// The contraction and deposition of run records overlapped (mm_overlap.hip):
// slabs of planes contracted in order on s, each slab's completed node planes
// deposited on a second stream of the device while the next slab contracts.
// overlap_slabs(g) is the number of slabs used (0: the grid is too small to
// gain; the caller runs the two phases one after the other).
int overlap_slabs(const GridDev& g);
// Planes per slab of that schedule (the last slab may be thinner), 0 when it is not used.
int overlap_slab_planes(const GridDev& g);
hipError_t launch_assemble_overlapped(const GridDev& g, bool f32, const Particles& P, const int32_t* bin_start,
                                      const int32_t* perm, double beta, double sigma, void* rec, int accumulate,
                                      void* M, hipStream_t s);

// The 2D problem (n2 == 1): per-bin fp64 records rec[bin][pair][comp] of the
// (R+1)^2 support, and their fixed-order sum into M [nnodes][(2R+1)^2][comp]
// (fp64 output).
size_t record_bytes_2d(int order, bool tensorial, int64_t nbins);
hipError_t launch_contract_2d(const GridDev& g, int order, const Particles& P, const int32_t* bin_start,
                              const int32_t* perm, double beta, double sigma, void* rec, hipStream_t s);
hipError_t launch_gather_2d(const GridDev& g, int order, bool tensorial, const void* rec, int accumulate, void* M,
                            hipStream_t s);

// Moment deposition m[g][k] = sum_p W_pg Q_p[k], k < nq <= 16, through
// per-bin fp64 records rec (moment_record_bytes) and a fixed-order gather.
size_t moment_record_bytes(int order, int nq, int64_t nbins);
hipError_t launch_moments(const GridDev& g, int order, bool f32, const void* pos, const void* Q, int nq,
                          const int32_t* bin_start, const int32_t* perm, int np, int accumulate, void* m, void* rec,
                          hipStream_t s, bool pos32 = false);

// y[g] = sum_o M[g][o] x[g+o] (3x3 blocks on 3-vectors, or scalars), from the
// full stencil or from its canonical half (M[g][-o] = M[g-o][o]).
hipError_t launch_stencil_matvec(const GridDev& g, int order, bool f32, bool tensorial, bool canonical, const void* M,
                                 const void* x, void* y, hipStream_t s);

}  // namespace mmk
