/*
 * mm.h - C ABI of the MI355X (gfx950) particle-to-grid mass-matrix library.
 *
 * The operation is the implicit-PIC mass matrix of Pennati & Markidis,
 * "Mass Matrix Assembly on Tensor Cores for Implicit Particle-In-Cell
 * Methods", Sec. 2.1 Eq. (6):
 *
 *     M^{ij}_{g g'} = sigma * sum_p s_p^{ij} W_pg W_pg'
 *
 * with tensor-product B-spline weights W_pg (Sec. 2.3 Eq. 12) of order 1
 * (CIC, 8 support nodes) or 2 (TSC, 27 support nodes), assembled cell by
 * cell as batched small matrix products (Sec. 3.1-3.2, Eq. 15) on the matrix
 * cores, and stored in the compact stencil format of Sec. 3.4.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Grid:    periodic, n[d] cells per axis and as many nodes; node k sits at
 *           origin[d] + k*h[d]. Node index g = x + n0*(y + n1*z).
 *  Support: per axis u = (x - origin)/h (IEEE division), j = floor(u),
 *           xi = u - j. CIC: nodes j, j+1 with weights (1-xi, xi). TSC: the
 *           stencil is centred on the nearest node m (m = j if xi < 1/2, else
 *           j+1, the tie going up as in Sec. 2.3), nodes m-1, m, m+1 with the
 *           quadratic B-spline weights. Node ids wrap modulo n.
 *  Output:  M[node][offset][comp], node-major. offset = (dx+R) + (2R+1)*((dy+R)
 *           + (2R+1)*(dz+R)) for the node-pair displacement d = g' - g in
 *           [-R,R]^3 (27 offsets for CIC, 125 for TSC). comp = 3*i + j
 *           (tensorial, 9 per entry, row i of alpha) or a single scalar.
 *           The full stencil is stored (both g->g' and g'->g).
 *  2D:      a grid with n[2] == 1 is the 2D problem (Sec. 5 reports 2D runs):
 *           z is ignored, the support is the (R+1)^2 nodes of the plane and
 *           the stencil has (2R+1)^2 offsets, offset = (dx+R) + (2R+1)(dy+R).
 *           It runs on the matrix-core path (MM_ALGO_MFMA) in MM_F64 or
 *           MM_MIX, through mm_bin_particles, mm_assemble_scalar,
 *           mm_assemble_ecsim, mm_contract_bins and mm_deposit_records (the
 *           records are fp64); every other combination is
 *           MM_ERR_UNSUPPORTED.
 *  dtype:   MM_F64: pos, w, B and M are double. MM_F32: all four are float;
 *           the cell decision (floor of u, the TSC half-cell test, the bin
 *           key) is taken in fp64 on the stored fp32 position, which fp64
 *           holds exactly, so a particle is placed as its exact value is;
 *           the weights, the response tensor and the matrix-core
 *           accumulation run in fp32 (sigma and beta are rounded to fp32).
 *           MM_MIX: the
 *           production layout of Sec. 5 ("Exactness and precision"):
 *           positions and fields (pos, B, Bgrid) are float, weights w,
 *           quantities Q, vectors x, y and the outputs M, m are double, and
 *           every step runs in fp64 on the fp32 values read exactly into fp64
 *           (the cell decision too). MM_ALGO_ATOMIC does not take MM_MIX
 *           (MM_ERR_UNSUPPORTED).
 *  Memory:  every array argument is a device pointer (hipMalloc or an
 *           allocator on top of it, e.g. torch) on the current device,
 *           owned by the caller. The library allocates no device memory and
 *           keeps no mutable global state; calls are reentrant. The
 *           exceptions: mm_assemble_ecsim_noalloc uses a fixed scratch array
 *           of the library per GPU (see there), and the overlapped assembly
 *           (mm_slab_planes) creates a second stream and its events per GPU on
 *           the first such call and keeps them.
 *  Streams: all work is enqueued asynchronously on `stream` (a hipStream_t,
 *           NULL = default stream); no call synchronizes the host. The
 *           overlapped assembly also enqueues on the GPU's second stream,
 *           fenced by events: it starts after the work already on `stream`,
 *           and `stream` waits for it before anything enqueued later.
 *  Workspace (CUB style): call with ws == NULL to receive the required byte
 *           count in *ws_bytes (nothing is enqueued, MM_OK is returned); then
 *           call again with a device buffer of at least that many bytes,
 *           aligned to 16 bytes (else MM_ERR_ARG).
 *  Errors:  arguments are validated on the host before any HIP call;
 *           a failed launch returns MM_ERR_HIP. Positions must be finite and
 *           |(x - origin)/h| < 2^31; that precondition is not checked.
 */
#ifndef MM_H
#define MM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MM_OK = 0,
  MM_ERR_NULL = 1,        /* a required pointer is NULL */
  MM_ERR_ARG = 2,         /* order, dtype, grid, sigma/beta or algo out of range */
  MM_ERR_UNSUPPORTED = 3, /* np or node count at or above 2^31, or a combination of dtype,
                             algorithm, field placement and grid dimension that is not
                             implemented (each entry point lists its own) */
  MM_ERR_WORKSPACE = 4,   /* *ws_bytes smaller than required */
  MM_ERR_HIP = 5,         /* a HIP launch or runtime call failed */
  MM_ERR_SCRATCH = 6      /* the workload needs more than the fixed scratch of
                             mm_assemble_ecsim_noalloc (MM_NOALLOC_SCRATCH_BYTES) */
} mm_status;

typedef enum { MM_F64 = 0, MM_F32 = 1, MM_MIX = 2 } mm_dtype;

/* Assembly algorithm. */
typedef enum {
  MM_ALGO_MFMA = 0,          /* per-bin matrix-core contraction + the library's default deposit */
  MM_ALGO_ATOMIC = 1,        /* conventional per-particle atomic scatter (comparison kernel);
                                ignores bin_start/perm, which may be NULL */
  MM_ALGO_MFMA_ATOMIC = 2,   /* per-bin matrix-core contraction, global-atomic deposit */
  MM_ALGO_VALU = 3           /* the same per-bin contraction and deposit as MM_ALGO_MFMA with the
                                products formed by fp64 vector FMAs instead of matrix instructions
                                (comparison kernel for the matrix cores); order 1 with MM_F64 or
                                MM_MIX and the field per particle only, else MM_ERR_UNSUPPORTED */
} mm_algo;

typedef struct {
  int32_t n[3];      /* cells (= nodes) per axis; each >= 2*order + 1 */
  double origin[3];  /* position of node (0,0,0) */
  double h[3];       /* node spacing, > 0 and finite */
} mm_grid;

/* Opaque stream handle: pass a hipStream_t (or NULL). */
typedef void* mm_stream_t;

/*
 * mm_bin_particles - counting sort of particles by support set.
 *
 * Groups particles whose B-spline supports coincide (the support-group
 * partition of Sec. 3.3; for CIC this is the cell, Sec. 2.3), keyed by the
 * linear index of the support's first node, which is a prerequisite of the
 * cell-wise assembly (Sec. 4.2 sorts particles by cell).
 *
 *  pos        [np][3] device array of dtype dt.
 *  bin_start  [n0*n1*n2 + 1] int32 output: bin k holds particles
 *             perm[bin_start[k] .. bin_start[k+1]-1]; bin_start[nbins] = np.
 *  perm       [np] int32 output: particle indices, bin by bin, ascending
 *             within a bin (a stable sort, so the result is unique).
 *  np == 0 fills bin_start with zeros. perm may be NULL when np == 0.
 */
mm_status mm_bin_particles(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                           int32_t* bin_start, int32_t* perm, void* ws, size_t* ws_bytes, mm_stream_t stream);

/*
 * mm_assemble_scalar - scalar mass matrix M_gg' = sigma * sum_p w_p W_pg W_pg'
 * (Eq. 6 with s_p = w_p; the scalar case of Sec. 3, as in FLIP/MPM, Sec. 1).
 *
 *  pos [np][3], w [np]: particle positions and weights (dtype dt).
 *  bin_start, perm: output of mm_bin_particles for the same grid, order,
 *             dtype and positions (required for the MFMA algorithms).
 *  M [nnodes][noff] output (dtype dt). accumulate == 0 overwrites M,
 *             accumulate != 0 adds to it (several species into one M).
 */
mm_status mm_assemble_scalar(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                             const void* w, const int32_t* bin_start, const int32_t* perm, double sigma,
                             int accumulate, mm_algo algo, void* M, void* ws, size_t* ws_bytes,
                             mm_stream_t stream);

/*
 * mm_assemble_ecsim - 3x3 tensorial ECSIM mass matrix
 *   M^{ij}_gg' = sigma * sum_p w_p alpha_p^{ij} W_pg W_pg'
 * with the per-particle magnetic response of the implicit-midpoint push,
 *   alpha_p = (I + beta^2 B_p B_p^T - beta [B_p]x) / (1 + beta^2 |B_p|^2),
 * [B]x u = B x u, beta = q dt / (2 m) of the species (Sec. 2.1 Eq. 6;
 * the page cites alpha as Eq. 5 in Sec. 4.1).
 *
 *  B [np][3]: magnetic field at each particle (dtype dt).
 *  M [nnodes][noff][3][3] output (dtype dt), row i of alpha first.
 *  Other arguments as for mm_assemble_scalar.
 * With MM_ALGO_MFMA on large second-order grids (mm_slab_planes) the
 * contraction and the deposition overlap by slabs of planes on two streams
 * of the device; M is bit-identical to mm_contract_bins followed by
 * mm_deposit_records, and the call stays ordered on `stream`.
 */
mm_status mm_assemble_ecsim(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                            const void* w, const void* B, const int32_t* bin_start, const int32_t* perm,
                            double beta, double sigma, int accumulate, mm_algo algo, void* M, void* ws,
                            size_t* ws_bytes, mm_stream_t stream);

/*
 * mm_assemble_ecsim_gridB - as mm_assemble_ecsim, with the magnetic field on
 * the grid nodes instead of per particle: each particle's field is gathered
 * with its own support weights, B_p = sum_a W_pa Bgrid[g_a] (the weights of
 * Sec. 2.3 Eq. 12), before alpha_p is formed. Sec. 4.1 names loading the field
 * and forming alpha_p as the non-matrix work of the tensorial kernels; here it
 * is fused into the particle preparation of the fp64 MFMA contraction, and
 * the other algorithms and fp32 interpolate B_p into the workspace first.
 *
 *  Bgrid [nnodes][3]: field at every node (dtype dt), node = x + nx*(y + ny*z).
 *  Other arguments as for mm_assemble_ecsim; the workspace size depends on
 *  whether the field is gathered in the contraction (query with ws == NULL).
 */
mm_status mm_assemble_ecsim_gridB(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                                  const void* w, const void* Bgrid, const int32_t* bin_start, const int32_t* perm,
                                  double beta, double sigma, int accumulate, mm_algo algo, void* M, void* ws,
                                  size_t* ws_bytes, mm_stream_t stream);

/*
 * The two phases of mm_assemble_* with MM_ALGO_MFMA, for callers that time,
 * overlap or reuse them. Calling both is the same as one MFMA assembly call.
 *
 * mm_contract_bins - the per-bin local matrices (Sec. 3.1 Eq. 15, batched as
 * in Sec. 3.2, one per support group of Sec. 3.3):
 *   rec[bin][pair(a,b)][comp] = sigma * sum_{p in bin} t_p^comp W_pa W_pb,
 * for support rows a <= b (upper triangle, pair(a,b) = a*N - a(a-1)/2 + b - a,
 * N = 8 or 27), comp as in M. B == NULL selects the scalar matrix (one comp);
 * with np == 0 a tensorial call still passes a non-NULL B (it is not read).
 * Order 2 tensorial on a 3D grid whose n[0] is a multiple of 4 (MM_F64,
 * MM_MIX, and MM_F32 with the field per particle or interpolated): the
 * records are instead summed over runs of four bins along x (first support
 * nodes 4r .. 4r+3, same y and z): one record per run holding the 999
 * canonical node pairs of the runs' 6 x 3 x 3 union support that some bin of
 * the run covers, 9,360 values per run (grouped by the row node's y and z,
 * each group's nine component planes padded to 16 values). The layout is the
 * library's own; the deposit entry points read it, and mm_record_bytes gives
 * its size.
 *  rec       device buffer of *rec_bytes bytes (query with rec == NULL),
 *            16-byte aligned (else MM_ERR_ARG). The records start at rec.
 *            For order 2 tensorial fp64 (and MM_MIX) the query also counts
 *            room after the records where the contraction orders the bins
 *            of each window of 256 by particle count (groups of bins with
 *            similar counts waste fewer matrix instructions); the records
 *            are the same.
 *  Other arguments as for mm_assemble_ecsim; bin_start/perm are required.
 *
 * mm_contract_bins_gridB - mm_contract_bins with the field on the grid
 * (Bgrid [nnodes][3], as for mm_assemble_ecsim_gridB); the records are
 * tensorial. For fp32 the query adds room after the records for the field
 * interpolated to the particles.
 *
 * mm_deposit_records - the sparse stencil deposition of Sec. 3.4: every
 * M[g][o][comp] is set (accumulate == 0) or incremented by the sum, in a fixed
 * order, of the records of all bins whose support holds both g and g+o.
 *  tensorial  1 for the 3x3 records (mm_contract_bins with B != NULL, or
 *             mm_contract_bins_gridB), else 0.
 */
mm_status mm_contract_bins(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos, const void* w,
                           const void* B, const int32_t* bin_start, const int32_t* perm, double beta, double sigma,
                           void* rec, size_t* rec_bytes, mm_stream_t stream);
mm_status mm_contract_bins_gridB(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                                 const void* w, const void* Bgrid, const int32_t* bin_start, const int32_t* perm,
                                 double beta, double sigma, void* rec, size_t* rec_bytes, mm_stream_t stream);
mm_status mm_deposit_records(const mm_grid* grid, int order, mm_dtype dt, int tensorial, const void* rec,
                             int accumulate, void* M, mm_stream_t stream);

/*
 * Strided particle arrays (fp64). The pages state the problem per particle
 * (position x_p, weight w_p and field B_p, Sec. 2.1 Eq. 6) and leave their
 * storage open; these entry points read them wherever the caller keeps them,
 * for instance one record per particle (an array of structures): particle p's
 * position is pos[p*pos_stride + 0..2], its weight w[p*w_stride] and its field
 * B[p*B_stride + 0..2], strides counted in doubles. With pos_stride 3,
 * w_stride 1 and B_stride 3 they are mm_bin_particles, mm_contract_bins and
 * mm_assemble_ecsim with MM_F64. Out of cell order a particle whose values
 * share one 64-byte record costs one random cache line of the contraction's
 * gathers instead of one per array.
 *
 * mm_bin_particles_strided - mm_bin_particles (MM_F64) on positions
 *   pos_stride doubles apart; bin_start and perm are bit for bit those of the
 *   dense copy of the positions. Any order.
 * mm_contract_bins_strided - mm_contract_bins (MM_F64, tensorial: B must not
 *   be NULL, even when np == 0); records bit for bit those of the dense arrays.
 * mm_assemble_ecsim_strided - mm_assemble_ecsim (MM_F64); M bit for bit that
 *   of the dense arrays.
 *  Strides other than the dense ones are read by the matrix-core path
 *  (MM_ALGO_MFMA) on a 3D grid, CIC and TSC (the other algorithms and the 2D
 *  problem are MM_ERR_UNSUPPORTED with them; at order 2 the strided assembly
 *  runs its two phases in turn, without the slab overlap). Each stride is at
 *  least 3 (pos, B) or 1 (w) and below 2^31, else MM_ERR_ARG; the arrays may
 *  overlap (they are only read). Other arguments, the workspace and the
 *  errors as for the dense entry points.
 */
mm_status mm_bin_particles_strided(const mm_grid* grid, int order, int64_t np, const double* pos,
                                   int64_t pos_stride, int32_t* bin_start, int32_t* perm, void* ws,
                                   size_t* ws_bytes, mm_stream_t stream);
mm_status mm_contract_bins_strided(const mm_grid* grid, int order, int64_t np, const double* pos,
                                   int64_t pos_stride, const double* w, int64_t w_stride, const double* B,
                                   int64_t B_stride, const int32_t* bin_start, const int32_t* perm, double beta,
                                   double sigma, void* rec, size_t* rec_bytes, mm_stream_t stream);
mm_status mm_assemble_ecsim_strided(const mm_grid* grid, int order, int64_t np, const double* pos,
                                    int64_t pos_stride, const double* w, int64_t w_stride, const double* B,
                                    int64_t B_stride, const int32_t* bin_start, const int32_t* perm, double beta,
                                    double sigma, int accumulate, mm_algo algo, void* M, void* ws,
                                    size_t* ws_bytes, mm_stream_t stream);

/*
 * Several species in one call. The ECSIM operator sums over the particles of
 * every species (Sec. 2.1 Eq. 6; Sec. 4.2 runs electrons and ions), each with
 * its own beta = q dt / (2 m). One species of the set:
 */
#define MM_MAX_SPECIES 8
typedef struct {
  int64_t np;                 /* particles of the species (>= 0, < 2^31) */
  const void* pos;            /* positions (dtype dt), particle p at pos[p*pos_stride + 0..2] */
  const void* w;              /* weights, w[p*w_stride] */
  const void* B;              /* field at each particle, B[p*B_stride + 0..2]; NULL: scalar records */
  const int32_t* bin_start;   /* mm_bin_particles of these positions (never NULL) */
  const int32_t* perm;        /* (may be NULL when np == 0) */
  double beta;                /* q dt / (2 m) of the species */
  int64_t pos_stride, w_stride, B_stride;  /* elements; 0 selects the dense 3, 1, 3 */
} mm_species;

/*
 * mm_contract_bins_species - mm_contract_bins of every species into ONE set
 * of records: each bin's record sums the particles of all species in it,
 * contracted in one launch (the per-bin accumulators run on from species to
 * species), so one record set is written and deposited instead of one per
 * species. rec, rec_bytes and the layout are those of mm_contract_bins.
 *  nspecies   1 .. MM_MAX_SPECIES (else MM_ERR_ARG); every species has a
 *             field (tensorial) or none (scalar), else MM_ERR_ARG.
 *  First order on a 3D grid with MM_F64 or MM_MIX only (other orders, MM_F32
 *  and 2D: MM_ERR_UNSUPPORTED; contract those species one by one and deposit
 *  with mm_deposit_records_multi). Strides as for the *_strided entry points
 *  (other than dense: MM_F64, tensorial).
 *
 * mm_assemble_ecsim_species - mm_assemble_ecsim of every species into one M
 * (accumulate as there, for the whole set). With MM_ALGO_MFMA where
 * mm_contract_bins_species applies, the species share one record set;
 * otherwise the species are assembled one after another into M, as by calls
 * of mm_assemble_ecsim (mm_assemble_ecsim_strided) with accumulate after the
 * first. Every species passes its field (B never NULL). The workspace query
 * covers whichever of the two is taken.
 */
mm_status mm_contract_bins_species(const mm_grid* grid, int order, mm_dtype dt, int nspecies,
                                   const mm_species* species, double sigma, void* rec, size_t* rec_bytes,
                                   mm_stream_t stream);
mm_status mm_assemble_ecsim_species(const mm_grid* grid, int order, mm_dtype dt, int nspecies,
                                    const mm_species* species, double sigma, int accumulate, mm_algo algo, void* M,
                                    void* ws, size_t* ws_bytes, mm_stream_t stream);

/*
 * mm_record_bytes - size in bytes of the records that mm_deposit_records,
 * mm_deposit_records_canonical and mm_deposit_records_multi read for this
 * grid, order, dtype (of M) and kind: the first part of the buffer that
 * mm_contract_bins fills (its own size query may add room after them). The
 * deposit entry points take no record length, so a caller that holds records
 * of unknown origin checks their size against this first. Nothing is enqueued.
 *  bytes  host output; NULL -> MM_ERR_NULL. Grid, order and dtype errors as
 *         for mm_deposit_records.
 */
mm_status mm_record_bytes(const mm_grid* grid, int order, mm_dtype dt, int tensorial, size_t* bytes);

/*
 * mm_deposit_records_canonical - mm_deposit_records into the canonical half of
 * the stencil (Sec. 3.4: (3^3+1)/2 = 14 offsets for CIC, (5^3+1)/2 = 63 for
 * TSC): only the displacements o >= 0 in (dz, dy, dx) lexicographic order are
 * stored, at Mc[g][k][comp] with k = o - centre (o the full offset index of
 * mm_assemble_*, centre = 13 or 62). The other half follows from the spatial
 * symmetry M[g][-o] = M[g-o][o] (component by component; not a transpose of
 * the 3x3 block). Each entry equals the full deposit's bit for bit.
 *  Mc  [nnodes][14 or 63][ncomp] (dtype dt); other arguments as for
 *      mm_deposit_records.
 */
mm_status mm_deposit_records_canonical(const mm_grid* grid, int order, mm_dtype dt, int tensorial, const void* rec,
                                       int accumulate, void* Mc, mm_stream_t stream);

/*
 * mm_deposit_records_multi - one deposition of several record sets, for the
 * sum over species of the field equation (Sec. 2.1: the mass matrices of all
 * species enter one operator). Each species is contracted into a record set
 * of its own (mm_contract_bins, same grid, order, dtype and kind); one pass
 * over M then adds, for every M[g][o][comp], the records of all bins whose
 * support holds both g and g+o, each term summed over the sets in their
 * order. The result equals depositing the sets one after the other
 * (accumulating) up to rounding, with one write of M instead of nrec, and
 * no re-read of M between species.
 *  canonical  0: the full stencil (as mm_deposit_records); 1: the canonical
 *             half (as mm_deposit_records_canonical).
 *  nrec       number of sets, 1 .. MM_MAX_RECORD_SETS (else MM_ERR_ARG).
 *  recs       host array of nrec device pointers (each as rec of
 *             mm_deposit_records; NULL entries give MM_ERR_NULL). The host
 *             array is read during the call only. M must not overlap any
 *             record set (the sets are read while M is written).
 *  2D grids: MM_ERR_UNSUPPORTED.
 */
#define MM_MAX_RECORD_SETS 4
mm_status mm_deposit_records_multi(const mm_grid* grid, int order, mm_dtype dt, int tensorial, int canonical,
                                   int nrec, const void* const* recs, int accumulate, void* M, mm_stream_t stream);

/*
 * Slabs of planes. The two phases above restricted to planes of the grid, for
 * callers that overlap them (mm_assemble_ecsim does so itself on large
 * grids) or bound the work of one call. The split by planes is this
 * library's; the page assembles the whole grid in one pass (Sec. 3). Only the
 * run records apply (order 2 tensorial on a 3D grid whose n[0] is a multiple
 * of 4; MM_F64 and MM_MIX, and MM_F32 with the field per particle); other
 * grids, orders or a NULL B give MM_ERR_UNSUPPORTED.
 *
 * mm_contract_bins_planes - mm_contract_bins for the bins whose first support
 * node lies in planes z0 <= z < z1 (0 <= z0 <= z1 <= n[2], else MM_ERR_ARG;
 * z0 == z1 enqueues nothing): the run records of those planes' runs, each
 * bit-identical to the one mm_contract_bins writes; the other runs' records
 * are not touched.
 *  rec        device buffer holding the records of the whole grid (rec_bytes
 *             of them, at least mm_record_bytes for dt, else
 *             MM_ERR_WORKSPACE), 16-byte aligned (else MM_ERR_ARG).
 *  Other arguments as for mm_contract_bins; bin_start and perm cover all
 *  particles (mm_bin_particles), the particles of other planes are not read.
 *
 * mm_deposit_records_planes - mm_deposit_records_multi for the nodes g of
 * planes z0 <= z < z1 only: it computes M[g][o] for those nodes and the
 * offsets o >= centre, and in the full stencil (canonical == 0) stores each
 * also at its mirrored entry M[g + d(o)][-o], a node of planes z .. z + 2
 * (periodic). Calls whose plane ranges partition 0 .. n[2] - 1 together
 * write every entry of M once, bit-identical to one mm_deposit_records_multi
 * call. The call reads the records of bin planes z0 - 2 .. z1 - 1 (periodic):
 * those must be complete, the others may still be written meanwhile.
 *  Arguments as for mm_deposit_records_multi, z0 and z1 as above.
 */
/*
 * mm_slab_planes - the slab thickness mm_assemble_ecsim and
 * mm_assemble_ecsim_gridB use with MM_ALGO_MFMA on this grid: on run-record
 * grids of at least 8192 cells per plane and 16 planes they contract slabs of
 * *planes bin planes in order (the last may be thinner) and deposit each
 * slab's completed node planes on a second stream of the device while the
 * next slab contracts (the library creates that stream and its events on the
 * device's first such call and keeps them; calls that overlap on one device
 * serialise their deposits on it). *planes = 0: the two phases run in turn.
 * The results are bit-identical either way. Nothing is enqueued.
 *  planes  host output; NULL -> MM_ERR_NULL. Grid and order errors as for
 *          mm_assemble_ecsim.
 */
mm_status mm_slab_planes(const mm_grid* grid, int order, int* planes);
mm_status mm_contract_bins_planes(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                                  const void* w, const void* B, const int32_t* bin_start, const int32_t* perm,
                                  double beta, double sigma, int z0, int z1, void* rec, size_t rec_bytes,
                                  mm_stream_t stream);
/*
 * mm_contract_bins_planes_gridB - mm_contract_bins_planes with the field on
 * the grid (Bgrid [nnodes][3], as for mm_contract_bins_gridB), gathered at
 * each particle inside the contraction: MM_F64 and MM_MIX (MM_F32, which
 * interpolates the field in a pass of its own first, gives
 * MM_ERR_UNSUPPORTED). Bgrid == NULL is MM_ERR_NULL.
 */
mm_status mm_contract_bins_planes_gridB(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                                        const void* w, const void* Bgrid, const int32_t* bin_start,
                                        const int32_t* perm, double beta, double sigma, int z0, int z1, void* rec,
                                        size_t rec_bytes, mm_stream_t stream);
mm_status mm_deposit_records_planes(const mm_grid* grid, int order, mm_dtype dt, int canonical, int nrec,
                                    const void* const* recs, int accumulate, int z0, int z1, void* M,
                                    mm_stream_t stream);

/*
 * mm_deposit_moments - deposition of per-particle quantities with the same
 * support weights: m[g][k] = sum_p W_pg Q_p[k], k < nq (1 <= nq <= 16), e.g.
 * charge and current (nq = 4) or the ten quantities of the implicit moment
 * method. Sec. 6 of the page names these scatters as further uses of the
 * same contraction, one operand holding the quantities and the other the
 * weights; here it runs per bin on the matrix cores with fp64 accumulation
 * (for both dtypes) and a fixed-order gather per node.
 *  pos [np][3], Q [np][nq] (dtype dt); bin_start, perm from mm_bin_particles
 *      (same grid, order, dtype and positions).
 *  m [nnodes][nq] (dtype dt): overwritten (accumulate == 0) or added to.
 *  ws: device workspace of *ws_bytes bytes, 16-byte aligned (query with
 *      ws == NULL): nnodes * (order + 1)^3 * nq * 8 bytes of per-bin records.
 *  nq outside [1, 16] is MM_ERR_ARG.
 */
mm_status mm_deposit_moments(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos, const void* Q,
                             int nq, const int32_t* bin_start, const int32_t* perm, int accumulate, void* m, void* ws,
                             size_t* ws_bytes, mm_stream_t stream);

/*
 * mm_stencil_matvec - the assembled matrix applied to a grid vector, as it
 * acts on the electric field in the implicit field equation (Sec. 2.1):
 *   y[g] = sum_o M[g][o] x[g+o]
 * with M[g][o] the 3x3 block (row i = comp / 3, column j = comp % 3) acting on
 * the 3-vector x[g+o] (tensorial != 0), or a scalar (tensorial == 0).
 *  canonical  0: M is the full stencil [nnodes][noff][ncomp]; 1: M is the
 *             canonical half of mm_deposit_records_canonical.
 *  x, y       [nnodes][3] (tensorial) or [nnodes], dtype dt; y is
 *             overwritten; x and y must not overlap (x == y is MM_ERR_ARG).
 */
mm_status mm_stencil_matvec(const mm_grid* grid, int order, mm_dtype dt, int tensorial, int canonical, const void* M,
                            const void* x, void* y, mm_stream_t stream);

/*
 * mm_probe_mfma_f64 - measurement aid, not part of the assembly: the on-box
 * throughput of v_mfma_f64_4x4x4_4b, the instruction of the fp64
 * contractions (the measured peak reported beside MI355X's published
 * 78.6 TFLOP/s fp64 matrix peak).
 *  nblocks  workgroups of 256 threads (1 .. 2^20); 4 per CU or more fill the chip
 *  iters    iterations (>= 1); every wave issues 16 * iters independent
 *           instructions of 512 flop each, so the work is
 *           nblocks * 4 * 16 * iters * 512 flop
 *  out      device buffer of nblocks * 256 doubles, owned by the caller;
 *           receives per-thread sums (so the work is not optimised away)
 * Enqueued on `stream`; time it with events. NULL out -> MM_ERR_NULL, counts
 * out of range -> MM_ERR_ARG.
 */
mm_status mm_probe_mfma_f64(int nblocks, int iters, double* out, mm_stream_t stream);

/*
 * mm_assemble_ecsim_noalloc - mm_assemble_ecsim with MM_ALGO_MFMA for callers
 * that cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, and harnesses that forbid allocation. It calls
 * no allocating routine. The per-bin records live in a fixed device array of
 * MM_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from the
 * library's first use on that GPU until the process ends; its address is
 * looked up once per device, on the first call with that device current.
 *
 *  Arguments as for mm_assemble_ecsim (algorithm MM_ALGO_MFMA, field per
 *  particle); the caller still owns pos, w, B, bin_start, perm and M, all on
 *  the current device.
 *  Limit: the records of the grid must fit the scratch: record bytes (see
 *  mm_record_bytes; rounded up to 256) <= MM_NOALLOC_SCRATCH_BYTES, e.g. CIC
 *  3x3 fp64 up to 25,890 nodes (29^3), CIC 3x3 fp32 up to 51,781 nodes, else
 *  MM_ERR_SCRATCH, before anything is enqueued.
 *  Every call on one GPU uses that GPU's one scratch array, whatever the
 *  stream: calls whose work overlaps on one GPU (other streams or threads)
 *  race on it and must be serialised by the caller. Each call writes the
 *  records it reads, so nothing left by an earlier call is read.
 */
#define MM_NOALLOC_SCRATCH_BYTES (64u << 20)
mm_status mm_assemble_ecsim_noalloc(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                                    const void* w, const void* B, const int32_t* bin_start, const int32_t* perm,
                                    double beta, double sigma, int accumulate, void* M, mm_stream_t stream);

/* Static description of a status code. */
const char* mm_status_string(mm_status s);

/* Library version string. */
const char* mm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MM_H */
