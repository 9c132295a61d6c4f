// C ABI of the mass-matrix library: host-side validation, workspace planning
// and kernel dispatch. Every argument error is reported before any HIP call.
#include <math.h>

#include <atomic>
#include <mutex>

#include "../../include/mm.h"
#include "mm_contract.h"

static_assert(MM_MAX_RECORD_SETS == mmk::MAX_REC, "record set limit of the ABI and the gather");
static_assert(MM_MAX_SPECIES == mmk::MAX_SPECIES, "species limit of the ABI and the contraction");

using namespace mmk;

namespace {

constexpr int64_t kMaxI32 = 2147483647LL;

bool is_finite_d(double v) { return isfinite(v) != 0; }

mm_status check_grid(const mm_grid* g, int order, int64_t* nnodes) {
  if (!g) return MM_ERR_NULL;
  if (order != 1 && order != 2) return MM_ERR_ARG;
  int64_t nn = 1;
  for (int d = 0; d < 3; ++d) {
    if (g->n[d] < 2 * order + 1 && !(d == 2 && g->n[2] == 1)) return MM_ERR_ARG;  // n[2] == 1: the 2D problem
    if (!(g->h[d] > 0.0) || !is_finite_d(g->h[d]) || !is_finite_d(g->origin[d])) return MM_ERR_ARG;
    nn *= g->n[d];
  }
  if (nn >= kMaxI32) return MM_ERR_UNSUPPORTED;
  *nnodes = nn;
  return MM_OK;
}

GridDev to_dev(const mm_grid* g) {
  GridDev d;
  d.n0 = g->n[0];
  d.n1 = g->n[1];
  d.n2 = g->n[2];
  d.o0 = g->origin[0];
  d.o1 = g->origin[1];
  d.o2 = g->origin[2];
  d.h0 = g->h[0];
  d.h1 = g->h[1];
  d.h2 = g->h[2];
  d.i0 = 1.0 / g->h[0];
  d.i1 = 1.0 / g->h[1];
  d.i2 = 1.0 / g->h[2];
  d.exact = 0;
  for (int k = 0; k < 3; ++k) {
    // a power of two well inside the fp32 range: multiplying by 1/h is then
    // exact in fp64 and in fp32 alike
    int ex = 0;
    const double m = frexp(g->h[k], &ex);
    if (m == 0.5 && ex > -100 && ex < 100) d.exact |= 1 << k;
  }
  return d;
}

mm_status hip_status(hipError_t e) { return e == hipSuccess ? MM_OK : MM_ERR_HIP; }

bool dtype_ok(mm_dtype dt) { return dt == MM_F64 || dt == MM_F32 || dt == MM_MIX; }

bool is2d(const mm_grid* g) { return g->n[2] == 1; }

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Element strides of the particle arrays: position p at pos[ps p + 0..2],
// weight at w[wst p], field at B[bst p + 0..2]. Dense arrays are 3, 1, 3.
struct Strides {
  int64_t ps = 3, wst = 1, bst = 3;
  bool dense() const { return ps == 3 && wst == 1 && bst == 3; }
  bool valid() const { return ps >= 3 && wst >= 1 && bst >= 3 && ps <= kMaxI32 && wst <= kMaxI32 && bst <= kMaxI32; }
};

// Other strides than the dense ones are read by the fp64 3x3 record
// contractions (CIC and TSC, 3D, field per particle) only.
mm_status check_strides(const Strides& st, const mm_grid* grid, mm_dtype dt, bool tensorial, const void* Bgrid) {
  if (st.dense()) return MM_OK;
  if (!st.valid()) return MM_ERR_ARG;
  if (dt != MM_F64 || is2d(grid) || Bgrid || !tensorial) return MM_ERR_UNSUPPORTED;
  return MM_OK;
}

// The record contraction of the two-phase path; strided second-order arrays
// go to the fp64 TSC kernel directly (the generic dispatch takes dense ones).
hipError_t contract_records(const GridDev& g, int order, bool f32, const Particles& P, const int32_t* bin_start,
                            const int32_t* perm, double beta, double sigma, void* rec, hipStream_t s) {
  if (P.strided() && order == 2) return launch_tsc64(g, P, bin_start, perm, beta, sigma, (double*)rec, s);
  return launch_contract(g, order, f32, P, bin_start, perm, beta, sigma, MODE_RECORD, rec, s);
}

// ------------------------------------------------------------ fixed scratch
// Device scratch of the allocation-free entry point mm_assemble_ecsim_noalloc:
// the per-bin records of the two-phase assembly live here instead of in a
// caller workspace. One copy per GPU, created when the library's code object
// is loaded there and held until the process ends. In host code `scratch`
// names a host-side stand-in, never the device memory: kernels and copies take
// the address hipGetSymbolAddress returns for the current device, looked up
// once per device and kept in scratch_ptr.
constexpr size_t kScratchBytes = (size_t)MM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];
std::mutex scratch_mu;

// The scratch address on the current device (looked up on the first call there).
mm_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MM_ERR_HIP;
  if (dev >= kMaxDevices) return MM_ERR_UNSUPPORTED;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return MM_ERR_HIP;
      scratch_ptr[dev].store(q, std::memory_order_release);
      p = q;
    }
  }
  *out = p;
  return MM_OK;
}

// Shared argument checks of the assembly entry points. The tensorial field is
// per particle (B) or on the grid nodes (Bgrid, gathered at each particle).
// fixed_max > 0: ws is the library's own fixed device scratch of fixed_max
// bytes (the allocation-free entry point): no size query, and a workload that
// needs more is MM_ERR_SCRATCH.
mm_status assemble_common(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos, const void* w,
                          const void* B, const void* Bgrid, bool tensorial, const int32_t* bin_start,
                          const int32_t* perm, double beta, double sigma, mm_algo algo, void* M, void* ws,
                          size_t* ws_bytes, mm_stream_t stream, int accumulate, size_t fixed_max = 0,
                          const Strides& str = Strides()) {
  if (!ws_bytes && fixed_max == 0) return MM_ERR_NULL;
  int64_t nnodes = 0;
  mm_status st = check_grid(grid, order, &nnodes);
  if (st != MM_OK) return st;
  if (!dtype_ok(dt)) return MM_ERR_ARG;
  if (algo != MM_ALGO_MFMA && algo != MM_ALGO_ATOMIC && algo != MM_ALGO_MFMA_ATOMIC && algo != MM_ALGO_VALU)
    return MM_ERR_ARG;
  if ((st = check_strides(str, grid, dt, tensorial, Bgrid)) != MM_OK) return st;
  if (!str.dense() && algo != MM_ALGO_MFMA) return MM_ERR_UNSUPPORTED;
  if (algo == MM_ALGO_ATOMIC && dt == MM_MIX) return MM_ERR_UNSUPPORTED;
  // the vector-FMA comparison contraction: CIC, fp64 arithmetic, 3D, field per particle
  if (algo == MM_ALGO_VALU && (order != 1 || dt == MM_F32 || is2d(grid) || Bgrid)) return MM_ERR_UNSUPPORTED;
  // 2D: the matrix-core path in fp64 (or the mixed layout), field per particle
  if (is2d(grid) && (algo != MM_ALGO_MFMA || dt == MM_F32 || Bgrid)) return MM_ERR_UNSUPPORTED;
  if (!is_finite_d(sigma) || !is_finite_d(beta)) return MM_ERR_ARG;
  if (np < 0) return MM_ERR_ARG;
  if (np >= kMaxI32) return MM_ERR_UNSUPPORTED;
  if (!M) return MM_ERR_NULL;
  const bool mfma = algo != MM_ALGO_ATOMIC;
  if (np > 0) {
    if (!pos || !w || (tensorial && !B && !Bgrid)) return MM_ERR_NULL;
    if (mfma && (!bin_start || !perm)) return MM_ERR_NULL;
  }
  const bool f32 = dt == MM_F32;
  const size_t elem = f32 ? 4 : 8;
  // The two-phase deposit keeps one packed record per bin; the atomic
  // deposits need no workspace. A grid field that the chosen kernel does not
  // gather itself is first interpolated to the particles, after the records.
  const bool records = (algo == MM_ALGO_MFMA || algo == MM_ALGO_VALU) && np > 0;
  const size_t rec_need =
      records ? align256(is2d(grid) ? record_bytes_2d(order, tensorial, nnodes) : record_bytes(order, f32, tensorial, to_dev(grid)))
              : 0;
  const bool interp = Bgrid && np > 0 &&
                      !(records && contract_gathers_field(order, f32, MODE_RECORD));
  // fp32 positions with an fp64 interpolated field: not a combination the kernels take
  if (interp && dt == MM_MIX) return MM_ERR_UNSUPPORTED;
  const size_t need = rec_need + (interp ? (size_t)np * 3 * elem : 0);
  if (fixed_max > 0) {
    if (need > fixed_max) return MM_ERR_SCRATCH;
    if (need > 0 && (st = scratch_of_current_device(&ws)) != MM_OK) return st;
  } else {
    if (!ws) {
      *ws_bytes = need;
      return MM_OK;
    }
    if (*ws_bytes < need) return MM_ERR_WORKSPACE;
    if (need > 0 && ((uintptr_t)ws & 15) != 0) return MM_ERR_ARG;
  }

  const int noff = is2d(grid) ? (order == 1 ? 9 : 25) : (order == 1 ? 27 : 125);
  const size_t count = (size_t)nnodes * noff * (tensorial ? 9 : 1);
  hipStream_t s = (hipStream_t)stream;
  GridDev g = to_dev(grid);
  hipError_t e = hipSuccess;
  Particles P{pos, w, tensorial ? B : nullptr, (int)np};
  P.pos32 = dt == MM_MIX;
  P.ps = str.ps;
  P.wst = str.wst;
  P.bst = str.bst;
  if (Bgrid && np > 0) {
    if (interp) {
      void* bp = (char*)ws + rec_need;
      e = launch_interp_field(g, order, f32, pos, (int)np, Bgrid, bp, s, P.pos32);
      if (e != hipSuccess) return hip_status(e);
      P.B = bp;
    } else {
      P.Bgrid = Bgrid;
    }
  }
  if (records && is2d(grid)) {
    e = launch_contract_2d(g, order, P, bin_start, perm, beta, sigma, ws, s);
    if (e == hipSuccess) e = launch_gather_2d(g, order, tensorial, ws, accumulate, M, s);
    return hip_status(e);
  }
  // Large run-record grids: the two phases overlapped by slabs of planes
  // (bit-identical results). Not in the allocation-free entry point, whose
  // callers may not let the library create its second stream.
  if (records && algo == MM_ALGO_MFMA && fixed_max == 0 && tensorial && order == 2 && overlap_slabs(g) >= 2 &&
      contract_planes_apply(g, order, f32, P))
    return hip_status(launch_assemble_overlapped(g, f32, P, bin_start, perm, beta, sigma, ws, accumulate, M, s));
  if (records) {
    e = algo == MM_ALGO_VALU ? launch_cic64_valu(g, P, bin_start, perm, beta, sigma, (double*)ws, s)
                             : contract_records(g, order, f32, P, bin_start, perm, beta, sigma, ws, s);
    if (e == hipSuccess) {
      const void* recs[1] = {ws};
      e = launch_gather(g, order, f32, tensorial, recs, 1, accumulate, M, s);
    }
    return hip_status(e);
  }
  if (!accumulate) e = launch_fill_zero(M, count, f32, s);
  if (e != hipSuccess || np == 0) return hip_status(e);
  if (algo == MM_ALGO_ATOMIC)
    e = launch_atomic_scatter(g, order, f32, P, beta, sigma, M, s);
  else
    e = launch_contract(g, order, f32, P, bin_start, perm, beta, sigma, MODE_ATOMIC, M, s);
  return hip_status(e);
}

// mm_contract_bins with the field per particle (B) or on the grid (Bgrid).
mm_status contract_common(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos, const void* w,
                          const void* B, const void* Bgrid, const int32_t* bin_start, const int32_t* perm,
                          double beta, double sigma, void* rec, size_t* rec_bytes, mm_stream_t stream,
                          const Strides& str = Strides()) {
  if (!rec_bytes) return MM_ERR_NULL;
  int64_t nnodes = 0;
  mm_status st = check_grid(grid, order, &nnodes);
  if (st != MM_OK) return st;
  if (!dtype_ok(dt)) return MM_ERR_ARG;
  if ((st = check_strides(str, grid, dt, B != nullptr || Bgrid != nullptr, Bgrid)) != MM_OK) return st;
  if (!is_finite_d(sigma) || !is_finite_d(beta)) return MM_ERR_ARG;
  if (np < 0) return MM_ERR_ARG;
  if (np >= kMaxI32) return MM_ERR_UNSUPPORTED;
  if (!bin_start || (np > 0 && (!pos || !w || !perm))) return MM_ERR_NULL;
  if (Bgrid && np > 0 && !pos) return MM_ERR_NULL;
  const bool f32 = dt == MM_F32;
  const bool tensorial = B != nullptr || Bgrid != nullptr;
  if (is2d(grid) && (f32 || Bgrid)) return MM_ERR_UNSUPPORTED;
  const size_t rec_need = is2d(grid) ? record_bytes_2d(order, tensorial, nnodes) : record_bytes(order, f32, tensorial, to_dev(grid));
  const bool interp = Bgrid && np > 0 && !contract_gathers_field(order, f32, MODE_RECORD);
  const size_t need = interp ? align256(rec_need) + (size_t)np * 3 * (f32 ? 4 : 8) : rec_need;
  if (!rec) {
    *rec_bytes = need;
    return MM_OK;
  }
  if (*rec_bytes < need) return MM_ERR_WORKSPACE;
  if (((uintptr_t)rec & 15) != 0) return MM_ERR_ARG;
  GridDev g = to_dev(grid);
  hipStream_t s = (hipStream_t)stream;
  Particles P{pos, w, B, (int)np};
  P.pos32 = dt == MM_MIX;
  P.ps = str.ps;
  P.wst = str.wst;
  P.bst = str.bst;
  if (Bgrid) {
    if (interp) {
      void* bp = (char*)rec + align256(rec_need);
      hipError_t e = launch_interp_field(g, order, f32, pos, (int)np, Bgrid, bp, s);
      if (e != hipSuccess) return hip_status(e);
      P.B = bp;
    } else {
      P.Bgrid = Bgrid;
    }
  }
  if (is2d(grid)) return hip_status(launch_contract_2d(g, order, P, bin_start, perm, beta, sigma, rec, s));
  return hip_status(contract_records(g, order, f32, P, bin_start, perm, beta, sigma, rec, s));
}

// mm_contract_bins_planes with the field per particle (B) or on the grid (Bgrid).
mm_status contract_planes_common(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                                 const void* w, const void* B, const void* Bgrid, const int32_t* bin_start,
                                 const int32_t* perm, double beta, double sigma, int z0, int z1, void* rec,
                                 size_t rec_bytes, mm_stream_t stream) {
  int64_t nnodes = 0;
  mm_status st = check_grid(grid, order, &nnodes);
  if (st != MM_OK) return st;
  if (!dtype_ok(dt)) return MM_ERR_ARG;
  if (!is_finite_d(sigma) || !is_finite_d(beta)) return MM_ERR_ARG;
  if (np < 0) return MM_ERR_ARG;
  if (np >= kMaxI32) return MM_ERR_UNSUPPORTED;
  if (!rec || !bin_start || (np > 0 && (!pos || !w || !perm))) return MM_ERR_NULL;
  if (z0 < 0 || z0 > z1 || z1 > grid->n[2]) return MM_ERR_ARG;
  const bool f32 = dt == MM_F32;
  const GridDev g = to_dev(grid);
  Particles P{pos, w, B, (int)np};
  P.pos32 = dt == MM_MIX;
  P.Bgrid = Bgrid;
  if (is2d(grid) || !(B || Bgrid) || !contract_planes_apply(g, order, f32, P)) return MM_ERR_UNSUPPORTED;
  if (rec_bytes < record_bytes(order, f32, true, g)) return MM_ERR_WORKSPACE;
  if (((uintptr_t)rec & 15) != 0) return MM_ERR_ARG;
  return hip_status(launch_contract_planes(g, f32, P, bin_start, perm, beta, sigma, rec, z0, z1,
                                           (hipStream_t)stream));
}

// ----------------------------------------------------------- species sets
// Strides of one species (0 selects the dense value).
Strides species_strides(const mm_species& sp) {
  Strides st;
  st.ps = sp.pos_stride ? sp.pos_stride : 3;
  st.wst = sp.w_stride ? sp.w_stride : 1;
  st.bst = sp.B_stride ? sp.B_stride : 3;
  return st;
}

// Whether one launch contracts the whole set: first order, 3D, fp64 arithmetic.
bool species_fused(const mm_grid* grid, int order, mm_dtype dt) {
  return order == 1 && !is2d(grid) && dt != MM_F32;
}

// Checks shared by the species entry points; *tensorial is the kind of the set.
mm_status check_species(const mm_grid* grid, int order, mm_dtype dt, int ns, const mm_species* sp,
                        bool* tensorial) {
  if (ns < 1 || ns > MM_MAX_SPECIES) return MM_ERR_ARG;
  if (!sp) return MM_ERR_NULL;
  *tensorial = sp[0].B != nullptr;
  for (int i = 0; i < ns; ++i) {
    const mm_species& s = sp[i];
    if (s.np < 0 || !is_finite_d(s.beta)) return MM_ERR_ARG;
    if (s.np >= kMaxI32) return MM_ERR_UNSUPPORTED;
    if ((s.B != nullptr) != *tensorial) return MM_ERR_ARG;
    if (!s.bin_start) return MM_ERR_NULL;
    if (s.np > 0 && (!s.pos || !s.w || !s.perm)) return MM_ERR_NULL;
    const mm_status st = check_strides(species_strides(s), grid, dt, *tensorial, nullptr);
    if (st != MM_OK) return st;
  }
  return MM_OK;
}

// The set as the contraction's particle descriptors.
struct SpeciesArgs {
  Particles P[MM_MAX_SPECIES];
  const int32_t* bin_start[MM_MAX_SPECIES];
  const int32_t* perm[MM_MAX_SPECIES];
  double beta[MM_MAX_SPECIES];
};
void species_args(mm_dtype dt, int ns, const mm_species* sp, SpeciesArgs* a) {
  for (int i = 0; i < ns; ++i) {
    a->P[i] = Particles{sp[i].pos, sp[i].w, sp[i].B, (int)sp[i].np};
    a->P[i].pos32 = dt == MM_MIX;
    const Strides st = species_strides(sp[i]);
    a->P[i].ps = st.ps;
    a->P[i].wst = st.wst;
    a->P[i].bst = st.bst;
    a->bin_start[i] = sp[i].bin_start;
    a->perm[i] = sp[i].perm;
    a->beta[i] = sp[i].beta;
  }
}

// mm_bin_particles with the positions ps elements apart (3 when dense).
mm_status bin_common(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos, int64_t ps,
                     int32_t* bin_start, int32_t* perm, void* ws, size_t* ws_bytes, mm_stream_t stream) {
  if (!ws_bytes) return MM_ERR_NULL;
  int64_t nnodes = 0;
  mm_status st = check_grid(grid, order, &nnodes);
  if (st != MM_OK) return st;
  if (!dtype_ok(dt)) return MM_ERR_ARG;
  if (np < 0 || ps < 3 || ps > kMaxI32) return MM_ERR_ARG;
  if (np >= kMaxI32) return MM_ERR_UNSUPPORTED;
  if (!bin_start) return MM_ERR_NULL;
  if (np > 0 && (!pos || !perm)) return MM_ERR_NULL;
  const size_t need = np > 0 ? bin_workspace_bytes(np, nnodes) : 0;
  if (!ws) {
    *ws_bytes = need;
    return MM_OK;
  }
  if (*ws_bytes < need) return MM_ERR_WORKSPACE;
  return hip_status(launch_bin(to_dev(grid), order, dt == MM_F32, pos, (int)np, (int)nnodes, bin_start, perm, ws,
                               (hipStream_t)stream, dt == MM_MIX, ps));
}

}  // namespace

extern "C" {

mm_status mm_assemble_ecsim_noalloc(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                                    const void* w, const void* B, const int32_t* bin_start, const int32_t* perm,
                                    double beta, double sigma, int accumulate, void* M, mm_stream_t stream) {
  // the scratch address is looked up inside, after every argument check passed
  return assemble_common(grid, order, dt, np, pos, w, B, nullptr, true, bin_start, perm, beta, sigma, MM_ALGO_MFMA,
                         M, nullptr, nullptr, stream, accumulate, kScratchBytes);
}

mm_status mm_bin_particles(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                           int32_t* bin_start, int32_t* perm, void* ws, size_t* ws_bytes, mm_stream_t stream) {
  return bin_common(grid, order, dt, np, pos, 3, bin_start, perm, ws, ws_bytes, stream);
}

mm_status mm_bin_particles_strided(const mm_grid* grid, int order, int64_t np, const double* pos,
                                   int64_t pos_stride, int32_t* bin_start, int32_t* perm, void* ws,
                                   size_t* ws_bytes, mm_stream_t stream) {
  return bin_common(grid, order, MM_F64, np, pos, pos_stride, bin_start, perm, ws, ws_bytes, stream);
}

mm_status mm_contract_bins_strided(const mm_grid* grid, int order, int64_t np, const double* pos,
                                   int64_t pos_stride, const double* w, int64_t w_stride, const double* B,
                                   int64_t B_stride, const int32_t* bin_start, const int32_t* perm, double beta,
                                   double sigma, void* rec, size_t* rec_bytes, mm_stream_t stream) {
  if (!B) return MM_ERR_NULL;  // the records are tensorial, also when np == 0
  Strides st;
  st.ps = pos_stride;
  st.wst = w_stride;
  st.bst = B_stride;
  return contract_common(grid, order, MM_F64, np, pos, w, B, nullptr, bin_start, perm, beta, sigma, rec, rec_bytes,
                         stream, st);
}

mm_status mm_assemble_ecsim_strided(const mm_grid* grid, int order, int64_t np, const double* pos,
                                    int64_t pos_stride, const double* w, int64_t w_stride, const double* B,
                                    int64_t B_stride, const int32_t* bin_start, const int32_t* perm, double beta,
                                    double sigma, int accumulate, mm_algo algo, void* M, void* ws,
                                    size_t* ws_bytes, mm_stream_t stream) {
  Strides st;
  st.ps = pos_stride;
  st.wst = w_stride;
  st.bst = B_stride;
  return assemble_common(grid, order, MM_F64, np, pos, w, B, nullptr, true, bin_start, perm, beta, sigma, algo, M,
                         ws, ws_bytes, stream, accumulate, 0, st);
}

mm_status mm_contract_bins_species(const mm_grid* grid, int order, mm_dtype dt, int nspecies,
                                   const mm_species* species, double sigma, void* rec, size_t* rec_bytes,
                                   mm_stream_t stream) {
  if (!rec_bytes) return MM_ERR_NULL;
  int64_t nnodes = 0;
  mm_status st = check_grid(grid, order, &nnodes);
  if (st != MM_OK) return st;
  if (!dtype_ok(dt) || !is_finite_d(sigma)) return MM_ERR_ARG;
  bool tensorial = false;
  if ((st = check_species(grid, order, dt, nspecies, species, &tensorial)) != MM_OK) return st;
  if (!species_fused(grid, order, dt)) return MM_ERR_UNSUPPORTED;
  const GridDev g = to_dev(grid);
  const size_t need = record_bytes(order, false, tensorial, g);
  if (!rec) {
    *rec_bytes = need;
    return MM_OK;
  }
  if (*rec_bytes < need) return MM_ERR_WORKSPACE;
  if (((uintptr_t)rec & 15) != 0) return MM_ERR_ARG;
  SpeciesArgs a;
  species_args(dt, nspecies, species, &a);
  return hip_status(launch_cic64_species(g, nspecies, a.P, a.bin_start, a.perm, a.beta, sigma, (double*)rec,
                                         (hipStream_t)stream));
}

mm_status mm_assemble_ecsim_species(const mm_grid* grid, int order, mm_dtype dt, int nspecies,
                                    const mm_species* species, double sigma, int accumulate, mm_algo algo, void* M,
                                    void* ws, size_t* ws_bytes, mm_stream_t stream) {
  if (!ws_bytes) return MM_ERR_NULL;
  int64_t nnodes = 0;
  mm_status st = check_grid(grid, order, &nnodes);
  if (st != MM_OK) return st;
  if (!dtype_ok(dt) || !is_finite_d(sigma)) return MM_ERR_ARG;
  if (algo != MM_ALGO_MFMA && algo != MM_ALGO_ATOMIC && algo != MM_ALGO_MFMA_ATOMIC && algo != MM_ALGO_VALU)
    return MM_ERR_ARG;
  bool tensorial = false;
  if ((st = check_species(grid, order, dt, nspecies, species, &tensorial)) != MM_OK) return st;
  if (!tensorial) return MM_ERR_NULL;
  if (!M) return MM_ERR_NULL;
  hipStream_t s = (hipStream_t)stream;
  if (algo == MM_ALGO_MFMA && species_fused(grid, order, dt)) {  // one record set for the whole set
    const GridDev g = to_dev(grid);
    const size_t need = align256(record_bytes(order, false, true, g));
    if (!ws) {
      *ws_bytes = need;
      return MM_OK;
    }
    if (*ws_bytes < need) return MM_ERR_WORKSPACE;
    if (((uintptr_t)ws & 15) != 0) return MM_ERR_ARG;
    SpeciesArgs a;
    species_args(dt, nspecies, species, &a);
    hipError_t e = launch_cic64_species(g, nspecies, a.P, a.bin_start, a.perm, a.beta, sigma, (double*)ws, s);
    if (e == hipSuccess) {
      const void* recs[1] = {ws};
      e = launch_gather(g, order, false, true, recs, 1, accumulate, M, s);
    }
    return hip_status(e);
  }
  // species after species, accumulating into M
  size_t need = 0;
  for (int i = 0; i < nspecies; ++i) {
    const mm_species& sp = species[i];
    size_t b = 0;
    st = assemble_common(grid, order, dt, sp.np, sp.pos, sp.w, sp.B, nullptr, true, sp.bin_start, sp.perm, sp.beta,
                         sigma, algo, M, nullptr, &b, stream, 1, 0, species_strides(sp));
    if (st != MM_OK) return st;
    need = b > need ? b : need;
  }
  if (!ws) {
    *ws_bytes = need;
    return MM_OK;
  }
  if (*ws_bytes < need) return MM_ERR_WORKSPACE;
  for (int i = 0; i < nspecies; ++i) {
    const mm_species& sp = species[i];
    size_t b = *ws_bytes;
    st = assemble_common(grid, order, dt, sp.np, sp.pos, sp.w, sp.B, nullptr, true, sp.bin_start, sp.perm, sp.beta,
                         sigma, algo, M, ws, &b, stream, accumulate || i > 0, 0, species_strides(sp));
    if (st != MM_OK) return st;
  }
  return MM_OK;
}

mm_status mm_assemble_scalar(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                             const void* w, const int32_t* bin_start, const int32_t* perm, double sigma,
                             int accumulate, mm_algo algo, void* M, void* ws, size_t* ws_bytes,
                             mm_stream_t stream) {
  return assemble_common(grid, order, dt, np, pos, w, nullptr, nullptr, false, bin_start, perm, 0.0, sigma, algo, M,
                         ws, ws_bytes, stream, accumulate);
}

mm_status mm_assemble_ecsim(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                            const void* w, const void* B, const int32_t* bin_start, const int32_t* perm,
                            double beta, double sigma, int accumulate, mm_algo algo, void* M, void* ws,
                            size_t* ws_bytes, mm_stream_t stream) {
  return assemble_common(grid, order, dt, np, pos, w, B, nullptr, true, bin_start, perm, beta, sigma, algo, M, ws,
                         ws_bytes, stream, accumulate);
}

mm_status mm_assemble_ecsim_gridB(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                                  const void* w, const void* Bgrid, const int32_t* bin_start, const int32_t* perm,
                                  double beta, double sigma, int accumulate, mm_algo algo, void* M, void* ws,
                                  size_t* ws_bytes, mm_stream_t stream) {
  return assemble_common(grid, order, dt, np, pos, w, nullptr, Bgrid, true, bin_start, perm, beta, sigma, algo, M,
                         ws, ws_bytes, stream, accumulate);
}

mm_status mm_contract_bins(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos, const void* w,
                           const void* B, const int32_t* bin_start, const int32_t* perm, double beta, double sigma,
                           void* rec, size_t* rec_bytes, mm_stream_t stream) {
  return contract_common(grid, order, dt, np, pos, w, B, nullptr, bin_start, perm, beta, sigma, rec, rec_bytes,
                         stream);
}

mm_status mm_contract_bins_gridB(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                                 const void* w, const void* Bgrid, const int32_t* bin_start, const int32_t* perm,
                                 double beta, double sigma, void* rec, size_t* rec_bytes, mm_stream_t stream) {
  if (!Bgrid) return MM_ERR_NULL;
  return contract_common(grid, order, dt, np, pos, w, nullptr, Bgrid, bin_start, perm, beta, sigma, rec, rec_bytes,
                         stream);
}

mm_status mm_record_bytes(const mm_grid* grid, int order, mm_dtype dt, int tensorial, size_t* bytes) {
  if (!bytes) return MM_ERR_NULL;
  int64_t nnodes = 0;
  mm_status st = check_grid(grid, order, &nnodes);
  if (st != MM_OK) return st;
  if (!dtype_ok(dt)) return MM_ERR_ARG;
  if (is2d(grid) && dt == MM_F32) return MM_ERR_UNSUPPORTED;
  *bytes = is2d(grid) ? record_bytes_2d(order, tensorial != 0, nnodes)
                      : record_bytes(order, dt == MM_F32, tensorial != 0, to_dev(grid));
  return MM_OK;
}

mm_status mm_deposit_records(const mm_grid* grid, int order, mm_dtype dt, int tensorial, const void* rec,
                             int accumulate, void* M, mm_stream_t stream) {
  int64_t nnodes = 0;
  mm_status st = check_grid(grid, order, &nnodes);
  if (st != MM_OK) return st;
  if (!dtype_ok(dt)) return MM_ERR_ARG;
  if (!rec || !M) return MM_ERR_NULL;
  if (is2d(grid)) {
    if (dt == MM_F32) return MM_ERR_UNSUPPORTED;
    return hip_status(launch_gather_2d(to_dev(grid), order, tensorial != 0, rec, accumulate, M, (hipStream_t)stream));
  }
  const void* recs[1] = {rec};
  return hip_status(launch_gather(to_dev(grid), order, dt == MM_F32, tensorial != 0, recs, 1, accumulate, M,
                                  (hipStream_t)stream));
}

mm_status mm_deposit_records_canonical(const mm_grid* grid, int order, mm_dtype dt, int tensorial, const void* rec,
                                       int accumulate, void* Mc, mm_stream_t stream) {
  int64_t nnodes = 0;
  mm_status st = check_grid(grid, order, &nnodes);
  if (st != MM_OK) return st;
  if (!dtype_ok(dt)) return MM_ERR_ARG;
  if (!rec || !Mc) return MM_ERR_NULL;
  if (is2d(grid)) return MM_ERR_UNSUPPORTED;
  const void* recs[1] = {rec};
  return hip_status(launch_gather(to_dev(grid), order, dt == MM_F32, tensorial != 0, recs, 1, accumulate, Mc,
                                  (hipStream_t)stream, true));
}

mm_status mm_deposit_records_multi(const mm_grid* grid, int order, mm_dtype dt, int tensorial, int canonical,
                                   int nrec, const void* const* recs, int accumulate, void* M, mm_stream_t stream) {
  int64_t nnodes = 0;
  mm_status st = check_grid(grid, order, &nnodes);
  if (st != MM_OK) return st;
  if (!dtype_ok(dt)) return MM_ERR_ARG;
  if (nrec < 1 || nrec > MM_MAX_RECORD_SETS) return MM_ERR_ARG;
  if (!recs || !M) return MM_ERR_NULL;
  for (int q = 0; q < nrec; ++q)
    if (!recs[q]) return MM_ERR_NULL;
  if (is2d(grid)) return MM_ERR_UNSUPPORTED;
  return hip_status(launch_gather(to_dev(grid), order, dt == MM_F32, tensorial != 0, recs, nrec, accumulate, M,
                                  (hipStream_t)stream, canonical != 0));
}

mm_status mm_slab_planes(const mm_grid* grid, int order, int* planes) {
  if (!planes) return MM_ERR_NULL;
  int64_t nnodes = 0;
  mm_status st = check_grid(grid, order, &nnodes);
  if (st != MM_OK) return st;
  *planes = order == 2 && !is2d(grid) ? overlap_slab_planes(to_dev(grid)) : 0;
  return MM_OK;
}

mm_status mm_contract_bins_planes(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                                  const void* w, const void* B, const int32_t* bin_start, const int32_t* perm,
                                  double beta, double sigma, int z0, int z1, void* rec, size_t rec_bytes,
                                  mm_stream_t stream) {
  return contract_planes_common(grid, order, dt, np, pos, w, B, nullptr, bin_start, perm, beta, sigma, z0, z1, rec,
                                rec_bytes, stream);
}

mm_status mm_contract_bins_planes_gridB(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos,
                                        const void* w, const void* Bgrid, const int32_t* bin_start,
                                        const int32_t* perm, double beta, double sigma, int z0, int z1, void* rec,
                                        size_t rec_bytes, mm_stream_t stream) {
  if (!Bgrid) return MM_ERR_NULL;
  return contract_planes_common(grid, order, dt, np, pos, w, nullptr, Bgrid, bin_start, perm, beta, sigma, z0, z1,
                                rec, rec_bytes, stream);
}

mm_status mm_deposit_records_planes(const mm_grid* grid, int order, mm_dtype dt, int canonical, int nrec,
                                    const void* const* recs, int accumulate, int z0, int z1, void* M,
                                    mm_stream_t stream) {
  int64_t nnodes = 0;
  mm_status st = check_grid(grid, order, &nnodes);
  if (st != MM_OK) return st;
  if (!dtype_ok(dt)) return MM_ERR_ARG;
  if (nrec < 1 || nrec > MM_MAX_RECORD_SETS) return MM_ERR_ARG;
  if (!recs || !M) return MM_ERR_NULL;
  for (int q = 0; q < nrec; ++q)
    if (!recs[q]) return MM_ERR_NULL;
  if (z0 < 0 || z0 > z1 || z1 > grid->n[2]) return MM_ERR_ARG;
  const GridDev g = to_dev(grid);
  if (is2d(grid) || order != 2 || !tsc_run_records(g)) return MM_ERR_UNSUPPORTED;
  return hip_status(launch_gather_run(g, recs, nrec, accumulate, M, (hipStream_t)stream, canonical != 0,
                                      dt == MM_F32, z0, z1));
}

mm_status mm_deposit_moments(const mm_grid* grid, int order, mm_dtype dt, int64_t np, const void* pos, const void* Q,
                             int nq, const int32_t* bin_start, const int32_t* perm, int accumulate, void* m, void* ws,
                             size_t* ws_bytes, mm_stream_t stream) {
  if (!ws_bytes) return MM_ERR_NULL;
  int64_t nnodes = 0;
  mm_status st = check_grid(grid, order, &nnodes);
  if (st != MM_OK) return st;
  if (!dtype_ok(dt)) return MM_ERR_ARG;
  if (nq < 1 || nq > 16) return MM_ERR_ARG;
  if (is2d(grid)) return MM_ERR_UNSUPPORTED;
  if (np < 0) return MM_ERR_ARG;
  if (np >= kMaxI32) return MM_ERR_UNSUPPORTED;
  if (!m) return MM_ERR_NULL;
  if (np > 0 && (!pos || !Q || !bin_start || !perm)) return MM_ERR_NULL;
  const bool f32 = dt == MM_F32;
  const size_t need = np > 0 ? moment_record_bytes(order, nq, nnodes) : 0;
  if (!ws) {
    *ws_bytes = need;
    return MM_OK;
  }
  if (*ws_bytes < need) return MM_ERR_WORKSPACE;
  if (need > 0 && ((uintptr_t)ws & 15) != 0) return MM_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (np == 0) {
    if (accumulate) return MM_OK;
    return hip_status(launch_fill_zero(m, (size_t)nnodes * nq, f32, s));
  }
  return hip_status(launch_moments(to_dev(grid), order, f32, pos, Q, nq, bin_start, perm, (int)np, accumulate, m, ws,
                                   s, dt == MM_MIX));
}

mm_status mm_stencil_matvec(const mm_grid* grid, int order, mm_dtype dt, int tensorial, int canonical, const void* M,
                            const void* x, void* y, mm_stream_t stream) {
  int64_t nnodes = 0;
  mm_status st = check_grid(grid, order, &nnodes);
  if (st != MM_OK) return st;
  if (!dtype_ok(dt)) return MM_ERR_ARG;
  if (!M || !x || !y) return MM_ERR_NULL;
  if (is2d(grid)) return MM_ERR_UNSUPPORTED;
  if (x == y) return MM_ERR_ARG;
  return hip_status(launch_stencil_matvec(to_dev(grid), order, dt == MM_F32, tensorial != 0, canonical != 0, M, x, y,
                                          (hipStream_t)stream));
}

mm_status mm_probe_mfma_f64(int nblocks, int iters, double* out, mm_stream_t stream) {
  if (!out) return MM_ERR_NULL;
  if (nblocks <= 0 || nblocks > (1 << 20) || iters <= 0) return MM_ERR_ARG;
  return hip_status(launch_probe_mfma_f64(nblocks, iters, out, (hipStream_t)stream));
}

const char* mm_status_string(mm_status s) {
  switch (s) {
    case MM_OK: return "ok";
    case MM_ERR_NULL: return "a required pointer is NULL";
    case MM_ERR_ARG: return "argument out of range (order, dtype, grid, sigma/beta, algo or alignment)";
    case MM_ERR_UNSUPPORTED:
      return "unsupported: particle or node count at or above 2^31, or a combination of dtype, algorithm, "
             "field placement and grid dimension that the library does not implement";
    case MM_ERR_WORKSPACE: return "workspace smaller than required";
    case MM_ERR_HIP: return "HIP launch or runtime error";
    case MM_ERR_SCRATCH:
      return "the records of this workload exceed the fixed device scratch of the allocation-free entry point "
             "(MM_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

const char* mm_version(void) { return "mm 0.1 gfx950"; }

}  // extern "C"
