// Deposit of run records (mm_run.h) into the stencil matrix, phase 2 of the
// second-order tensorial assembly (fp64, and fp32 with the field per
// particle) on grids whose x extent is a multiple of four.
//
// Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for Implicit
// Particle-In-Cell Methods", Sec. 3.4: every stencil entry M[g][o] is the sum
// of the local matrices of the support groups whose support holds both g and
// g + o. Here the local matrices arrive already summed over runs of four bins
// along x, so an entry gathers at most 2 runs along x (the runs overlap in two
// node columns) times the bins along y and z whose support holds both nodes:
// about 4.5 terms on average against 5.8 per-bin records. Each term is read
// from the run record of the bins (r, ky, kz) with the row node's position
// (X, Y, Z) in the run's union support.
//
// Blocks of three waves: the waves take rows i = 0, 1, 2 of the 3x3 block for
// the same 64 (node, offset) pairs, which share the y and z parts of their
// offsets and run over consecutive nodes x times the five x parts. A wave's
// term reads one short stretch of each of its three component planes of a
// run record (the (X, dX) of one (dY, dZ) row are consecutive entries,
// mm_run.h). The block stages its sums in LDS and stores whole 72-byte
// blocks: at M[g][o], where consecutive pairs fill consecutive entries, and,
// for the full stencil, at the mirrored entry M[g + d(o)][-o] (equal by the
// spatial symmetry of the matrix, Table 1 footnote), so every record value is
// read once. Terms are added in a fixed order (z, y, then the run that starts
// at or before the node's column, then the one before it), and several record
// sets (species) are added term by term in set order: results are
// deterministic. A launch covers the node rows of a range of planes (all of
// them, or one slab's worth when the assembly overlaps the two phases); the
// partition of the rows between launches does not change any sum.
#include "mm_contract.h"
#include "mm_run.h"

namespace mmk {

namespace {

static __constant__ run::Tables kRunG = run::make_tables();

constexpr int ZB = 1;  // node rows in plain order, y fastest: consecutive rows read adjacent slices of a record row

constexpr int PAIRS = 64;  // (node, offset) pairs per block, one per lane of each wave

template <typename T, bool CANON, int NR>
__global__ __launch_bounds__(3 * PAIRS) void k_gather_run(GridDev g, RecSet<T> recs, int accumulate,
                                                          T* __restrict__ M, int blocks_per_row, int rv0) {
  constexpr int NC = 9;
  constexpr int NOFF = 125;
  __shared__ T st[PAIRS * NC];
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int rl = blk / blocks_per_row;  // the launch's node rows start at row rv0 (plane rv0 / n1)
  const int rv = rv0 + rl;              // visit order of the node row
  const int lane = threadIdx.x & 63, i = threadIdx.x >> 6;
  const int per = g.n0 * 5;             // pairs per (dY, dZ) row of offsets
  const int p = (blk - rl * blocks_per_row) * PAIRS + lane;
  const int nfull = g.n2 / ZB;
  const int inb = g.n1 * ZB;
  int gy, gz;
  if (rv < nfull * inb) {
    const int zb = rv / inb, rem = rv - zb * inb;
    gy = rem / ZB;
    gz = zb * ZB + (rem - gy * ZB);
  } else {
    const int zl = g.n2 - nfull * ZB, rem = rv - nfull * inb;
    gy = rem / zl;
    gz = nfull * ZB + (rem - gy * zl);
  }
  const int oyz = run::ROW0 + p / per;
  const int rem = p - (oyz - run::ROW0) * per;
  const int gx = rem / 5;
  const int oxi = rem - gx * 5;
  const int o = oxi + 5 * oyz;
  // pairs past the row's end, and the other half of the (0, 0) row of offsets
  const bool active = p < run::NROW * per && o >= run::CENTRE;
  const int ox = oxi - 2, oy = oyz % 5 - 2, oz = oyz / 5 - 2;
  const int nruns = g.n0 / run::RUN;
  const bool first = oyz == run::ROW0;
  // the node's column in the run that starts at or before it (X in 0..3), and
  // in the run before that (X + 4; only 4 and 5 lie in its union)
  const int r1 = gx >> 2, x1 = gx & 3;
  const int r2 = r1 == 0 ? nruns - 1 : r1 - 1, x2 = x1 + 4;
  const bool use1 = active && ox >= run::dx_min(x1, first) && ox <= run::dx_max(x1);
  const bool use2 = active && x2 < run::UX && ox >= run::dx_min(x2, first) && ox <= run::dx_max(x2);
  const int c1 = kRunG.col_start[first][x1] + ox - run::dx_min(x1, first);
  const int c2 = x2 < run::UX ? kRunG.col_start[first][x2] + ox - run::dx_min(x2, first) : 0;

  T sum[3] = {T(0), T(0), T(0)};
  if (active) {
#pragma unroll
    for (int Z = 0; Z < 3; ++Z) {
      if (Z + oz < 0 || Z + oz > 2) continue;
      const int kz = gz - Z < 0 ? gz - Z + g.n2 : gz - Z;
#pragma unroll
      for (int Y = 0; Y < 3; ++Y) {
        if (Y + oy < 0 || Y + oy > 2) continue;
        const int ky = gy - Y < 0 ? gy - Y + g.n1 : gy - Y;
        const size_t rowrun = (size_t)nruns * ((size_t)ky + (size_t)g.n1 * kz);
        // slice 3 Z + Y of the record: its component planes of slice_stride values
        const int sl = 3 * Z + Y;
        const int stride = kRunG.slice_stride[sl];
        const int seg = kRunG.seg_start[sl * run::NROW + oyz - run::ROW0] + kRunG.slice_off[sl] + 3 * i * stride;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 0 ? !use1 : !use2) continue;
          const size_t off = (rowrun + (h == 0 ? r1 : r2)) * run::RUNREC + (size_t)(seg + (h == 0 ? c1 : c2));
#pragma unroll
          for (int q = 0; q < NR; ++q) {
            if (q == 0 || q < recs.n) {  // (uniform)
              const T* src = recs.r[q] + off;
#pragma unroll
              for (int j = 0; j < 3; ++j) sum[j] += src[j * stride];
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) st[lane * NC + 3 * i + j] = sum[j];
  __syncthreads();
  const int p0 = (blk - rl * blocks_per_row) * PAIRS;
  for (int idx = threadIdx.x; idx < PAIRS * NC; idx += 3 * PAIRS) {
    const int l = idx / NC, c = idx - l * NC;
    const int pp = p0 + l;
    const int qyz = run::ROW0 + pp / per;
    const int qrem = pp - (qyz - run::ROW0) * per;
    const int qx = qrem / 5, qxi = qrem - qx * 5;
    const int qo = qxi + 5 * qyz;
    if (pp >= run::NROW * per || qo < run::CENTRE) continue;
    const T v = st[idx];
    const size_t node = (size_t)qx + (size_t)g.n0 * ((size_t)gy + (size_t)g.n1 * gz);
    T* dst = CANON ? M + (node * 63 + (qo - run::CENTRE)) * NC + c : M + (node * NOFF + qo) * NC + c;
    *dst = accumulate ? *dst + v : v;
    if (!CANON && qo != run::CENTRE) {  // the mirrored entry M[g + d][-o]
      int mx = qx + qxi - 2, my = gy + qyz % 5 - 2, mz = gz + qyz / 5 - 2;
      mx = mx < 0 ? mx + g.n0 : (mx >= g.n0 ? mx - g.n0 : mx);
      my = my < 0 ? my + g.n1 : (my >= g.n1 ? my - g.n1 : my);
      mz = mz < 0 ? mz + g.n2 : (mz >= g.n2 ? mz - g.n2 : mz);
      T* mdst =
          M + (((size_t)mx + (size_t)g.n0 * ((size_t)my + (size_t)g.n1 * mz)) * NOFF + (NOFF - 1 - qo)) * NC + c;
      *mdst = accumulate ? *mdst + v : v;
    }
  }
}

template <typename T, bool CANON, int NR>
hipError_t go(const GridDev& g, const RecSet<T>& rs, int accumulate, void* M, hipStream_t s, int z0, int z1) {
  const size_t row_pairs = (size_t)run::NROW * 5 * g.n0;  // (dY, dZ) rows x dX x nodes of a node row
  const int bpr = (int)((row_pairs + PAIRS - 1) / PAIRS);
  const size_t blocks = (size_t)bpr * g.n1 * (z1 - z0);
  if (blocks > 0x7fffffffULL) return hipErrorInvalidValue;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((k_gather_run<T, CANON, NR>), dim3((unsigned)blocks), dim3(3 * PAIRS), 0, s, g, rs, accumulate,
                     (T*)M, bpr, z0 * g.n1);
  return hipGetLastError();
}

template <typename T>
hipError_t gather_run_t(const GridDev& g, const void* const* rec, int nrec, int accumulate, void* M, hipStream_t s,
                        bool canonical, int z0, int z1) {
  RecSet<T> rs{};
  for (int q = 0; q < nrec; ++q) rs.r[q] = (const T*)rec[q];
  rs.n = nrec;
  if (nrec > 1)
    return canonical ? go<T, true, MAX_REC>(g, rs, accumulate, M, s, z0, z1)
                     : go<T, false, MAX_REC>(g, rs, accumulate, M, s, z0, z1);
  return canonical ? go<T, true, 1>(g, rs, accumulate, M, s, z0, z1) : go<T, false, 1>(g, rs, accumulate, M, s, z0, z1);
}

}  // namespace

hipError_t launch_gather_run(const GridDev& g, const void* const* rec, int nrec, int accumulate, void* M,
                             hipStream_t s, bool canonical, bool f32, int z0, int z1) {
  if (nrec < 1 || nrec > MAX_REC || !tsc_run_records(g)) return hipErrorInvalidValue;
  if (z1 < 0) z1 = g.n2;
  if (z0 < 0 || z0 > z1 || z1 > g.n2) return hipErrorInvalidValue;
  return f32 ? gather_run_t<float>(g, rec, nrec, accumulate, M, s, canonical, z0, z1)
             : gather_run_t<double>(g, rec, nrec, accumulate, M, s, canonical, z0, z1);
}

}  // namespace mmk
