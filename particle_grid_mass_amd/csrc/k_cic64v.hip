// First-order (CIC) fp64 per-bin contraction on vector FMAs: the comparison
// kernel for the matrix-core contraction k_cic64 (same bins, same records,
// same deposit; MM_ALGO_VALU).
//
// Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for Implicit
// Particle-In-Cell Methods", Sec. 5 ("Kernel-level speedup") credits the
// tensor cores against a conventional kernel. On gfx950 the fp64 vector and
// fp64 matrix rates are equal, so the fair baseline for k_cic64 is the same
// binned contraction with the products formed by the vector unit:
//   Mhat^c_ab = sum_p t_p^c W_pa W_pb                       (Sec. 3.1, Eq. 15)
// for the 36 pairs a <= b of the 8 corner nodes (Sec. 2.3, Table 1 symmetry).
//
// Mapping. One wave owns a group of 16 consecutive bins; the four lanes of a
// bin split its 36 pairs, nine each, and keep their nine pairs' 9 (or 1)
// components in registers. Particles are prepared one per lane (4 per bin per
// chunk) as in the matrix-core kernels, but the staged values are the 36 pair
// products W_a W_b and the coefficients t^c. A step advances every bin by one
// particle: each lane reads its nine products and the nine coefficients from
// LDS and does 81 (or 9) fused multiply-adds, so a particle costs 324 FMAs for
// the 3x3 matrix, against 27 matrix instructions per 16 particles (432
// multiply-adds per particle, the diagonal blocks in full) in k_cic64. The
// next chunk's particle data is in flight during the steps. Each lane writes
// its nine pairs' record values, contiguous in rec[bin][pair][comp].
// On grids of few bins (SK) a wave owns 4 bins and each bin 16 lanes: four
// slices of four, each slice taking every fourth particle of the bin's chunks
// of 16, and the slices' sums are added across lanes before the record is
// written (four times the waves, the same FMAs per particle).
#include "mm_contract.h"

namespace mmk {

namespace {

constexpr int NB = 16;     // bins per wave group
constexpr int CH = 4;      // particles per bin per chunk (one per lane)
constexpr int NPAIR = 36;  // packed upper triangle of 8 x 8
constexpr int PPL = 9;     // pairs per lane (four lanes per bin)

template <int NC>
struct Cfg {
  static constexpr int PS = 10;                // staged doubles per quarter: nine products and a pad
  static constexpr int TS = NC == 9 ? 10 : 2;  // staged doubles of t per slot
  static constexpr int SLOT = 4 * PS + TS;     // doubles per staged particle
  static constexpr int SMEM = 64 * SLOT;
};

struct Group {
  int s, n;
  int maxn;
  int nchunks;
};

template <bool SK>
__device__ __forceinline__ Group load_group(const int32_t* __restrict__ bin_start, int g, int nbins, int np,
                                            int lane) {
  Group G;
  const int bin = SK ? 4 * g + (lane >> 4) : NB * g + (lane >> 2);
  int s = 0, e = 0;
  if (bin < nbins) {
    s = bin_start[bin];
    e = bin_start[bin + 1];
    s = s < 0 ? 0 : (s > np ? np : s);
    e = e < s ? s : (e > np ? np : e);
  }
  G.s = s;
  G.n = e - s;
  int m = G.n;
#pragma unroll
  for (int off = 4; off < 64; off <<= 1) m = max(m, __shfl_xor(m, off));
  G.maxn = __builtin_amdgcn_readfirstlane(m);
  G.nchunks = G.maxn > 0 ? (G.maxn + (SK ? 4 * CH : CH) - 1) / (SK ? 4 * CH : CH) : 1;
  return G;
}

template <bool SK>
__device__ __forceinline__ int chunk_perm(const int32_t* __restrict__ perm, const Group& G, int j, int lane) {
  const int q = SK ? j * 4 * CH + (lane & 15) : j * CH + (lane & 3);
  return q < G.n ? perm[G.s + q] : -1;
}

struct Raw {
  double x, y, z, w, bx, by, bz;
  bool valid;
};

template <typename PT, int NC>
__device__ __forceinline__ Raw load_raw(const PT* __restrict__ pos, const double* __restrict__ w,
                                        const PT* __restrict__ Bf, int p, int np) {
  Raw r{0, 0, 0, 0, 0, 0, 0, false};
  if ((unsigned)p < (unsigned)np) {
    r.valid = true;
    r.x = pos[3 * (size_t)p];
    r.y = pos[3 * (size_t)p + 1];
    r.z = pos[3 * (size_t)p + 2];
    r.w = w[p];
    if (NC == 9) {
      r.bx = Bf[3 * (size_t)p];
      r.by = Bf[3 * (size_t)p + 1];
      r.bz = Bf[3 * (size_t)p + 2];
    }
  }
  return r;
}

// The rows (a, b) of packed pair p of the 8 x 8 upper triangle.
constexpr int pair_a(int p) { return p < 8 ? 0 : p < 15 ? 1 : p < 21 ? 2 : p < 26 ? 3 : p < 30 ? 4 : p < 33 ? 5 : p < 35 ? 6 : 7; }
constexpr int pair_first(int a) { return a * 8 - (a * (a - 1)) / 2; }
constexpr int pair_b(int p) { return p - pair_first(pair_a(p)) + pair_a(p); }

template <int NC>
__device__ __forceinline__ void stage(const Raw& r, const GridDev& g, double beta, double sigma, double* sm,
                                      int lane) {
  double wx[2] = {0, 0}, wy[2] = {0, 0}, wz[2] = {0, 0}, t[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) t[c] = 0.0;
  if (r.valid) {
    support_axis<double, 1, 0>(r.x, g, wx);
    support_axis<double, 1, 1>(r.y, g, wy);
    support_axis<double, 1, 2>(r.z, g, wz);
    const double f = sigma * r.w;
    if (NC == 9)
      response<double>(r.bx, r.by, r.bz, beta, f, t);
    else
      t[0] = f;
  }
  double W[8];
#pragma unroll
  for (int a = 0; a < 8; ++a) W[a] = (wx[a & 1] * wy[(a >> 1) & 1]) * wz[a >> 2];
  double* s = sm + lane * Cfg<NC>::SLOT;
#pragma unroll
  for (int p = 0; p < NPAIR; ++p) s[(p / PPL) * Cfg<NC>::PS + p % PPL] = W[pair_a(p)] * W[pair_b(p)];
#pragma unroll
  for (int c = 0; c + 1 < NC; c += 2) *reinterpret_cast<double2*>(s + 4 * Cfg<NC>::PS + c) = double2{t[c], t[c + 1]};
  s[4 * Cfg<NC>::PS + NC - 1] = t[NC - 1];
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace

template <typename PT, int NC, bool SK>
__global__ __launch_bounds__(64) void k_cic64v(GridDev g, const PT* __restrict__ pos, const double* __restrict__ w,
                                               const PT* __restrict__ Bf, const int32_t* __restrict__ bin_start,
                                               const int32_t* __restrict__ perm, int np, int nbins, double beta,
                                               double sigma, double* __restrict__ rec) {
  __shared__ __attribute__((aligned(16))) double sm[Cfg<NC>::SMEM];
  const int lane = threadIdx.x;
  constexpr int NBW = SK ? 4 : NB;  // bins per wave
  const int ngroups = (nbins + NBW - 1) / NBW;
  const int grp = xcd_chunk_remap(blockIdx.x, gridDim.x, 16);  // chunks of groups dealt round the XCDs
  if (grp >= ngroups) return;
  const Group G = load_group<SK>(bin_start, grp, nbins, np, lane);
  // the lane's bin in the group, slice of the bin's particles (SK) and quarter of its pairs
  const int bl = SK ? lane >> 4 : lane >> 2, sl = SK ? (lane >> 2) & 3 : 0, q = lane & 3;

  double acc[PPL][NC];
#pragma unroll
  for (int k = 0; k < PPL; ++k)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[k][c] = 0.0;

  Raw raw = load_raw<PT, NC>(pos, w, Bf, chunk_perm<SK>(perm, G, 0, lane), np);
  int pnext = chunk_perm<SK>(perm, G, 1, lane);
  for (int j = 0; j < G.nchunks; ++j) {
    stage<NC>(raw, g, beta, sigma, sm, lane);
    wave_sync();
    raw = load_raw<PT, NC>(pos, w, Bf, pnext, np);  // next chunk, in flight during the steps
    pnext = chunk_perm<SK>(perm, G, j + 2, lane);
    // steps with particles; with SK step rd takes particle 4 rd + sl of the bin's 16
    const int left = G.maxn - j * (SK ? 4 * CH : CH);
    const int nr = SK ? (left >= 4 * CH ? CH : (left + 3) / 4) : (left >= CH ? CH : left);
    for (int rd = 0; rd < nr; ++rd) {
      const double* s = sm + (SK ? 4 * CH * bl + 4 * rd + sl : CH * bl + rd) * Cfg<NC>::SLOT;
      const double* sp = s + q * Cfg<NC>::PS;
      double ww[PPL + 1], t[NC];
#pragma unroll
      for (int k = 0; k < PPL + 1; k += 2) {
        const double2 v = *reinterpret_cast<const double2*>(sp + k);
        ww[k] = v.x;
        ww[k + 1] = v.y;
      }
#pragma unroll
      for (int c = 0; c + 1 < NC; c += 2) {
        const double2 v = *reinterpret_cast<const double2*>(s + 4 * Cfg<NC>::PS + c);
        t[c] = v.x;
        t[c + 1] = v.y;
      }
      t[NC - 1] = s[4 * Cfg<NC>::PS + NC - 1];
#pragma unroll
      for (int k = 0; k < PPL; ++k)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[k][c] = fma(t[c], ww[k], acc[k][c]);
    }
    wave_sync();
  }
  const int bin = NBW * grp + bl;
  if (SK) {
    // add the four slices' sums through LDS, one pair at a time (all at once
    // in registers would take a hundred more), in slice order
    double* dst = rec + ((size_t)bin * NPAIR + PPL * q) * NC;
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
#pragma unroll
      for (int c = 0; c < NC; ++c) sm[lane * NC + c] = acc[k][c];
      wave_sync();
      if (sl == 0 && bin < nbins) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
          dst[k * NC + c] = ((sm[lane * NC + c] + sm[(lane + 4) * NC + c]) + sm[(lane + 8) * NC + c]) +
                            sm[(lane + 12) * NC + c];
      }
      wave_sync();
    }
    return;
  }
  if (bin < nbins) {
    double* dst = rec + ((size_t)bin * NPAIR + PPL * q) * NC;
#pragma unroll
    for (int k = 0; k < PPL; ++k)
#pragma unroll
      for (int c = 0; c < NC; ++c) dst[k * NC + c] = acc[k][c];
  }
}

template <typename PT, bool SK>
static hipError_t cic64v_launch(const GridDev& g, const Particles& P, const int32_t* bin_start, const int32_t* perm,
                                double beta, double sigma, double* rec, hipStream_t s) {
  const int nbins = g.n0 * g.n1 * g.n2;
  const int ngroups = (nbins + (SK ? 4 : NB) - 1) / (SK ? 4 : NB);
  if (P.B)
    hipLaunchKernelGGL((k_cic64v<PT, 9, SK>), dim3(ngroups), dim3(64), 0, s, g, (const PT*)P.pos,
                       (const double*)P.w, (const PT*)P.B, bin_start, perm, P.np, nbins, beta, sigma, rec);
  else
    hipLaunchKernelGGL((k_cic64v<PT, 1, SK>), dim3(ngroups), dim3(64), 0, s, g, (const PT*)P.pos,
                       (const double*)P.w, (const PT*)nullptr, bin_start, perm, P.np, nbins, beta, sigma, rec);
  return hipGetLastError();
}

// Split K when groups of 16 bins would leave the SIMDs with fewer than two
// waves each (the kernel runs two per SIMD) and the bins average at least 16
// particles.
template <typename PT>
static hipError_t cic64v_t(const GridDev& g, const Particles& P, const int32_t* bin_start, const int32_t* perm,
                           double beta, double sigma, double* rec, hipStream_t s) {
  const int64_t nbins = (int64_t)g.n0 * g.n1 * g.n2;
  const bool sk = (nbins + NB - 1) / NB < 2048 && (int64_t)P.np >= 16 * nbins;
  return sk ? cic64v_launch<PT, true>(g, P, bin_start, perm, beta, sigma, rec, s)
            : cic64v_launch<PT, false>(g, P, bin_start, perm, beta, sigma, rec, s);
}

hipError_t launch_cic64_valu(const GridDev& g, const Particles& P, const int32_t* bin_start, const int32_t* perm,
                             double beta, double sigma, double* rec, hipStream_t s) {
  if (P.Bgrid) return hipErrorInvalidValue;  // field per particle
  return P.pos32 ? cic64v_t<float>(g, P, bin_start, perm, beta, sigma, rec, s)
                 : cic64v_t<double>(g, P, bin_start, perm, beta, sigma, rec, s);
}

}  // namespace mmk
