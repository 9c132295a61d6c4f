// First-order (CIC) fp64 per-bin contraction on v_mfma_f64_4x4x4_4b, phase 1
// of the two-phase assembly.
//
// Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for Implicit
// Particle-In-Cell Methods": every particle of a CIC cell touches the same
// 8 corner nodes (Sec. 2.3), so the cell's local matrix is
//   Mhat^c_ab = sum_p t_p^c W_pa W_pb                       (Sec. 3.1, Eq. 15)
// accumulated over batches of K_t particles (Sec. 3.2); the lower off-diagonal
// quadrant is skipped by the spatial symmetry Mhat_ab = Mhat_ba (Table 1).
//
// gfx950 mapping. One wave owns a group of four consecutive bins and gives
// each bin one of the four 4x4x4 blocks of the instruction, so the block
// results are final (no cross-block reduction). The 8 support rows split by
// the z corner into two halves; per component three instructions form the
// quadrants Q00, Q01, Q11 for four particles of each of the four bins (K_t = 4).
// Per 16 particles: 27 instructions (ECSIM) or 3 (scalar).
//
//  * Particle preparation runs one particle per lane (16 per bin per chunk):
//    the support weights W_a (Eq. 12) and the coefficients t^c = sigma w alpha^c
//    are computed once and staged in LDS, W interleaved so that the two rows a
//    lane feeds (r and 4 + r) are one 16-byte read, and laid out so that
//    staging stores and round loads meet no LDS bank conflict.
//  * The particle data of the next two chunks, and the permutation entries of
//    the two after those, are in flight while the current chunk is contracted
//    (the loads are unconditional, so that the compiler's waits count them
//    exactly). With 9 KB of LDS and about 144 registers per wave, 12 waves
//    fit on a CU; the deeper prefetch beats 16 waves with one chunk in flight
//    (the same at 64 particles per cell, 15% faster at 125).
//  * A finished group stages its packed upper-triangle records in LDS, two
//    bins at a time, and writes them with 16-byte stores (the records of
//    consecutive bins are contiguous).
//  * One launch may contract several species (each with its own arrays,
//    binning and beta): a group's accumulators run on from one species'
//    particles to the next, so their records are written once, summed.
//  * The particle arrays may have any element stride (ST), as when each
//    particle is one record of its position, weight and field: out of cell
//    order a particle then costs one random cache line instead of one per
//    array.
#include "mm_contract.h"

namespace mmk {

namespace {

constexpr int NB = 4;          // bins per wave group (= 4x4x4 blocks)
constexpr int CH = 16;         // particles per bin per chunk
constexpr int SW = 8;          // staged doubles per particle for W
constexpr int NPAIR = 36;      // packed upper triangle of 8 x 8

constexpr int WREG = 64 * SW + NB * SW;  // W region: SW per slot plus 64 bytes per bin (w_unit)

template <int NC>
struct Cfg {
  static constexpr int ST = NC == 9 ? 10 : 2;                 // staged doubles per particle for t
  static constexpr int STAGE = WREG + 64 * ST + 8;             // doubles of particle staging (t_base)
  static constexpr int FIELD = NB * 8 * 3;                     // grid field at the group's support nodes
  static constexpr int REC = 2 * NPAIR * NC;                   // records of two bins (staged in halves)
  static constexpr int SMEM = STAGE > REC ? STAGE : REC;
  static constexpr int SMEM_GB = STAGE + FIELD > REC ? STAGE + FIELD : REC;  // field on the grid
};

// A group is bins 4g .. 4g+3. Prep lane l serves bin 4g + (l >> 4): `s` and
// `n` are that bin's start in perm and particle count; `maxn` is the largest
// count of the group (wave-uniform).
struct Group {
  int s, n;
  int maxn;
  int nchunks;
};

// Split-K form (SK): the group is the single bin g, and every lane serves it.
template <bool SK>
__device__ __forceinline__ Group load_group(const int32_t* __restrict__ bin_start, int g, int nbins, int np,
                                            int lane) {
  Group G;
  const int bin = SK ? g : NB * g + (lane >> 4);
  int s = 0, e = 0;
  if (bin < nbins) {
    s = bin_start[bin];
    e = bin_start[bin + 1];
    s = s < 0 ? 0 : (s > np ? np : s);
    e = e < s ? s : (e > np ? np : e);
  }
  G.s = s;
  G.n = e - s;
  int m = __builtin_amdgcn_readlane(G.n, 0);
  m = max(m, __builtin_amdgcn_readlane(G.n, 16));
  m = max(m, __builtin_amdgcn_readlane(G.n, 32));
  m = max(m, __builtin_amdgcn_readlane(G.n, 48));
  G.maxn = m;
  // an empty group still writes zero records; SK chunks hold 4 CH particles of its bin
  G.nchunks = m > 0 ? (m + (SK ? 4 * CH : CH) - 1) / (SK ? 4 * CH : CH) : 1;
  return G;
}

// Permutation entry that prep lane `lane` loads for chunk j of group G. The
// load is unconditional (np > 0); `ok` says whether the entry exists, and the
// choice is made only where the value is used, so that no wait for the load
// is forced early.
struct PermRef {
  int v;
  bool ok;
};
template <bool SK>
__device__ __forceinline__ PermRef chunk_perm(const int32_t* __restrict__ perm, const Group& G, int j, int lane) {
  const int q = SK ? j * 4 * CH + lane : j * CH + (lane & 15);
  PermRef r;
  r.ok = q < G.n;
  r.v = perm[r.ok ? G.s + q : 0];
  return r;
}
__device__ __forceinline__ int perm_index(const PermRef& r) { return r.ok ? r.v : -1; }

struct Raw {
  double x, y, z, w, bx, by, bz;
  bool valid;
};

// Element strides of the particle arrays (used when the kernel's ST is set).
struct Strides {
  int64_t ps, wst, bst;
};

// The species contracted by one launch: each bin's records sum the particles
// of every species in it, each with its own arrays, binning and beta.
template <typename PT>
struct SpeciesSet {
  const PT* pos[MAX_SPECIES];
  const double* w[MAX_SPECIES];
  const PT* B[MAX_SPECIES];  // per-particle field (NULL when scalar or on the grid)
  const int32_t* bin_start[MAX_SPECIES];
  const int32_t* perm[MAX_SPECIES];
  double beta[MAX_SPECIES];
  int64_t ps[MAX_SPECIES], wst[MAX_SPECIES], bst[MAX_SPECIES];
  int np[MAX_SPECIES];
  int n;
};

// GB: the field is on the grid (gathered in stage), not per particle.
// PT: type of the stored positions and field (fp64, or fp32 read into fp64).
// ST: particle values st.ps, st.wst and st.bst elements apart (say records of
// several values per particle) instead of the dense 3, 1 and 3.
template <typename PT, int NC, bool GB, bool ST>
__device__ __forceinline__ Raw load_raw(const PT* __restrict__ pos, const double* __restrict__ w,
                                        const PT* __restrict__ Bf, int p, int np, const Strides& st) {
  // unconditional loads (particle 0 stands in for a lane without a particle;
  // np > 0 here) keep the number of loads in flight the same on every path
  Raw r;
  r.valid = (unsigned)p < (unsigned)np;
  const size_t q = r.valid ? (size_t)p : 0;
  const size_t qp = ST ? st.ps * q : 3 * q, qw = ST ? st.wst * q : q, qb = ST ? st.bst * q : 3 * q;
  r.x = pos[qp];
  r.y = pos[qp + 1];
  r.z = pos[qp + 2];
  r.w = w[qw];
  if (NC == 9 && !GB) {
    r.bx = Bf[qb];
    r.by = Bf[qb + 1];
    r.bz = Bf[qb + 2];
  } else {
    r.bx = r.by = r.bz = 0.0;
  }
  return r;
}

// LDS layout of the staged particles, chosen so that neither the staging
// stores (lane = slot) nor the operand loads of a round (lanes = 4 bins x 4
// rows, each group of 16 lanes served together) meet two lanes on one bank.
// W: slot s holds the 16-byte units (W_r, W_{4+r}), r = 0..3; each bin's 16
// slots start 64 bytes further on, and unit r sits at r ^ ((s >> 2) & 3).
__device__ __forceinline__ int w_unit(int s, int r) { return (s + ((s >> 4) & 3)) * (SW / 2) + (r ^ ((s >> 2) & 3)); }
// t: ST doubles per slot after the W region, and 16 bytes more per bin.
template <int NC>
__device__ __forceinline__ int t_base(int s) { return WREG + s * Cfg<NC>::ST + ((s >> 4) & 3) * 2; }

// Weights and coefficients of the lane's particle into LDS slot `lane` (zeros
// for a lane without a particle). With GB the field at the particle is
// gathered from sB, the grid field at the 8 support nodes of each bin of the
// group (node a = ax + 2 ay + 4 az, 3 components), with the particle's weights.
template <int NC, bool GB, bool SK>
__device__ __forceinline__ void stage(const Raw& r, const GridDev& g, double beta, double sigma, double* sm,
                                      const double* sB, int lane) {
  double wx[2] = {0, 0}, wy[2] = {0, 0}, wz[2] = {0, 0}, t[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) t[c] = 0.0;
  if (r.valid) {
    support_axis<double, 1, 0>((double)r.x, g, wx);
    support_axis<double, 1, 1>((double)r.y, g, wy);
    support_axis<double, 1, 2>((double)r.z, g, wz);
    const double f = sigma * r.w;
    double bx = r.bx, by = r.by, bz = r.bz;
    if (NC == 9 && GB) {
      const double* fb = sB + (SK ? 0 : (lane >> 4)) * 24;
      bx = by = bz = 0.0;
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const double W = (wx[a & 1] * wy[(a >> 1) & 1]) * wz[a >> 2];
        bx += W * fb[3 * a];
        by += W * fb[3 * a + 1];
        bz += W * fb[3 * a + 2];
      }
    }
    if (NC == 9)
      response<double>(bx, by, bz, beta, f, t);
    else
      t[0] = f;
  }
  double2* su = reinterpret_cast<double2*>(sm);
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const double wxy = wx[r4 & 1] * wy[r4 >> 1];
    double2 v;
    v.x = wxy * wz[0];
    v.y = wxy * wz[1];
    su[w_unit(lane, r4)] = v;
  }
  double* st = sm + t_base<NC>(lane);
  if (NC == 9) {
#pragma unroll
    for (int c = 0; c < 8; c += 2) *reinterpret_cast<double2*>(st + c) = double2{t[c], t[c + 1]};
    st[8] = t[NC - 1];
  } else {
    st[0] = t[0];
  }
}

template <int NC>
struct Acc {
  double q[NC][3];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int c = 0; c < NC; ++c) q[c][0] = q[c][1] = q[c][2] = 0.0;
  }
};

}  // namespace

// SK (split K, for grids of few bins): one bin per wave, the four blocks of
// the instruction taking different particles of it (16 per block and chunk);
// their four partial matrices are summed across lanes before the record is
// written. Four times as many waves, for the same matrix work.
template <typename PT, int NC, bool GB, bool ST, bool SK>
__global__ __launch_bounds__(64) void k_cic64(GridDev g, const SpeciesSet<PT> S, const PT* __restrict__ Bgrid,
                                              int nbins, double sigma, double* __restrict__ rec) {
  __shared__ __attribute__((aligned(16))) double sm[GB ? Cfg<NC>::SMEM_GB : Cfg<NC>::SMEM];
  const int lane = threadIdx.x;
  const int ngroups = SK ? nbins : (nbins + NB - 1) / NB;
  const int grp = blockIdx.x;
  if (grp >= ngroups) return;
  double* sB = sm + Cfg<NC>::STAGE;
  if (GB && lane < (SK ? 8 : NB * 8)) {
    // Bf is the grid field [nnodes][3]: node a of bin 4 grp + (lane >> 3) is
    // the bin's own node (its first support node) shifted by (ax, ay, az).
    const int bin = SK ? grp : NB * grp + (lane >> 3), a = lane & 7;
    double f0 = 0.0, f1 = 0.0, f2 = 0.0;
    if (bin < nbins) {
      const int kx = bin % g.n0, ky = (bin / g.n0) % g.n1, kz = bin / (g.n0 * g.n1);
      const int x = kx + (a & 1) < g.n0 ? kx + (a & 1) : 0;
      const int y = ky + ((a >> 1) & 1) < g.n1 ? ky + ((a >> 1) & 1) : 0;
      const int z = kz + (a >> 2) < g.n2 ? kz + (a >> 2) : 0;
      const PT* f = Bgrid + 3 * ((size_t)x + (size_t)g.n0 * ((size_t)y + (size_t)g.n1 * z));
      f0 = f[0];
      f1 = f[1];
      f2 = f[2];
    }
    sB[3 * lane] = f0;
    sB[3 * lane + 1] = f1;
    sB[3 * lane + 2] = f2;
  }
  if (GB) __syncthreads();

  // MFMA lane roles: particle k of the K_t batch, block (= bin) mb, row/column mr.
  const int mk = lane >> 4, mb = (lane >> 2) & 3, mr = lane & 3;
  const int wl = w_unit(CH * mb + mk, 0);  // = (17 mb + mk) * 4; round rd adds 16 rd, unit mr ^ rd
  const int tl = t_base<NC>(CH * mb + mk);

  Acc<NC> acc;
  acc.zero();
  for (int sp = 0; sp < S.n; ++sp) {  // the accumulators run on over the species
    const PT* __restrict__ pos = S.pos[sp];
    const double* __restrict__ w = S.w[sp];
    const PT* __restrict__ Bf = S.B[sp];
    const int32_t* __restrict__ perm = S.perm[sp];
    const int np = S.np[sp];
    if (np == 0) continue;
    const double beta = S.beta[sp];
    const Strides str{S.ps[sp], S.wst[sp], S.bst[sp]};
    const Group G = load_group<SK>(S.bin_start[sp], grp, nbins, np, lane);
    // Two chunks of particle data in flight ahead of the one being contracted.
    // The loop is unrolled by two so that each register set is reloaded right
    // after its chunk is staged (no copies, which would wait for the loads).
    // The loop starts two steps early (j = -2, -1) with only the loads, so
    // that every load is issued by the loop body in one order.
    Raw ra, rb;
    PermRef pa = chunk_perm<SK>(perm, G, 0, lane), pb = chunk_perm<SK>(perm, G, 1, lane);
    // resolved here, so that the loop is entered with no load in flight
    pa.v = perm_index(pa);
    pb.v = perm_index(pb);
    auto step = [&](Raw& r, PermRef& pr, int j) {
      if (j >= 0) {
        stage<NC, GB, SK>(r, g, beta, sigma, sm, sB, lane);
        __syncthreads();
      }
      r = load_raw<PT, NC, GB, ST>(pos, w, Bf, perm_index(pr), np, str);  // chunk j + 2
      pr = chunk_perm<SK>(perm, G, j + 4, lane);
      // rounds with particles: slot 16 mb + 4 rd + mk; with SK every block's
      // first 4 nr slots, so that a prefix of the chunk's 64 is covered
      const int left = G.maxn - j * (SK ? 4 * CH : CH);
      const int nr = j < 0 ? 0 : (left >= CH ? CH / 4 : (left > 0 ? (left + 3) / 4 : 0));
      for (int rd = 0; rd < nr; ++rd) {
        // slot = 16 mb + 4 rd + mk: w_unit(slot, mr) and t_base(slot) with the
        // lane's constant part taken out of the loop
        const double2 wv = reinterpret_cast<const double2*>(sm)[wl + 16 * rd + (mr ^ rd)];
        const double* st = sm + tl + 4 * Cfg<NC>::ST * rd;
        double tv[NC];
        if (NC == 9) {
#pragma unroll
          for (int c = 0; c < 8; c += 2) {
            const double2 tt = *reinterpret_cast<const double2*>(st + c);
            tv[c] = tt.x;
            tv[c + 1] = tt.y;
          }
          tv[NC - 1] = st[8];
        } else {
          tv[0] = st[0];
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const double alo = tv[c] * wv.x, ahi = tv[c] * wv.y;
          acc.q[c][0] = mfma_f64_4x4x4(alo, wv.x, acc.q[c][0]);
          acc.q[c][1] = mfma_f64_4x4x4(alo, wv.y, acc.q[c][1]);
          acc.q[c][2] = mfma_f64_4x4x4(ahi, wv.y, acc.q[c][2]);
        }
      }
      if (j >= 0) __syncthreads();
    };
    const int nsteps = (G.nchunks + 1) & ~1;  // an odd count ends with an empty chunk
    for (int j = -2; j < nsteps; j += 2) {
      step(ra, pa, j);
      step(rb, pb, j + 1);
    }
  }

  if (SK) {
    // the four blocks hold partial sums of the one bin: add them (lanes that
    // differ in the block bits 2 and 3) through LDS, one component at a time
    // (all at once in registers would cost a wave per SIMD), then write its
    // record
    const int db = (lane >> 2) & 3;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int k = 0; k < 3; ++k) sm[3 * lane + k] = acc.q[c][k];
      __syncthreads();
      if (db == 0) {
#pragma unroll
        for (int k = 0; k < 3; ++k)
          acc.q[c][k] = ((sm[3 * lane + k] + sm[3 * (lane + 4) + k]) + sm[3 * (lane + 8) + k]) + sm[3 * (lane + 12) + k];
      }
      __syncthreads();
    }
    const int di = lane >> 4, dj = lane & 3;
    const int p00 = di * 8 - (di * (di - 1)) / 2 + (dj - di);
    const int p01 = di * 8 - (di * (di - 1)) / 2 + (4 + dj - di);
    const int a1 = 4 + di;
    const int p11 = a1 * 8 - (a1 * (a1 - 1)) / 2 + (dj - di);
    if (db == 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (di <= dj) sm[p00 * NC + c] = acc.q[c][0];
        sm[p01 * NC + c] = acc.q[c][1];
        if (di <= dj) sm[p11 * NC + c] = acc.q[c][2];
      }
    }
    __syncthreads();
    double2* dst = reinterpret_cast<double2*>(rec + (size_t)grp * NPAIR * NC);
    const double2* src = reinterpret_cast<const double2*>(sm);
    for (int i = lane; i < NPAIR * NC / 2; i += 64) dst[i] = src[i];
    return;
  }

  // D_blk[i][j] sits in lane (i << 4) | (blk << 2) | j. Stage the packed
  // records rec[bin][pair(a, b)][c] (a <= b, pair(a, b) = 8a - a(a-1)/2 + b - a)
  // two bins at a time in LDS and write them with 16-byte stores (the records
  // of consecutive bins are contiguous).
  const int di = lane >> 4, db = (lane >> 2) & 3, dj = lane & 3;
  const int p00 = di * 8 - (di * (di - 1)) / 2 + (dj - di);
  const int p01 = di * 8 - (di * (di - 1)) / 2 + (4 + dj - di);
  const int a1 = 4 + di;
  const int p11 = a1 * 8 - (a1 * (a1 - 1)) / 2 + (dj - di);
  const int b0 = NB * grp;
  const int nvalid = nbins - b0 < NB ? nbins - b0 : NB;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((db >> 1) == half) {
      double* sr = sm + (db & 1) * NPAIR * NC;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (di <= dj) sr[p00 * NC + c] = acc.q[c][0];
        sr[p01 * NC + c] = acc.q[c][1];
        if (di <= dj) sr[p11 * NC + c] = acc.q[c][2];
      }
    }
    __syncthreads();
    const int nb = nvalid - 2 * half < 2 ? nvalid - 2 * half : 2;
    const int n2 = nb > 0 ? nb * NPAIR * NC / 2 : 0;  // NPAIR is even: whole 16-byte words
    double2* dst = reinterpret_cast<double2*>(rec + (size_t)(b0 + 2 * half) * NPAIR * NC);
    const double2* src = reinterpret_cast<const double2*>(sm);
    for (int i = lane; i < n2; i += 64) dst[i] = src[i];
    __syncthreads();
  }
}

template <typename PT, bool ST, bool SK>
static hipError_t cic64_t(const GridDev& g, const SpeciesSet<PT>& S, const PT* Bgrid, bool tensorial, double sigma,
                          double* rec, hipStream_t s) {
  const int nbins = g.n0 * g.n1 * g.n2;
  // one single-wave workgroup per group of four bins, or per bin (SK)
  const int ngroups = SK ? nbins : (nbins + NB - 1) / NB;
  if (Bgrid)
    hipLaunchKernelGGL((k_cic64<PT, 9, true, ST, SK>), dim3(ngroups), dim3(64), 0, s, g, S, Bgrid, nbins, sigma,
                       rec);
  else if (tensorial)
    hipLaunchKernelGGL((k_cic64<PT, 9, false, ST, SK>), dim3(ngroups), dim3(64), 0, s, g, S, Bgrid, nbins, sigma,
                       rec);
  else
    hipLaunchKernelGGL((k_cic64<PT, 1, false, ST, SK>), dim3(ngroups), dim3(64), 0, s, g, S, Bgrid, nbins, sigma,
                       rec);
  return hipGetLastError();
}

// Split K when groups of four bins would leave the SIMDs with fewer than
// three waves each and the bins hold at least a chunk of 16 particles on
// average (below that the chunks of 64 would be mostly empty).
static bool use_split_k(const GridDev& g, int64_t np_total) {
  const int64_t nbins = (int64_t)g.n0 * g.n1 * g.n2;
  return (nbins + NB - 1) / NB < 3072 && np_total >= 16 * nbins;
}

template <typename PT>
static hipError_t cic64_species(const GridDev& g, int ns, const Particles* P, const int32_t* const* bin_start,
                                const int32_t* const* perm, const double* beta, double sigma, double* rec,
                                hipStream_t s) {
  SpeciesSet<PT> S = {};
  S.n = ns;
  bool strided = false;
  for (int i = 0; i < ns; ++i) {
    S.pos[i] = (const PT*)P[i].pos;
    S.w[i] = (const double*)P[i].w;
    S.B[i] = (const PT*)P[i].B;
    S.bin_start[i] = bin_start[i];
    S.perm[i] = perm[i];
    S.beta[i] = beta[i];
    S.ps[i] = P[i].ps;
    S.wst[i] = P[i].wst;
    S.bst[i] = P[i].bst;
    S.np[i] = P[i].np;
    strided = strided || P[i].strided();
  }
  const PT* Bgrid = (const PT*)P[0].Bgrid;
  const bool tensorial = P[0].B != nullptr || Bgrid;
  int64_t np_total = 0;
  for (int i = 0; i < ns; ++i) np_total += P[i].np;
  const bool sk = use_split_k(g, np_total);
  if (strided) {
    // strided arrays: fp64 values with the field per particle
    if (Bgrid || !tensorial) return hipErrorInvalidValue;
    return sk ? cic64_t<PT, true, true>(g, S, Bgrid, true, sigma, rec, s)
              : cic64_t<PT, true, false>(g, S, Bgrid, true, sigma, rec, s);
  }
  return sk ? cic64_t<PT, false, true>(g, S, Bgrid, tensorial, sigma, rec, s)
            : cic64_t<PT, false, false>(g, S, Bgrid, tensorial, sigma, rec, s);
}

hipError_t launch_cic64_species(const GridDev& g, int ns, const Particles* P, const int32_t* const* bin_start,
                                const int32_t* const* perm, const double* beta, double sigma, double* rec,
                                hipStream_t s) {
  if (ns < 1 || ns > MAX_SPECIES) return hipErrorInvalidValue;
  // one kind of storage, field and records for the whole set
  for (int i = 1; i < ns; ++i)
    if (P[i].pos32 != P[0].pos32 || P[i].Bgrid != P[0].Bgrid || (P[i].B != nullptr) != (P[0].B != nullptr))
      return hipErrorInvalidValue;
  if (P[0].pos32) {
    for (int i = 0; i < ns; ++i)
      if (P[i].strided()) return hipErrorInvalidValue;
    return cic64_species<float>(g, ns, P, bin_start, perm, beta, sigma, rec, s);
  }
  return cic64_species<double>(g, ns, P, bin_start, perm, beta, sigma, rec, s);
}

hipError_t launch_cic64(const GridDev& g, const Particles& P, const int32_t* bin_start, const int32_t* perm,
                        double beta, double sigma, double* rec, hipStream_t s) {
  return launch_cic64_species(g, 1, &P, &bin_start, &perm, &beta, sigma, rec, s);
}

}  // namespace mmk
