// Deposition of per-particle quantities on the matrix cores: m[g][k] =
// sum_p W_pg Q_p[k] (charge and current: 4 quantities; the implicit moment
// method: 10). Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for
// Implicit Particle-In-Cell Methods", Sec. 6: the same contraction serves any
// particle-to-grid scatter, one operand holding the quantities and the other
// the interpolation weights (Eq. 12); here the per-bin product is
//   Mhat_ak = sum_{p in bin} W_pa Q_pk      (bins as in Sec. 3.3)
// batched over K_t = 4 particles per block (Sec. 3.2), then gathered per node.
//
// gfx950 mapping, as for the mass matrix: one wave per group of four
// consecutive bins, one bin per 4x4x4 block of v_mfma_f64_4x4x4_4b. The N
// support rows (8 or 27, padded to 8 or 28) form NR/4 row blocks and the nq
// quantities (padded to a multiple of 4) KB column blocks: NR/4 * KB
// instructions per 16 particles. Accumulation is fp64 for both dtypes.
// Particle preparation runs one particle per lane into LDS; the records
// rec[bin][a][k] (fp64) are summed per node by k_gather_moments in a fixed
// order, so the result is deterministic.
#include "mm_contract.h"

namespace mmk {

namespace {

constexpr int NB = 4;   // bins per group
constexpr int CH = 16;  // particles per bin per chunk

template <int R>
struct MGeo {
  static constexpr int NS = R + 1;
  static constexpr int N = NS * NS * NS;   // support nodes
  static constexpr int NR = (N + 3) / 4 * 4;  // rows padded to blocks of 4
  // staged weights per particle: the 27 products at order 1 would be 8, the
  // 3 x 3 one-dimensional weights at order 2 (products formed in the rounds)
  static constexpr int WS = R == 2 ? 9 : NR;
};

// LDS slots: W per slot with 32 bytes more per bin, then Q.
template <int R>
__device__ __forceinline__ int w_base(int s) { return s * MGeo<R>::WS + (s >> 4) * 4; }
template <int R, int KB>
__device__ __forceinline__ int q_base(int s) {
  return 64 * MGeo<R>::WS + NB * 4 + s * (4 * KB) + (s >> 4) * 4;
}

// Data of the particle a lane prepares: position and quantities.
template <typename T, int KB>
struct MRaw {
  T x, y, z;
  T q[4 * KB];
  bool valid;
};

template <typename T, int KB, typename PT>
__device__ __forceinline__ MRaw<T, KB> load_mraw(const PT* __restrict__ pos, const T* __restrict__ Q, int nq, int p,
                                                 int np) {
  MRaw<T, KB> r;
  r.valid = (unsigned)p < (unsigned)np;
  r.x = r.y = r.z = T(0);
#pragma unroll
  for (int k = 0; k < 4 * KB; ++k) r.q[k] = T(0);
  if (r.valid) {
    r.x = (T)pos[3 * (size_t)p];
    r.y = (T)pos[3 * (size_t)p + 1];
    r.z = (T)pos[3 * (size_t)p + 2];
#pragma unroll
    for (int k = 0; k < 4 * KB; ++k)
      if (k < nq) r.q[k] = Q[(size_t)p * nq + k];
  }
  return r;
}

}  // namespace

// T: arithmetic of the weights and type of Q; PT: stored positions (T, or fp32 into fp64).
// The particle data of the next chunk, and the permutation entries of the
// chunk after it, are in flight while the current chunk is contracted.
template <typename T, int R, int KB, typename PT>
__global__ __launch_bounds__(64) void k_moments(GridDev g, const PT* __restrict__ pos, const T* __restrict__ Q, int nq,
                                                const int32_t* __restrict__ bin_start, const int32_t* __restrict__ perm,
                                                int np, int nbins, double* __restrict__ rec) {
  constexpr int NS = MGeo<R>::NS, N = MGeo<R>::N, NR = MGeo<R>::NR, NRB = NR / 4;
  constexpr int STAGE = 64 * MGeo<R>::WS + NB * 4 + 64 * 4 * KB + NB * 4;
  constexpr int RECS = NB * N * 4 * KB;  // the group's records, staged after the rounds
  constexpr int SMEM = STAGE > RECS ? STAGE : RECS;
  __shared__ __attribute__((aligned(16))) double sm[SMEM];
  const int lane = threadIdx.x;
  const int ngroups = (nbins + NB - 1) / NB;
  const int grp = xcd_chunk_remap(blockIdx.x, gridDim.x, 16);  // chunks of groups dealt round the XCDs
  if (grp >= ngroups) return;
  // prep lane l serves bin 4 grp + (l >> 4)
  const int bin_l = NB * grp + (lane >> 4);
  int s0 = 0, e0 = 0;
  if (bin_l < nbins) {
    s0 = bin_start[bin_l];
    e0 = bin_start[bin_l + 1];
    s0 = s0 < 0 ? 0 : (s0 > np ? np : s0);
    e0 = e0 < s0 ? s0 : (e0 > np ? np : e0);
  }
  const int n_l = e0 - s0;
  int maxn = __builtin_amdgcn_readlane(n_l, 0);
  maxn = max(maxn, __builtin_amdgcn_readlane(n_l, 16));
  maxn = max(maxn, __builtin_amdgcn_readlane(n_l, 32));
  maxn = max(maxn, __builtin_amdgcn_readlane(n_l, 48));
  const int nchunks = (maxn + CH - 1) / CH;

  const int mk = lane >> 4, mb = (lane >> 2) & 3, mr = lane & 3;
  // order 2: this lane's support rows a = 4 I + mr as indices of their x, y, z weights
  int ix[NRB], iy[NRB], iz[NRB];
#pragma unroll
  for (int I = 0; I < NRB; ++I) {
    const int a = 4 * I + mr;
    ix[I] = a % NS;
    iy[I] = NS + (a / NS) % NS;
    iz[I] = 2 * NS + a / (NS * NS);
  }
  double acc[NRB][KB];
#pragma unroll
  for (int I = 0; I < NRB; ++I)
#pragma unroll
    for (int J = 0; J < KB; ++J) acc[I][J] = 0.0;

  auto chunk_perm = [&](int j) {
    const int qi = j * CH + (lane & 15);
    return qi < n_l ? perm[s0 + qi] : -1;
  };
  MRaw<T, KB> raw = load_mraw<T, KB, PT>(pos, Q, nq, chunk_perm(0), np);
  int pnext = chunk_perm(1);
  for (int j = 0; j < nchunks; ++j) {
    // stage: one particle per lane (zeros for an empty lane)
    {
      T wx[3] = {T(0), T(0), T(0)}, wy[3] = {T(0), T(0), T(0)}, wz[3] = {T(0), T(0), T(0)};
      if (raw.valid) {
        support_axis<T, R, 0>((double)raw.x, g, wx);
        support_axis<T, R, 1>((double)raw.y, g, wy);
        support_axis<T, R, 2>((double)raw.z, g, wz);
      }
      double* sw = sm + w_base<R>(lane);
      if (R == 2) {
#pragma unroll
        for (int k = 0; k < NS; ++k) {
          sw[k] = (double)wx[k];
          sw[NS + k] = (double)wy[k];
          sw[2 * NS + k] = (double)wz[k];
        }
      } else {
#pragma unroll
        for (int a = 0; a < NR; ++a)
          sw[a] = a < N ? (double)((wx[a % NS] * wy[(a / NS) % NS]) * wz[a / (NS * NS)]) : 0.0;
      }
      double* sq = sm + q_base<R, KB>(lane);
#pragma unroll
      for (int k = 0; k < 4 * KB; ++k) sq[k] = (double)raw.q[k];
    }
    __syncthreads();
    raw = load_mraw<T, KB, PT>(pos, Q, nq, pnext, np);  // next chunk, in flight during the rounds
    pnext = chunk_perm(j + 2);

    const int left = maxn - j * CH;
    const int nr = left >= CH ? CH / 4 : (left + 3) / 4;
    for (int rd = 0; rd < nr; ++rd) {
      const int slot = CH * mb + 4 * rd + mk;
      const double* wv = sm + w_base<R>(slot);
      const double* qv = sm + q_base<R, KB>(slot);
      double qb[KB];
#pragma unroll
      for (int J = 0; J < KB; ++J) qb[J] = qv[4 * J + mr];
#pragma unroll
      for (int I = 0; I < NRB; ++I) {
        double a;
        if (R == 2)  // W_a = (wx wy) wz in the weights' own type, as staged at order 1
          a = 4 * I + mr < N ? (double)(((T)wv[ix[I]] * (T)wv[iy[I]]) * (T)wv[iz[I]]) : 0.0;
        else
          a = wv[4 * I + mr];
#pragma unroll
        for (int J = 0; J < KB; ++J) acc[I][J] = mfma_f64_4x4x4(a, qb[J], acc[I][J]);
      }
    }
    __syncthreads();
  }
  // D_blk[i][j] at lane (i << 4) | (blk << 2) | j: node row 4I + i, quantity 4J + j of bin 4 grp + blk.
  // The group's records rec[bin][a][k] are contiguous: stage them in LDS and
  // store them with consecutive lanes on consecutive values.
  const int di = lane >> 4, db = (lane >> 2) & 3, dj = lane & 3;
  const int b0 = NB * grp;
  const int nvalid = nbins - b0 < NB ? nbins - b0 : NB;
#pragma unroll
  for (int I = 0; I < NRB; ++I)
#pragma unroll
    for (int J = 0; J < KB; ++J) {
      const int a = 4 * I + di, k = 4 * J + dj;
      if (a < N && k < nq && db < nvalid) sm[(db * N + a) * nq + k] = acc[I][J];
    }
  __syncthreads();
  const int nval = nvalid * N * nq;
  double* dst = rec + (size_t)b0 * N * nq;
  for (int i = lane; i < nval; i += 64) dst[i] = sm[i];
}

// m[g][k] (=|+=) sum over the support offsets a of rec[bin g - a][a][k], in a
// fixed order. One thread per (node, quantity).
template <typename T, int R>
__global__ __launch_bounds__(256) void k_gather_moments(GridDev g, const double* __restrict__ rec, int nq,
                                                        int accumulate, T* __restrict__ m) {
  constexpr int NS = R + 1, N = NS * NS * NS;
  const size_t nn = (size_t)g.n0 * g.n1 * g.n2;
  const size_t t = (size_t)xcd_remap(blockIdx.x, gridDim.x) * blockDim.x + threadIdx.x;
  if (t >= nn * nq) return;
  const size_t node = t / nq;
  const int k = (int)(t - node * nq);
  const int gx = (int)(node % g.n0), gy = (int)((node / g.n0) % g.n1), gz = (int)(node / ((size_t)g.n0 * g.n1));
  double sum = 0.0;
#pragma unroll
  for (int a = 0; a < N; ++a) {
    const int ax = a % NS, ay = (a / NS) % NS, az = a / (NS * NS);
    const int bx = gx - ax < 0 ? gx - ax + g.n0 : gx - ax;
    const int by = gy - ay < 0 ? gy - ay + g.n1 : gy - ay;
    const int bz = gz - az < 0 ? gz - az + g.n2 : gz - az;
    const size_t b = (size_t)bx + (size_t)g.n0 * ((size_t)by + (size_t)g.n1 * bz);
    sum += rec[(b * N + a) * nq + k];
  }
  m[t] = accumulate ? (T)((double)m[t] + sum) : (T)sum;
}

size_t moment_record_bytes(int order, int nq, int64_t nbins) {
  const int n = (order + 1) * (order + 1) * (order + 1);
  return (size_t)nbins * n * nq * sizeof(double);
}

template <typename T, int R, typename PT>
static hipError_t moments_t(const GridDev& g, const void* pos, const void* Q, int nq, const int32_t* bin_start,
                            const int32_t* perm, int np, int accumulate, void* m, double* rec, hipStream_t s) {
  const int nbins = g.n0 * g.n1 * g.n2;
  const dim3 grid((unsigned)((nbins + NB - 1) / NB)), block(64);
  const int kb = (nq + 3) / 4;
  const PT* P = (const PT*)pos;
  const T* Qt = (const T*)Q;
  switch (kb) {
    case 1: hipLaunchKernelGGL((k_moments<T, R, 1, PT>), grid, block, 0, s, g, P, Qt, nq, bin_start, perm, np, nbins, rec); break;
    case 2: hipLaunchKernelGGL((k_moments<T, R, 2, PT>), grid, block, 0, s, g, P, Qt, nq, bin_start, perm, np, nbins, rec); break;
    case 3: hipLaunchKernelGGL((k_moments<T, R, 3, PT>), grid, block, 0, s, g, P, Qt, nq, bin_start, perm, np, nbins, rec); break;
    case 4: hipLaunchKernelGGL((k_moments<T, R, 4, PT>), grid, block, 0, s, g, P, Qt, nq, bin_start, perm, np, nbins, rec); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t nt = (size_t)nbins * nq;
  const size_t blocks = (nt + 255) / 256;
  if (blocks > 0x7fffffffULL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gather_moments<T, R>), dim3((unsigned)blocks), dim3(256), 0, s, g, (const double*)rec, nq,
                     accumulate, (T*)m);
  return hipGetLastError();
}

hipError_t launch_moments(const GridDev& g, int order, bool f32, const void* pos, const void* Q, int nq,
                          const int32_t* bin_start, const int32_t* perm, int np, int accumulate, void* m, void* rec,
                          hipStream_t s, bool pos32) {
  double* r = (double*)rec;
  if (f32)
    return order == 1 ? moments_t<float, 1, float>(g, pos, Q, nq, bin_start, perm, np, accumulate, m, r, s)
                      : moments_t<float, 2, float>(g, pos, Q, nq, bin_start, perm, np, accumulate, m, r, s);
  if (pos32)
    return order == 1 ? moments_t<double, 1, float>(g, pos, Q, nq, bin_start, perm, np, accumulate, m, r, s)
                      : moments_t<double, 2, float>(g, pos, Q, nq, bin_start, perm, np, accumulate, m, r, s);
  return order == 1 ? moments_t<double, 1, double>(g, pos, Q, nq, bin_start, perm, np, accumulate, m, r, s)
                    : moments_t<double, 2, double>(g, pos, Q, nq, bin_start, perm, np, accumulate, m, r, s);
}

}  // namespace mmk
