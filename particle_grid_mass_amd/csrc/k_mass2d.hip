// The 2D mass matrix (a grid with one node plane: z ignored), for the 2D runs
// Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for Implicit
// Particle-In-Cell Methods", report in Sec. 5 ("End-to-end impact"). The
// support is the (R+1)^2 nodes of the plane, so per bin
//   Mhat^c_ab = sum_p t_p^c W_pa W_pb          (Sec. 3.1, Eq. 15)
// is a 4x4 (CIC) or 9x9 (TSC, padded to 12) matrix per component, and the
// stencil has (2R+1)^2 offsets, offset = (dx+R) + (2R+1)(dy+R).
//
// gfx950 mapping as for 3D: one wave per group of four bins, one bin per
// 4x4x4 block of v_mfma_f64_4x4x4_4b, K_t = 4 particles per block; the upper
// row blocks (I <= J) only: 1 (CIC) or 6 (TSC) instructions per component per
// 16 particles. fp64 arithmetic (fp32 stored positions and fields are widened
// in registers). Records rec[bin][pair(a,b)][comp] (a <= b) go to k_gather2d,
// which sums them per node in a fixed order.
#include "mm_contract.h"

namespace mmk {

namespace {

constexpr int NB = 4;   // bins per group
constexpr int CH = 16;  // particles per bin per chunk

template <int R>
struct G2 {
  static constexpr int NS = R + 1;
  static constexpr int N = NS * NS;              // support nodes
  static constexpr int NR = (N + 3) / 4 * 4;     // padded to row blocks of 4
  static constexpr int NRB = NR / 4;
  static constexpr int NBP = NRB * (NRB + 1) / 2;  // upper blocks
  static constexpr int NPAIR = N * (N + 1) / 2;
  static constexpr int NO = 2 * R + 1;
  static constexpr int NOFF = NO * NO;
};

}  // namespace

template <typename PT, int R, int NC>
__global__ __launch_bounds__(64) void k_mass2d(GridDev g, const PT* __restrict__ pos, const double* __restrict__ w,
                                               const PT* __restrict__ Bf, const int32_t* __restrict__ bin_start,
                                               const int32_t* __restrict__ perm, int np, int nbins, double beta,
                                               double sigma, double* __restrict__ rec) {
  using G = G2<R>;
  constexpr int NS = G::NS, N = G::N, NR = G::NR, NRB = G::NRB, NBP = G::NBP;
  constexpr int TS = NC == 9 ? 10 : 2;                 // staged doubles per slot for t
  constexpr int WOFF = 0, TOFF = 64 * NR + NB * 4;     // W and t regions (16 bytes more per bin)
  __shared__ __attribute__((aligned(16))) double sm[TOFF + 64 * TS + NB * 2];
  const int lane = threadIdx.x;
  const int ngroups = (nbins + NB - 1) / NB;
  const int grp = xcd_chunk_remap(blockIdx.x, gridDim.x, 16);  // chunks of groups dealt round the XCDs
  if (grp >= ngroups) return;
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
  auto wb = [](int s) { return WOFF + s * NR + (s >> 4) * 4; };
  auto tb = [](int s) { return TOFF + s * TS + (s >> 4) * 2; };

  const int mk = lane >> 4, mb = (lane >> 2) & 3, mr = lane & 3;
  double acc[NC][NBP];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int k = 0; k < NBP; ++k) acc[c][k] = 0.0;

  // The particle data of the next chunk, and the permutation entries of the
  // chunk after it, are in flight while the current chunk is contracted.
  struct Raw2 {
    double x, y, w, bx, by, bz;
    bool valid;
  };
  auto chunk_perm = [&](int j) {
    const int qi = j * CH + (lane & 15);
    return qi < n_l ? perm[s0 + qi] : -1;
  };
  auto load_raw2 = [&](int p) {
    Raw2 r{0, 0, 0, 0, 0, 0, false};
    if ((unsigned)p < (unsigned)np) {
      r.valid = true;
      r.x = (double)pos[3 * (size_t)p];
      r.y = (double)pos[3 * (size_t)p + 1];
      r.w = w[p];
      if (NC == 9) {
        r.bx = (double)Bf[3 * (size_t)p];
        r.by = (double)Bf[3 * (size_t)p + 1];
        r.bz = (double)Bf[3 * (size_t)p + 2];
      }
    }
    return r;
  };
  Raw2 raw = load_raw2(chunk_perm(0));
  int pnext = chunk_perm(1);
  for (int j = 0; j < nchunks; ++j) {
    // stage one particle per lane: W_a (a = ax + NS ay) and t^c = sigma w alpha^c
    double wx[3] = {0, 0, 0}, wy[3] = {0, 0, 0}, t[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) t[c] = 0.0;
    if (raw.valid) {
      support_axis<double, R, 0>((double)raw.x, g, wx);
      support_axis<double, R, 1>((double)raw.y, g, wy);
      const double f = sigma * raw.w;
      if (NC == 9)
        response<double>(raw.bx, raw.by, raw.bz, beta, f, t);
      else
        t[0] = f;
    }
    double* sw = sm + wb(lane);
#pragma unroll
    for (int a = 0; a < NR; ++a) sw[a] = a < N ? wx[a % NS] * wy[a / NS] : 0.0;
    double* st = sm + tb(lane);
#pragma unroll
    for (int c = 0; c < NC; ++c) st[c] = t[c];
    __syncthreads();
    raw = load_raw2(pnext);  // next chunk, in flight during the rounds
    pnext = chunk_perm(j + 2);

    const int left = maxn - j * CH;
    const int nr = left >= CH ? CH / 4 : (left + 3) / 4;
    for (int rd = 0; rd < nr; ++rd) {
      const int slot = CH * mb + 4 * rd + mk;
      const double* wv = sm + wb(slot);
      const double* tv = sm + tb(slot);
      double wr[NRB];
#pragma unroll
      for (int I = 0; I < NRB; ++I) wr[I] = wv[4 * I + mr];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const double tc = tv[c];
        int k = 0;
#pragma unroll
        for (int I = 0; I < NRB; ++I) {
          const double a = tc * wr[I];
#pragma unroll
          for (int J = I; J < NRB; ++J, ++k) acc[c][k] = mfma_f64_4x4x4(a, wr[J], acc[c][k]);
        }
      }
    }
    __syncthreads();
  }
  // D_blk[i][j] of block (I, J) at lane (i << 4) | (blk << 2) | j: entry (4I + i, 4J + j) of bin 4 grp + blk
  const int di = lane >> 4, db = (lane >> 2) & 3, dj = lane & 3;
  const int bin = NB * grp + db;
  if (bin >= nbins) return;
  int k = 0;
#pragma unroll
  for (int I = 0; I < NRB; ++I)
#pragma unroll
    for (int J = I; J < NRB; ++J, ++k) {
      const int a = 4 * I + di, b = 4 * J + dj;
      if (a < N && b < N && (I < J || di <= dj)) {
        const int pair = a * N - (a * (a - 1)) / 2 + (b - a);
#pragma unroll
        for (int c = 0; c < NC; ++c) rec[((size_t)bin * G::NPAIR + pair) * NC + c] = acc[c][k];
      }
    }
}

// M[g][o][c] (=|+=) sum over the support nodes a with a + o in the support of
// rec[bin g - a][pair(a, a + o)][c], in a fixed order. One thread per (node,
// offset o >= centre), which stores its sum at M[g][o] and at the mirrored
// entry M[g + d(o)][-o] (equal by the spatial symmetry), so that each record
// entry is read once (one thread per offset read each pair twice: the TSC
// deposit on 256^2 cells took 134 instead of 112 us, CIC 38.4 instead of 36.9).
template <typename T, int R, int NC>
__global__ __launch_bounds__(256) void k_gather2d(GridDev g, const double* __restrict__ rec, int accumulate,
                                                  T* __restrict__ M) {
  using G = G2<R>;
  constexpr int NS = G::NS, N = G::N, NO = G::NO, NOFF = G::NOFF;
  constexpr int O0 = (NOFF - 1) / 2;            // first offset computed: the centre
  constexpr int NIT = NOFF - O0;                // offsets computed per node
  const size_t nn = (size_t)g.n0 * g.n1;
  const size_t t = (size_t)xcd_remap(blockIdx.x, gridDim.x) * blockDim.x + threadIdx.x;
  if (t >= nn * NIT) return;
  const size_t node = t / NIT;
  const int o = O0 + (int)(t - node * NIT);
  const int gx = (int)(node % g.n0), gy = (int)(node / g.n0);
  const int ox = o % NO - R, oy = o / NO - R;
  double sum[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) sum[c] = 0.0;
#pragma unroll
  for (int ay = 0; ay < NS; ++ay) {
    if (ay + oy < 0 || ay + oy > R) continue;
#pragma unroll
    for (int ax = 0; ax < NS; ++ax) {
      if (ax + ox < 0 || ax + ox > R) continue;
      const int a = ax + NS * ay, b = a + ox + NS * oy;
      const int lo = a < b ? a : b, hi = a < b ? b : a;
      const int pair = lo * N - (lo * (lo - 1)) / 2 + (hi - lo);
      const int kx = gx - ax < 0 ? gx - ax + g.n0 : gx - ax;
      const int ky = gy - ay < 0 ? gy - ay + g.n1 : gy - ay;
      const double* src = rec + (((size_t)kx + (size_t)g.n0 * ky) * G::NPAIR + pair) * NC;
#pragma unroll
      for (int c = 0; c < NC; ++c) sum[c] += src[c];
    }
  }
  T* dst = M + (node * NOFF + o) * NC;
#pragma unroll
  for (int c = 0; c < NC; ++c) dst[c] = accumulate ? (T)((double)dst[c] + sum[c]) : (T)sum[c];
  if (o != O0) {
    int mx = gx + ox, my = gy + oy;
    mx = mx < 0 ? mx + g.n0 : (mx >= g.n0 ? mx - g.n0 : mx);
    my = my < 0 ? my + g.n1 : (my >= g.n1 ? my - g.n1 : my);
    T* mdst = M + (((size_t)mx + (size_t)g.n0 * my) * NOFF + (NOFF - 1 - o)) * NC;
#pragma unroll
    for (int c = 0; c < NC; ++c) mdst[c] = accumulate ? (T)((double)mdst[c] + sum[c]) : (T)sum[c];
  }
}

size_t record_bytes_2d(int order, bool tensorial, int64_t nbins) {
  const int n = (order + 1) * (order + 1);
  return (size_t)nbins * (n * (n + 1) / 2) * (tensorial ? 9 : 1) * sizeof(double);
}

template <typename PT, int R>
static hipError_t mass2d_t(const GridDev& g, const Particles& P, const int32_t* bin_start, const int32_t* perm,
                           double beta, double sigma, double* rec, hipStream_t s) {
  const int nbins = g.n0 * g.n1;
  const dim3 grid((unsigned)((nbins + NB - 1) / NB)), block(64);
  if (P.B)
    hipLaunchKernelGGL((k_mass2d<PT, R, 9>), grid, block, 0, s, g, (const PT*)P.pos, (const double*)P.w,
                       (const PT*)P.B, bin_start, perm, P.np, nbins, beta, sigma, rec);
  else
    hipLaunchKernelGGL((k_mass2d<PT, R, 1>), grid, block, 0, s, g, (const PT*)P.pos, (const double*)P.w,
                       (const PT*)nullptr, bin_start, perm, P.np, nbins, beta, sigma, rec);
  return hipGetLastError();
}

hipError_t launch_contract_2d(const GridDev& g, int order, const Particles& P, const int32_t* bin_start,
                              const int32_t* perm, double beta, double sigma, void* rec, hipStream_t s) {
  double* r = (double*)rec;
  if (P.pos32)
    return order == 1 ? mass2d_t<float, 1>(g, P, bin_start, perm, beta, sigma, r, s)
                      : mass2d_t<float, 2>(g, P, bin_start, perm, beta, sigma, r, s);
  return order == 1 ? mass2d_t<double, 1>(g, P, bin_start, perm, beta, sigma, r, s)
                    : mass2d_t<double, 2>(g, P, bin_start, perm, beta, sigma, r, s);
}

hipError_t launch_gather_2d(const GridDev& g, int order, bool tensorial, const void* rec, int accumulate, void* M,
                            hipStream_t s) {
  const int noff = order == 1 ? 9 : 25;
  const size_t nt = (size_t)g.n0 * g.n1 * ((noff + 1) / 2);  // threads: nodes x offsets from the centre on
  const size_t blocks = (nt + 255) / 256;
  if (blocks > 0x7fffffffULL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(256);
  const double* r = (const double*)rec;
  if (order == 1) {
    if (tensorial)
      hipLaunchKernelGGL((k_gather2d<double, 1, 9>), grid, block, 0, s, g, r, accumulate, (double*)M);
    else
      hipLaunchKernelGGL((k_gather2d<double, 1, 1>), grid, block, 0, s, g, r, accumulate, (double*)M);
  } else {
    if (tensorial)
      hipLaunchKernelGGL((k_gather2d<double, 2, 9>), grid, block, 0, s, g, r, accumulate, (double*)M);
    else
      hipLaunchKernelGGL((k_gather2d<double, 2, 1>), grid, block, 0, s, g, r, accumulate, (double*)M);
  }
  return hipGetLastError();
}

}  // namespace mmk
