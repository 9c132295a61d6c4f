// Per-bin matrix-core contraction of the mass matrix (gfx950 MFMA).
//
// Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for Implicit
// Particle-In-Cell Methods": within one support group (here: one bin of
// particles sharing their first support node, Sec. 3.3) the local matrix is
//   Mhat^{c}_{ab} = sum_p t_p^c W_pa W_pb          (Sec. 3.1, Eq. 15)
// i.e. A^c B with A^c = W diag(t^c) and B = W^T (Sec. 3.1, Eq. 14), computed
// as batched products whose inner dimension is a batch of particles
// (Sec. 3.2), exploiting the spatial symmetry Mhat_ab = Mhat_ba to skip the
// lower off-diagonal tile (Table 1 and Sec. 4). The page's kernels target
// NVIDIA 8x8x4 / 16x16x8 tiles; these map the same contraction to the CDNA
// matrix instructions:
//
//  CIC fp64: v_mfma_f64_4x4x4 with 4 independent blocks. The 8 support rows
//   split by az into two 4-row halves, giving quadrants Q00, Q01, Q11 per
//   component (Q10 = Q01^T). Each instruction computes ONE (component,
//   quadrant) product for FOUR different 4-particle batches at once (block =
//   batch), so no block is padded; the four block partial sums are added
//   across lanes once per bin. 16 particles per round, 27 (ECSIM) or 3
//   (scalar) instructions per round.
//  CIC fp32: v_mfma_f32_4x4x1 with 16 blocks, one particle per block (K = 1),
//   same quadrant scheme: 16 particles per round.
//  TSC: 27 support rows padded to 32; tiles (0,0), (0,1), (1,1) of
//   v_mfma_{f64,f32}_16x16x4 per component, 4 particles per batch.
//
// Deposit (this file): every local entry is added into the global stencil
// matrix with one hardware atomic add; Q01 / tile (0,1) entries are added at
// both (a,b) and (b,a).
#include "mm_internal.h"

namespace mmk {

// Node id of support node (ax, ay, az) relative to the bin's first node.
__device__ __forceinline__ size_t support_node(int fx, int fy, int fz, int ax, int ay, int az, const GridDev& g) {
  int x = fx + ax, y = fy + ay, z = fz + az;
  x = x >= g.n0 ? x - g.n0 : x;
  y = y >= g.n1 ? y - g.n1 : y;
  z = z >= g.n2 ? z - g.n2 : z;
  return (size_t)x + (size_t)g.n0 * ((size_t)y + (size_t)g.n1 * (size_t)z);
}

template <typename T, int R, int NC>
__device__ __forceinline__ void deposit_pair(T* __restrict__ M, const GridDev& g, int fx, int fy, int fz, int a, int b,
                                             int c, T v) {
  constexpr int NS = R + 1, NO = 2 * R + 1, NOFF = NO * NO * NO;
  int ax = a % NS, ay = (a / NS) % NS, az = a / (NS * NS);
  int bx = b % NS, by = (b / NS) % NS, bz = b / (NS * NS);
  size_t node = support_node(fx, fy, fz, ax, ay, az, g);
  int o = (bx - ax + R) + NO * ((by - ay + R) + NO * (bz - az + R));
  atomic_add(M + (node * NOFF + o) * NC + c, v);
}

// Load particle p and compute its three 1D weight sets plus coefficients.
template <typename T, int R, int NC>
__device__ __forceinline__ void particle_prep(const GridDev& g, const T* __restrict__ pos, const T* __restrict__ w,
                                              const T* __restrict__ Bf, int p, T beta, T sigma, T* wx, T* wy, T* wz,
                                              T* t) {
  axis_support<T, R>(pos[3 * (size_t)p], (T)g.o0, (T)g.h0, g.n0, wx);
  axis_support<T, R>(pos[3 * (size_t)p + 1], (T)g.o1, (T)g.h1, g.n1, wy);
  axis_support<T, R>(pos[3 * (size_t)p + 2], (T)g.o2, (T)g.h2, g.n2, wz);
  T f = sigma * w[p];
  if (NC == 9)
    response<T>(Bf[3 * (size_t)p], Bf[3 * (size_t)p + 1], Bf[3 * (size_t)p + 2], beta, f, t);
  else
    t[0] = f;
}

// ------------------------------------------------------------------ CIC fp64
template <int NC>
__global__ __launch_bounds__(256) void k_cic_f64_atomic(GridDev g, const double* __restrict__ pos,
                                                        const double* __restrict__ w, const double* __restrict__ Bf,
                                                        const int32_t* __restrict__ bin_start,
                                                        const int32_t* __restrict__ perm, int np, int nbins,
                                                        double beta, double sigma, double* __restrict__ M) {
  const int lane = threadIdx.x & 63;
  const int bin = xcd_remap(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
  if (bin >= nbins) return;
  const int slot = (lane >> 2) & 3, r4 = lane & 3, kq = lane >> 4;
  const int pslot = 4 * slot + kq;  // particle of this lane within a 16-particle round
  const int ax = r4 & 1, ay = r4 >> 1;
  int s = bin_start[bin], e = bin_start[bin + 1];
  s = s < 0 ? 0 : s;
  e = e > np ? np : e;

  double acc[NC][3];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c][0] = acc[c][1] = acc[c][2] = 0.0;

  for (int r0 = s; r0 < e; r0 += 16) {
    const int q = r0 + pslot;
    double wlo = 0.0, whi = 0.0, t[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) t[c] = 0.0;
    if (q < e) {
      const int p = perm[q];
      if ((unsigned)p < (unsigned)np) {
        double wx[2], wy[2], wz[2];
        particle_prep<double, 1, NC>(g, pos, w, Bf, p, beta, sigma, wx, wy, wz, t);
        double wxy = wx[ax] * wy[ay];
        wlo = wxy * wz[0];
        whi = wxy * wz[1];
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      double alo = t[c] * wlo, ahi = t[c] * whi;
      acc[c][0] = mfma_f64_4x4x4(alo, wlo, acc[c][0]);
      acc[c][1] = mfma_f64_4x4x4(alo, whi, acc[c][1]);
      acc[c][2] = mfma_f64_4x4x4(ahi, whi, acc[c][2]);
    }
  }
  // Sum the four block partials (lane bits 2-3).
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int qd = 0; qd < 3; ++qd) {
      double v = acc[c][qd];
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 8);
      acc[c][qd] = v;
    }
  if (s >= e) return;
  const int fx = bin % g.n0, fy = (bin / g.n0) % g.n1, fz = bin / (g.n0 * g.n1);
  const int i = lane >> 4, j = lane & 3;  // D row / column within a quadrant
  if (NC == 9) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if ((c & 3) != slot) continue;
      deposit_pair<double, 1, NC>(M, g, fx, fy, fz, i, j, c, acc[c][0]);
      deposit_pair<double, 1, NC>(M, g, fx, fy, fz, 4 + i, 4 + j, c, acc[c][2]);
      deposit_pair<double, 1, NC>(M, g, fx, fy, fz, i, 4 + j, c, acc[c][1]);
      deposit_pair<double, 1, NC>(M, g, fx, fy, fz, 4 + j, i, c, acc[c][1]);
    }
  } else {
    if (slot == 0) deposit_pair<double, 1, NC>(M, g, fx, fy, fz, i, j, 0, acc[0][0]);
    if (slot == 1) deposit_pair<double, 1, NC>(M, g, fx, fy, fz, i, 4 + j, 0, acc[0][1]);
    if (slot == 2) deposit_pair<double, 1, NC>(M, g, fx, fy, fz, 4 + j, i, 0, acc[0][1]);
    if (slot == 3) deposit_pair<double, 1, NC>(M, g, fx, fy, fz, 4 + i, 4 + j, 0, acc[0][2]);
  }
}

// ------------------------------------------------------------------ CIC fp32
template <int NC>
__global__ __launch_bounds__(256) void k_cic_f32_atomic(GridDev g, const float* __restrict__ pos,
                                                        const float* __restrict__ w, const float* __restrict__ Bf,
                                                        const int32_t* __restrict__ bin_start,
                                                        const int32_t* __restrict__ perm, int np, int nbins,
                                                        float beta, float sigma, float* __restrict__ M) {
  const int lane = threadIdx.x & 63;
  const int bin = xcd_remap(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
  if (bin >= nbins) return;
  const int pslot = lane >> 2, r4 = lane & 3;  // block = particle of the round; row/col within quadrant
  const int ax = r4 & 1, ay = r4 >> 1;
  int s = bin_start[bin], e = bin_start[bin + 1];
  s = s < 0 ? 0 : s;
  e = e > np ? np : e;

  v4f acc[NC][3];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int qd = 0; qd < 3; ++qd) acc[c][qd] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int r0 = s; r0 < e; r0 += 16) {
    const int q = r0 + pslot;
    float wlo = 0.f, whi = 0.f, t[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) t[c] = 0.f;
    if (q < e) {
      const int p = perm[q];
      if ((unsigned)p < (unsigned)np) {
        float wx[2], wy[2], wz[2];
        particle_prep<float, 1, NC>(g, pos, w, Bf, p, beta, sigma, wx, wy, wz, t);
        float wxy = wx[ax] * wy[ay];
        wlo = wxy * wz[0];
        whi = wxy * wz[1];
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float alo = t[c] * wlo, ahi = t[c] * whi;
      acc[c][0] = mfma_f32_4x4x1(alo, wlo, acc[c][0]);
      acc[c][1] = mfma_f32_4x4x1(alo, whi, acc[c][1]);
      acc[c][2] = mfma_f32_4x4x1(ahi, whi, acc[c][2]);
    }
  }
  // Sum the 16 block partials (lane bits 2-5).
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int qd = 0; qd < 3; ++qd)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = acc[c][qd][r];
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc[c][qd][r] = v;
      }
  if (s >= e) return;
  const int fx = bin % g.n0, fy = (bin / g.n0) % g.n1, fz = bin / (g.n0 * g.n1);
  const int blk = lane >> 2, j = lane & 3;  // D_blk[i][j] at lane 4 blk + j, register i
  if (NC == 9) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c != blk) continue;  // lane group blk deposits component blk
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        deposit_pair<float, 1, NC>(M, g, fx, fy, fz, i, j, c, acc[c][0][i]);
        deposit_pair<float, 1, NC>(M, g, fx, fy, fz, 4 + i, 4 + j, c, acc[c][2][i]);
        deposit_pair<float, 1, NC>(M, g, fx, fy, fz, i, 4 + j, c, acc[c][1][i]);
        deposit_pair<float, 1, NC>(M, g, fx, fy, fz, 4 + j, i, c, acc[c][1][i]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (blk == 0) deposit_pair<float, 1, NC>(M, g, fx, fy, fz, i, j, 0, acc[0][0][i]);
      if (blk == 1) deposit_pair<float, 1, NC>(M, g, fx, fy, fz, i, 4 + j, 0, acc[0][1][i]);
      if (blk == 2) deposit_pair<float, 1, NC>(M, g, fx, fy, fz, 4 + j, i, 0, acc[0][1][i]);
      if (blk == 3) deposit_pair<float, 1, NC>(M, g, fx, fy, fz, 4 + i, 4 + j, 0, acc[0][2][i]);
    }
  }
}

// ------------------------------------------------------------------ TSC
// W of support row a (a = ax + 3 ay + 9 az, a < 27), selecting the 1D
// weights without dynamic register indexing.
template <typename T>
__device__ __forceinline__ T sel3(const T* v, int k) {
  return k == 0 ? v[0] : (k == 1 ? v[1] : v[2]);
}
template <typename T>
__device__ __forceinline__ T tsc_row_weight(const T* wx, const T* wy, const T* wz, int a) {
  if (a >= 27) return T(0);
  int ax = a % 3, ay = (a / 3) % 3, az = a / 9;
  return (sel3(wx, ax) * sel3(wy, ay)) * sel3(wz, az);
}

template <typename T>
struct TscAcc;
template <>
struct TscAcc<double> {
  typedef v4d V;
  static __device__ __forceinline__ V mma(double a, double b, V c) { return mfma_f64_16x16x4(a, b, c); }
  // D[i][j] for lane l, register r
  static __device__ __forceinline__ int row(int l, int r) { return 4 * r + (l >> 4); }
};
template <>
struct TscAcc<float> {
  typedef v4f V;
  static __device__ __forceinline__ V mma(float a, float b, V c) { return mfma_f32_16x16x4(a, b, c); }
  static __device__ __forceinline__ int row(int l, int r) { return 4 * (l >> 4) + r; }
};

template <typename T, int NC>
__global__ __launch_bounds__(256) void k_tsc_atomic(GridDev g, const T* __restrict__ pos, const T* __restrict__ w,
                                                    const T* __restrict__ Bf, const int32_t* __restrict__ bin_start,
                                                    const int32_t* __restrict__ perm, int np, int nbins, T beta,
                                                    T sigma, T* __restrict__ M) {
  typedef typename TscAcc<T>::V V;
  const int lane = threadIdx.x & 63;
  const int bin = xcd_remap(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
  if (bin >= nbins) return;
  const int i16 = lane & 15, kq = lane >> 4;  // A row / B column, particle of the 4-batch
  int s = bin_start[bin], e = bin_start[bin + 1];
  s = s < 0 ? 0 : s;
  e = e > np ? np : e;

  V acc[NC][3];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int tl = 0; tl < 3; ++tl) acc[c][tl] = V{0, 0, 0, 0};

  for (int r0 = s; r0 < e; r0 += 4) {
    const int q = r0 + kq;
    T w0 = T(0), w1 = T(0), t[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) t[c] = T(0);
    if (q < e) {
      const int p = perm[q];
      if ((unsigned)p < (unsigned)np) {
        T wx[3], wy[3], wz[3];
        particle_prep<T, 2, NC>(g, pos, w, Bf, p, beta, sigma, wx, wy, wz, t);
        w0 = tsc_row_weight<T>(wx, wy, wz, i16);
        w1 = tsc_row_weight<T>(wx, wy, wz, 16 + i16);
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      T a0 = t[c] * w0, a1 = t[c] * w1;
      acc[c][0] = TscAcc<T>::mma(a0, w0, acc[c][0]);
      acc[c][1] = TscAcc<T>::mma(a0, w1, acc[c][1]);
      acc[c][2] = TscAcc<T>::mma(a1, w1, acc[c][2]);
    }
  }
  if (s >= e) return;
  const int fx = bin % g.n0, fy = (bin / g.n0) % g.n1, fz = bin / (g.n0 * g.n1);
  const int j = lane & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = TscAcc<T>::row(lane, r);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      // tile (0,0): a = i, b = j
      deposit_pair<T, 2, NC>(M, g, fx, fy, fz, i, j, c, acc[c][0][r]);
      // tile (1,1): a = 16 + i, b = 16 + j (rows/cols >= 27 are padding)
      if (16 + i < 27 && 16 + j < 27) deposit_pair<T, 2, NC>(M, g, fx, fy, fz, 16 + i, 16 + j, c, acc[c][2][r]);
      // tile (0,1) and its transpose
      if (16 + j < 27) {
        deposit_pair<T, 2, NC>(M, g, fx, fy, fz, i, 16 + j, c, acc[c][1][r]);
        deposit_pair<T, 2, NC>(M, g, fx, fy, fz, 16 + j, i, c, acc[c][1][r]);
      }
    }
  }
}

template <typename T>
static hipError_t mfma_atomic_t(const GridDev& g, int order, const Particles& P, const int32_t* bin_start,
                                const int32_t* perm, double beta, double sigma, void* M, hipStream_t s) {
  const int nbins = g.n0 * g.n1 * g.n2;
  dim3 grid((nbins + 3) / 4), block(256);
  const T* pos = (const T*)P.pos;
  const T* w = (const T*)P.w;
  const T* B = (const T*)P.B;
  T* Mo = (T*)M;
  const T tb = (T)beta, ts = (T)sigma;
  if (order == 1) {
    if (sizeof(T) == 8) {
      if (B)
        hipLaunchKernelGGL(k_cic_f64_atomic<9>, grid, block, 0, s, g, (const double*)pos, (const double*)w,
                           (const double*)B, bin_start, perm, P.np, nbins, beta, sigma, (double*)Mo);
      else
        hipLaunchKernelGGL(k_cic_f64_atomic<1>, grid, block, 0, s, g, (const double*)pos, (const double*)w,
                           (const double*)B, bin_start, perm, P.np, nbins, beta, sigma, (double*)Mo);
    } else {
      if (B)
        hipLaunchKernelGGL(k_cic_f32_atomic<9>, grid, block, 0, s, g, (const float*)pos, (const float*)w,
                           (const float*)B, bin_start, perm, P.np, nbins, (float)beta, (float)sigma, (float*)Mo);
      else
        hipLaunchKernelGGL(k_cic_f32_atomic<1>, grid, block, 0, s, g, (const float*)pos, (const float*)w,
                           (const float*)B, bin_start, perm, P.np, nbins, (float)beta, (float)sigma, (float*)Mo);
    }
  } else {
    if (B)
      hipLaunchKernelGGL((k_tsc_atomic<T, 9>), grid, block, 0, s, g, pos, w, B, bin_start, perm, P.np, nbins, tb, ts,
                         Mo);
    else
      hipLaunchKernelGGL((k_tsc_atomic<T, 1>), grid, block, 0, s, g, pos, w, B, bin_start, perm, P.np, nbins, tb, ts,
                         Mo);
  }
  return hipGetLastError();
}

hipError_t launch_mfma_atomic(const GridDev& g, int order, bool f32, const Particles& P, const int32_t* bin_start,
                              const int32_t* perm, double beta, double sigma, void* M, hipStream_t s) {
  return f32 ? mfma_atomic_t<float>(g, order, P, bin_start, perm, beta, sigma, M, s)
             : mfma_atomic_t<double>(g, order, P, bin_start, perm, beta, sigma, M, s);
}

}  // namespace mmk
