// Zero fill and the conventional per-particle atomic-scatter kernel.
//
// The atomic scatter is the in-house comparison for the matrix-core path: it
// evaluates Eq. (6) of Pennati & Markidis (Sec. 2.1) particle by particle and
// adds each of the N^2 * ncomp products straight into the stencil-format
// matrix with hardware fp atomics - the "naive atomic-based mass matrix
// kernel on unsorted particles" of their Sec. 4.2, variant (i). It needs no
// binning and accepts any particle order.
#include "mm_internal.h"

namespace mmk {

template <typename T>
__global__ void k_fill_zero(T* __restrict__ M, size_t count) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < count; i += stride) M[i] = T(0);
}

hipError_t launch_fill_zero(void* M, size_t count, bool f32, hipStream_t s) {
  if (count == 0) return hipSuccess;
  size_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (f32)
    hipLaunchKernelGGL(k_fill_zero<float>, dim3((unsigned)blocks), dim3(256), 0, s, (float*)M, count);
  else
    hipLaunchKernelGGL(k_fill_zero<double>, dim3((unsigned)blocks), dim3(256), 0, s, (double*)M, count);
  return hipGetLastError();
}

// One thread per particle: support, weights, coefficients, then one atomic
// add per (a, b, comp).
template <typename T, int R, int NC>
__global__ __launch_bounds__(256) void k_atomic_scatter(GridDev g, const T* __restrict__ pos,
                                                        const T* __restrict__ w, const T* __restrict__ Bf, int np,
                                                        T beta, T sigma, T* __restrict__ M) {
  constexpr int NS = R + 1, N = NS * NS * NS, NO = 2 * R + 1, NOFF = NO * NO * NO;
  int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= np) return;
  T x[3] = {pos[3 * (size_t)p], pos[3 * (size_t)p + 1], pos[3 * (size_t)p + 2]};
  T wx[3], wy[3], wz[3];
  int fx = support_axis<T, R, 0>((double)x[0], g, wx);
  int fy = support_axis<T, R, 1>((double)x[1], g, wy);
  int fz = support_axis<T, R, 2>((double)x[2], g, wz);
  T t[NC];
  if (NC == 9) {
    response<T>(Bf[3 * (size_t)p], Bf[3 * (size_t)p + 1], Bf[3 * (size_t)p + 2], beta, sigma * w[p], t);
  } else {
    t[0] = sigma * w[p];
  }
  int gx[NS], gy[NS], gz[NS];
#pragma unroll
  for (int a = 0; a < NS; ++a) {
    gx[a] = fx + a >= g.n0 ? fx + a - g.n0 : fx + a;
    gy[a] = fy + a >= g.n1 ? fy + a - g.n1 : fy + a;
    gz[a] = fz + a >= g.n2 ? fz + a - g.n2 : fz + a;
  }
  for (int a = 0; a < N; ++a) {
    int ax = a % NS, ay = (a / NS) % NS, az = a / (NS * NS);
    T Wa = (wx[ax] * wy[ay]) * wz[az];
    size_t node = (size_t)gx[ax] + (size_t)g.n0 * ((size_t)gy[ay] + (size_t)g.n1 * (size_t)gz[az]);
    T* row = M + node * NOFF * NC;
    for (int b = 0; b < N; ++b) {
      int bx = b % NS, by = (b / NS) % NS, bz = b / (NS * NS);
      T ww = Wa * ((wx[bx] * wy[by]) * wz[bz]);
      int o = (bx - ax + R) + NO * ((by - ay + R) + NO * (bz - az + R));
#pragma unroll
      for (int c = 0; c < NC; ++c) atomic_add(row + o * NC + c, t[c] * ww);
    }
  }
}

template <typename T>
static hipError_t atomic_scatter_t(const GridDev& g, int order, const Particles& P, double beta, double sigma,
                                   void* M, hipStream_t s) {
  dim3 grid((P.np + 255) / 256), block(256);
  const T* pos = (const T*)P.pos;
  const T* w = (const T*)P.w;
  const T* B = (const T*)P.B;
  T* Mo = (T*)M;
  if (order == 1) {
    if (B)
      hipLaunchKernelGGL((k_atomic_scatter<T, 1, 9>), grid, block, 0, s, g, pos, w, B, P.np, (T)beta, (T)sigma, Mo);
    else
      hipLaunchKernelGGL((k_atomic_scatter<T, 1, 1>), grid, block, 0, s, g, pos, w, B, P.np, (T)beta, (T)sigma, Mo);
  } else {
    if (B)
      hipLaunchKernelGGL((k_atomic_scatter<T, 2, 9>), grid, block, 0, s, g, pos, w, B, P.np, (T)beta, (T)sigma, Mo);
    else
      hipLaunchKernelGGL((k_atomic_scatter<T, 2, 1>), grid, block, 0, s, g, pos, w, B, P.np, (T)beta, (T)sigma, Mo);
  }
  return hipGetLastError();
}

hipError_t launch_atomic_scatter(const GridDev& g, int order, bool f32, const Particles& P, double beta,
                                 double sigma, void* M, hipStream_t s) {
  if (P.np == 0) return hipSuccess;
  return f32 ? atomic_scatter_t<float>(g, order, P, beta, sigma, M, s)
             : atomic_scatter_t<double>(g, order, P, beta, sigma, M, s);
}

}  // namespace mmk
