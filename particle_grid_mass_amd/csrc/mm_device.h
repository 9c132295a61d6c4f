// Device-side helpers shared by the mass-matrix kernels (gfx950 only).
//
// Support rule and weights: Pennati & Markidis, "Mass Matrix Assembly on
// Tensor Cores for Implicit Particle-In-Cell Methods", Sec. 2.3 (Eq. 12 and
// the CIC/TSC support placement). Response tensor: the implicit-midpoint
// alpha the page cites as Eq. (5) in Sec. 4.1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmk {

typedef double v4d __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Grid passed by value to every kernel (origin and h in fp64; the support of a
// particle is always found in fp64, see support_axis).
// Bit d of `exact` is set when h_d is a power of two: then (x - o) * (1/h)
// equals the IEEE quotient (x - o) / h bit for bit, and the cheaper product is used.
struct GridDev {
  int n0, n1, n2;
  int exact;
  double o0, o1, o2;
  double h0, h1, h2;
  double i0, i1, i2;  // 1 / h
};

// Grid coordinate u = (x - origin) / h along axis D.
template <typename T, int D>
__device__ __forceinline__ T grid_coord(T x, const GridDev& g) {
  const T o = (T)(D == 0 ? g.o0 : D == 1 ? g.o1 : g.o2);
  const T dx = x - o;
  if ((g.exact >> D) & 1) return dx * (T)(D == 0 ? g.i0 : D == 1 ? g.i1 : g.i2);
  return dx / (T)(D == 0 ? g.h0 : D == 1 ? g.h1 : g.h2);
}

__device__ __forceinline__ int wrap_node(int j, int n) {
  int r = j % n;
  return r < 0 ? r + n : r;
}

// One axis of the support of a stored coordinate x (read exactly into fp64,
// whatever its storage type): returns the first support node (wrapped) and
// writes the R+1 one-dimensional B-spline weights in the precision T.
// The grid coordinate u = (x - origin)/h, j = floor(u), xi = u - j and the
// TSC half-cell decision are taken in fp64 arithmetic for every T, so the
// binning and every kernel agree on each particle's support, and an fp32
// position is placed as its exact value is; the weights are then formed in T
// from the fraction rounded to T.
//   CIC: nodes j, j+1 with (1 - xi, xi).
//   TSC: centre m = j (xi < 1/2) or j+1 (xi >= 1/2); delta = offset from m;
//        nodes m-1, m, m+1 with (1/2 (1/2 - delta)^2, 3/4 - delta^2, 1/2 (1/2 + delta)^2).
template <typename T, int R, int D>
__device__ __forceinline__ int support_axis(double x, const GridDev& g, T* wt) {
  const int n = D == 0 ? g.n0 : D == 1 ? g.n1 : g.n2;
  const double u = grid_coord<double, D>(x, g);
  const double fl = floor(u);
  const int j = (int)fl;
  const double xi = u - fl;
  if (R == 1) {
    const T t = (T)xi;
    wt[0] = T(1) - t;
    wt[1] = t;
    return wrap_node(j, n);
  } else {
    int m = j;
    double dd = xi;
    if (!(xi < 0.5)) {
      m = j + 1;
      dd = xi - 1.0;
    }
    const T d = (T)dd;
    const T p = T(0.5) - d, q = T(0.5) + d;
    wt[0] = T(0.5) * p * p;
    wt[1] = T(0.75) - d * d;
    wt[2] = T(0.5) * q * q;
    return wrap_node(m - 1, n);
  }
}

// First support node of a particle as a linear node index (the bin key),
// decided in fp64 on the stored position (see support_axis).
// On a 2D grid (n2 == 1) z is ignored and the key is the node in the plane.
template <int R, typename PT>
__device__ __forceinline__ int particle_key(const PT* p3, const GridDev& g) {
  double wt[3];
  int fx = support_axis<double, R, 0>((double)p3[0], g, wt);
  int fy = support_axis<double, R, 1>((double)p3[1], g, wt);
  int fz = g.n2 == 1 ? 0 : support_axis<double, R, 2>((double)p3[2], g, wt);
  return fx + g.n0 * (fy + g.n1 * fz);
}

// t^{ij} = f * alpha^{ij}, f = sigma * w, row-major 3x3:
//   alpha = (I + beta^2 B B^T - beta [B]x) / (1 + beta^2 |B|^2),
//   [B]x = [[0,-Bz,By],[Bz,0,-Bx],[-By,Bx,0]].
template <typename T>
__device__ __forceinline__ void response(T bx, T by, T bz, T beta, T f, T* t) {
  T b2 = beta * beta;
  T den = T(1) + b2 * (bx * bx + by * by + bz * bz);
  T gq = f / den;
  T sx = b2 * bx, sy = b2 * by, sz = b2 * bz;
  T cx = beta * bx, cy = beta * by, cz = beta * bz;
  t[0] = gq * (T(1) + sx * bx);
  t[1] = gq * (sx * by + cz);
  t[2] = gq * (sx * bz - cy);
  t[3] = gq * (sy * bx - cz);
  t[4] = gq * (T(1) + sy * by);
  t[5] = gq * (sy * bz + cx);
  t[6] = gq * (sz * bx + cy);
  t[7] = gq * (sz * by - cx);
  t[8] = gq * (T(1) + sz * bz);
}

// Matrix-core wrappers. Operand lane layouts (measured on gfx950 with
// one-hot probes; l = lane 0..63):
//  f64 4x4x4 (4 blocks): A_blk[i][k] at l = (k<<4)|(blk<<2)|i,
//                        B_blk[k][j] at l = (k<<4)|(blk<<2)|j,
//                        D_blk[i][j] at l = (i<<4)|(blk<<2)|j.
//  f64 16x16x4:          A[i][k] at l = 16k + i, B[k][j] at l = 16k + j,
//                        D[i][j] at lane 16(i%4) + j, register i/4.
//  f32 16x16x4:          A, B as f64 16x16x4; D[i][j] at lane 16(i/4) + j, register i%4.
//  f32 4x4x1 (16 blocks):A_blk[i] at l = 4blk + i, B_blk[j] at l = 4blk + j,
//                        D_blk[i][j] at lane 4blk + j, register i.
__device__ __forceinline__ double mfma_f64_4x4x4(double a, double b, double c) {
  return __builtin_amdgcn_mfma_f64_4x4x4f64(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4d mfma_f64_16x16x4(double a, double b, v4d c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_f32_16x16x4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_f32_4x4x1(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void atomic_add(double* p, double v) { unsafeAtomicAdd(p, v); }
__device__ __forceinline__ void atomic_add(float* p, float v) { unsafeAtomicAdd(p, v); }

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2). Remap the hardware block id so that XCD x receives a contiguous range
// of logical blocks, keeping neighbouring bins on one L2. Bijective on [0, nb).
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int NX = 8;
  int x = b % NX, idx = b / NX;
  int per = nb / NX, rem = nb % NX;
  return x * per + (x < rem ? x : rem) + idx;
}

// Hardware block b runs on XCD b % 8. Give XCD x the chunks x, x + 8, x + 16,
// ... of CH consecutive logical blocks: neighbouring blocks still share an
// XCD (and its L2) inside a chunk, and every XCD sweeps the whole grid, so
// work whose cost varies across the grid (clustered particles) is spread
// evenly over the XCDs. Bijective on [0, nb); the last nb mod (8 CH) blocks
// map to themselves.
__device__ __forceinline__ int xcd_chunk_remap(int b, int nb, int CH) {
  const int full = nb - nb % (8 * CH);
  if (b >= full) return b;
  const int x = b % 8, idx = b / 8;
  return ((idx / CH) * 8 + x) * CH + idx % CH;
}

}  // namespace mmk
