// The assembled mass matrix applied to a grid vector, read off the stencil
// storage: y[g] = sum_o M[g][o] x[g+o]. This is how the matrix enters the
// implicit field equation of Pennati & Markidis, "Mass Matrix Assembly on
// Tensor Cores for Implicit Particle-In-Cell Methods" (Sec. 2.1), acting on
// the grid electric field; M[g][o] is a 3x3 block (row i, column j) on the
// 3-vector x[g+o] in the tensorial case, a scalar otherwise.
//
// From the canonical half (Sec. 3.4: offsets o >= centre, stored at
// o - centre) the other half comes from the symmetry M[g][-o] = M[g-o][o]:
//   y[g] = sum_{k} Mc[g][k] x[g+o_k] + sum_{k>0} Mc[g-o_k][k] x[g-o_k].
//
// HBM-bound: every stencil entry is read once (the canonical half is read
// twice, the second time from the rows of the R planes just visited, which
// are in L2), the vector x a few times through the cache.
#include "mm_contract.h"

namespace mmk {

// One thread per (node, row i); the three threads of a node read its
// 9-component blocks as contiguous 24-byte rows.
template <typename T, int R, int NC, bool CANON>
__global__ __launch_bounds__(256) void k_stencil_matvec(GridDev g, const T* __restrict__ M, const T* __restrict__ x,
                                                        T* __restrict__ y) {
  constexpr int NO = 2 * R + 1, NOFF = NO * NO * NO;
  constexpr int C = (NOFF - 1) / 2;               // centre offset
  constexpr int NOUT = CANON ? NOFF - C : NOFF;   // offsets stored per node
  constexpr int TPN = NC == 9 ? 3 : 1;            // threads per node (rows)
  const size_t nn = (size_t)g.n0 * g.n1 * g.n2;
  // each XCD takes a contiguous range of nodes, so the rows of the planes just
  // behind (the canonical second term) and the vector x are in its L2
  const size_t t = (size_t)xcd_remap(blockIdx.x, gridDim.x) * blockDim.x + threadIdx.x;
  if (t >= nn * TPN) return;
  const size_t node = t / TPN;
  const int i = (int)(t - node * TPN);
  const int gx = (int)(node % g.n0), gy = (int)((node / g.n0) % g.n1), gz = (int)(node / ((size_t)g.n0 * g.n1));
  // wrapped coordinates g + d for d in [-R, R] per axis
  int xs[NO], ys[NO], zs[NO];
#pragma unroll
  for (int d = 0; d < NO; ++d) {
    int v = gx + d - R;
    xs[d] = v < 0 ? v + g.n0 : (v >= g.n0 ? v - g.n0 : v);
    v = gy + d - R;
    ys[d] = v < 0 ? v + g.n1 : (v >= g.n1 ? v - g.n1 : v);
    v = gz + d - R;
    zs[d] = v < 0 ? v + g.n2 : (v >= g.n2 ? v - g.n2 : v);
  }
  auto nb = [&](int ix, int iy, int iz) -> size_t {
    return (size_t)xs[ix] + (size_t)g.n0 * ((size_t)ys[iy] + (size_t)g.n1 * zs[iz]);
  };
  T acc = T(0);
  const T* Mg = M + node * (NOUT * NC) + (NC == 9 ? 3 * i : 0);
#pragma unroll
  for (int k = 0; k < NOUT; ++k) {
    const int o = CANON ? C + k : k;
    const int ox = o % NO, oy = (o / NO) % NO, oz = o / (NO * NO);  // d + R per axis
    const size_t q = nb(ox, oy, oz);                                  // g + o
    if (NC == 9) {
      const T* m = Mg + k * NC;
      const T* xq = x + 3 * q;
      acc += m[0] * xq[0] + m[1] * xq[1] + m[2] * xq[2];
    } else {
      acc += Mg[k] * x[q];
    }
    if (CANON && k > 0) {  // M[g][-o] = M[g-o][o]
      const size_t p = nb(2 * R - ox, 2 * R - oy, 2 * R - oz);  // g - o
      const T* m = M + p * (NOUT * NC) + k * NC + (NC == 9 ? 3 * i : 0);
      if (NC == 9) {
        const T* xp = x + 3 * p;
        acc += m[0] * xp[0] + m[1] * xp[1] + m[2] * xp[2];
      } else {
        acc += m[0] * x[p];
      }
    }
  }
  y[t] = acc;
}

template <typename T, int R, int NC>
static hipError_t matvec_launch(const GridDev& g, bool canonical, const void* M, const void* x, void* y,
                                hipStream_t s) {
  const size_t n = (size_t)g.n0 * g.n1 * g.n2 * (NC == 9 ? 3 : 1);
  const size_t blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffULL) return hipErrorInvalidValue;
  if (canonical)
    hipLaunchKernelGGL((k_stencil_matvec<T, R, NC, true>), dim3((unsigned)blocks), dim3(256), 0, s, g, (const T*)M,
                       (const T*)x, (T*)y);
  else
    hipLaunchKernelGGL((k_stencil_matvec<T, R, NC, false>), dim3((unsigned)blocks), dim3(256), 0, s, g, (const T*)M,
                       (const T*)x, (T*)y);
  return hipGetLastError();
}

hipError_t launch_stencil_matvec(const GridDev& g, int order, bool f32, bool tensorial, bool canonical, const void* M,
                                 const void* x, void* y, hipStream_t s) {
  if (f32) {
    if (order == 1)
      return tensorial ? matvec_launch<float, 1, 9>(g, canonical, M, x, y, s)
                       : matvec_launch<float, 1, 1>(g, canonical, M, x, y, s);
    return tensorial ? matvec_launch<float, 2, 9>(g, canonical, M, x, y, s)
                     : matvec_launch<float, 2, 1>(g, canonical, M, x, y, s);
  }
  if (order == 1)
    return tensorial ? matvec_launch<double, 1, 9>(g, canonical, M, x, y, s)
                     : matvec_launch<double, 1, 1>(g, canonical, M, x, y, s);
  return tensorial ? matvec_launch<double, 2, 9>(g, canonical, M, x, y, s)
                   : matvec_launch<double, 2, 1>(g, canonical, M, x, y, s);
}

}  // namespace mmk
