// The grid's magnetic field at each particle, gathered with the particle's own
// support weights: B_p = sum_a W_pa B[g_a] over the N support nodes (Eq. 12
// weights of Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for
// Implicit Particle-In-Cell Methods", Sec. 2.3). Sec. 4.1 of that page names
// loading the field and forming alpha_p as the preparation work of the
// tensorial assembly. The fp64 matrix-core contractions gather the field
// themselves; this kernel serves the other paths, which then read B_p as a
// per-particle field.
//
// One thread per particle; the N nodes of one particle are gathered through
// the cache (neighbouring particles share them).
#include "mm_internal.h"

namespace mmk {

// T: arithmetic and output; PT: stored positions and field (T, or fp32 into fp64).
template <typename T, int R, typename PT>
__global__ __launch_bounds__(256) void k_interp_field(GridDev g, const PT* __restrict__ pos, int np,
                                                      const PT* __restrict__ F, T* __restrict__ out) {
  constexpr int NS = R + 1;
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= np) return;
  T wx[3], wy[3], wz[3];
  const int fx = support_axis<T, R, 0>((double)pos[3 * (size_t)p], g, wx);
  const int fy = support_axis<T, R, 1>((double)pos[3 * (size_t)p + 1], g, wy);
  const int fz = support_axis<T, R, 2>((double)pos[3 * (size_t)p + 2], g, wz);
  T b[3] = {T(0), T(0), T(0)};
#pragma unroll
  for (int az = 0; az < NS; ++az) {
    const int z = fz + az < g.n2 ? fz + az : fz + az - g.n2;
#pragma unroll
    for (int ay = 0; ay < NS; ++ay) {
      const int y = fy + ay < g.n1 ? fy + ay : fy + ay - g.n1;
      const size_t row = (size_t)g.n0 * ((size_t)y + (size_t)g.n1 * z);
#pragma unroll
      for (int ax = 0; ax < NS; ++ax) {
        const int x = fx + ax < g.n0 ? fx + ax : fx + ax - g.n0;
        const T W = (wx[ax] * wy[ay]) * wz[az];
        const PT* f = F + 3 * (row + x);
        b[0] += W * (T)f[0];
        b[1] += W * (T)f[1];
        b[2] += W * (T)f[2];
      }
    }
  }
  out[3 * (size_t)p] = b[0];
  out[3 * (size_t)p + 1] = b[1];
  out[3 * (size_t)p + 2] = b[2];
}

template <typename T, typename PT>
static hipError_t interp_t(const GridDev& g, int order, const void* pos, int np, const void* F, void* out,
                           hipStream_t s) {
  const dim3 grid((unsigned)((np + 255) / 256)), block(256);
  if (order == 1)
    hipLaunchKernelGGL((k_interp_field<T, 1, PT>), grid, block, 0, s, g, (const PT*)pos, np, (const PT*)F, (T*)out);
  else
    hipLaunchKernelGGL((k_interp_field<T, 2, PT>), grid, block, 0, s, g, (const PT*)pos, np, (const PT*)F, (T*)out);
  return hipGetLastError();
}

hipError_t launch_interp_field(const GridDev& g, int order, bool f32, const void* pos, int np, const void* F,
                               void* out, hipStream_t s, bool pos32) {
  if (np <= 0) return hipSuccess;
  if (f32) return interp_t<float, float>(g, order, pos, np, F, out, s);
  return pos32 ? interp_t<double, float>(g, order, pos, np, F, out, s)
               : interp_t<double, double>(g, order, pos, np, F, out, s);
}

}  // namespace mmk
