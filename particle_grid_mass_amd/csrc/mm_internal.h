// Host-side launcher interface between the C ABI (mm_abi.hip) and the kernel
// translation units. Not part of the public API.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mm_device.h"

namespace mmk {

struct Particles {
  const void* pos;  // [np][3]
  const void* w;    // [np]
  const void* B;    // [np][3] or NULL (scalar, or the field is on the grid)
  int np;
  const void* Bgrid = nullptr;  // [nnodes][3]: field on the grid nodes, gathered at each particle
  bool pos32 = false;           // fp64 arithmetic on fp32 positions and fields (w and outputs fp64)
  // Elements from one particle's values to the next one's: position p is
  // pos[ps p + 0..2], weight w[wst p], field B[bst p + 0..2]. Other strides
  // than the dense 3, 1, 3 (records of several values per particle) are
  // taken by the binning and the fp64 CIC record contraction only.
  int64_t ps = 3, wst = 1, bst = 3;
  bool strided() const { return ps != 3 || wst != 1 || bst != 3; }
};

// out[p] = sum_a W_pa F[g_a]: the nodal field F [nnodes][3] at every particle.
// pos32: fp32 positions and field, fp64 arithmetic and output (f32 must be false).
hipError_t launch_interp_field(const GridDev& g, int order, bool f32, const void* pos, int np, const void* F,
                               void* out, hipStream_t s, bool pos32 = false);

// M <- 0 (a fill kernel, so the stream stays capturable).
hipError_t launch_fill_zero(void* M, size_t count, bool f32, hipStream_t s);

// Conventional per-particle atomic scatter (comparison kernel).
hipError_t launch_atomic_scatter(const GridDev& g, int order, bool f32, const Particles& P, double beta,
                                 double sigma, void* M, hipStream_t s);

// Binning: stable LSD radix sort of first-support-node keys.
size_t bin_workspace_bytes(int64_t np, int64_t nbins);
// pos32 (with f32 false): fp32 positions, keys found in fp64 arithmetic.
// ps: elements from one particle's position to the next one's (3 when dense).
hipError_t launch_bin(const GridDev& g, int order, bool f32, const void* pos, int np, int nbins, int32_t* bin_start,
                      int32_t* perm, void* ws, hipStream_t s, bool pos32 = false, int64_t ps = 3);

}  // namespace mmk
