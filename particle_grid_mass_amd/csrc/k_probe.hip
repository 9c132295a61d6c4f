// On-box peak of the fp64 matrix instruction the contractions use, for the
// roofline's measured peak beside the published one. Each thread keeps 16
// independent accumulators and issues 16 v_mfma_f64_4x4x4_4b per iteration;
// each instruction is 4 blocks x 4 x 4 x 4 fused multiply-adds = 512 flop per
// wave. The sums go to `out` so that the work is kept.
#include "mm_internal.h"

namespace mmk {

namespace {
constexpr int PROBE_ACC = 16;
}

__global__ __launch_bounds__(256) void k_probe_mfma_f64(double* __restrict__ out, int iters, double a, double b) {
  double acc[PROBE_ACC];
#pragma unroll
  for (int i = 0; i < PROBE_ACC; ++i) acc[i] = 0.0;
  const double x = a + threadIdx.x * 1e-9, y = b;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < PROBE_ACC; ++i) acc[i] = mfma_f64_4x4x4(x, y, acc[i]);
  }
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < PROBE_ACC; ++i) s += acc[i];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

hipError_t launch_probe_mfma_f64(int nblocks, int iters, double* out, hipStream_t s) {
  hipLaunchKernelGGL(k_probe_mfma_f64, dim3(nblocks), dim3(256), 0, s, out, iters, 1.0, 0.5);
  return hipGetLastError();
}

}  // namespace mmk
