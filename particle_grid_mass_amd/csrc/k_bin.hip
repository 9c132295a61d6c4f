// Particle binning by support set: a stable LSD radix sort of each
// particle's first-support-node index.
//
// Pennati & Markidis (Sec. 3.3) partition the particles of a cell into
// support groups whose members touch the same N grid nodes, and require the
// particles sorted by cell (Sec. 4.2; the counting sort of their reference
// [2]). Keying every particle by the linear index of its first support node
// makes each key one support group (for CIC: the cell), so one bin = one
// group with a single local matrix.
//
// Pipeline (all on the caller's stream):
//   k_keys          key[p] = first support node of particle p
//   per 8-bit digit: k_radix_hist (per-tile digit counts, digit-major)
//                    exclusive scan of the counts (multi-level)
//                    k_radix_scatter (stable in-tile ranks by wave ballots)
//   k_bin_bounds    bin_start[k] = lower_bound(sorted keys, k)
#include "mm_internal.h"

namespace mmk {

constexpr int RS_THREADS = 256;
constexpr int RS_ITEMS = 16;
constexpr int RS_TILE = RS_THREADS * RS_ITEMS;  // elements per block
constexpr int SCAN_THREADS = 256;
constexpr int SCAN_ITEMS = 8;
constexpr int SCAN_TILE = SCAN_THREADS * SCAN_ITEMS;

template <typename T, int R>
__global__ void k_keys(GridDev g, const T* __restrict__ pos, int np, uint32_t* __restrict__ keys) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < np) keys[i] = (uint32_t)particle_key<T, R>(pos + 3 * (size_t)i, g);
}

__global__ __launch_bounds__(RS_THREADS) void k_radix_hist(const uint32_t* __restrict__ keys, int n, int shift,
                                                           int32_t* __restrict__ ghist, int nblocks) {
  __shared__ int h[256];
  const int tid = threadIdx.x;
  h[tid] = 0;
  __syncthreads();
  const int base = blockIdx.x * RS_TILE;
  for (int it = 0; it < RS_ITEMS; ++it) {
    int idx = base + it * RS_THREADS + tid;
    if (idx < n) atomicAdd(&h[(keys[idx] >> shift) & 255], 1);
  }
  __syncthreads();
  ghist[(size_t)tid * nblocks + blockIdx.x] = h[tid];
}

// Stable scatter: elements are ranked in index order (round, wave, lane).
__global__ __launch_bounds__(RS_THREADS) void k_radix_scatter(const uint32_t* __restrict__ keys_in,
                                                              const int32_t* __restrict__ vals_in, int n, int shift,
                                                              const int32_t* __restrict__ goff, int nblocks,
                                                              uint32_t* __restrict__ keys_out,
                                                              int32_t* __restrict__ vals_out) {
  __shared__ int cnt[256];
  __shared__ int wcnt[RS_THREADS / 64][256];
  __shared__ int boff[256];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  cnt[tid] = 0;
  boff[tid] = goff[(size_t)tid * nblocks + blockIdx.x];
#pragma unroll
  for (int wv = 0; wv < RS_THREADS / 64; ++wv) wcnt[wv][tid] = 0;
  __syncthreads();
  const unsigned long long lt = __lanemask_lt();
  const int base = blockIdx.x * RS_TILE;
  for (int it = 0; it < RS_ITEMS; ++it) {
    const int idx = base + it * RS_THREADS + tid;
    const bool valid = idx < n;
    uint32_t key = valid ? keys_in[idx] : 0u;
    int32_t val = valid ? (vals_in ? vals_in[idx] : idx) : 0;
    int d = (int)((key >> shift) & 255u);
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      bool bit = (d >> b) & 1;
      unsigned long long m = __ballot(valid && bit);
      peers &= bit ? m : ~m;
    }
    int rank = __popcll(peers & lt);
    if (valid && rank == 0) wcnt[wave][d] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = boff[d] + cnt[d] + rank;
      for (int wv = 0; wv < wave; ++wv) pos += wcnt[wv][d];
      keys_out[pos] = key;
      vals_out[pos] = val;
    }
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int wv = 0; wv < RS_THREADS / 64; ++wv) {
      tot += wcnt[wv][tid];
      wcnt[wv][tid] = 0;
    }
    cnt[tid] += tot;
    __syncthreads();
  }
}

// Exclusive scan of one tile per block; tile totals go to sums[block].
__global__ __launch_bounds__(SCAN_THREADS) void k_scan_tile(const int32_t* in, int32_t* out, int n,
                                                            int32_t* sums) {
  __shared__ int wsum[SCAN_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t base = (size_t)blockIdx.x * SCAN_TILE + (size_t)tid * SCAN_ITEMS;
  int v[SCAN_ITEMS];
  int run = 0;
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; ++i) {
    size_t idx = base + i;
    v[i] = idx < (size_t)n ? in[idx] : 0;
    run += v[i];
  }
  // inclusive wave scan of thread totals
  int incl = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int wbase = 0, total = 0;
#pragma unroll
  for (int wv = 0; wv < SCAN_THREADS / 64; ++wv) {
    if (wv < wave) wbase += wsum[wv];
    total += wsum[wv];
  }
  int excl = wbase + incl - run;
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; ++i) {
    size_t idx = base + i;
    if (idx < (size_t)n) out[idx] = excl;
    excl += v[i];
  }
  if (tid == 0) sums[blockIdx.x] = total;
}

__global__ __launch_bounds__(SCAN_THREADS) void k_scan_add(int32_t* out, int n, const int32_t* sums) {
  const int add = sums[blockIdx.x];
  const size_t base = (size_t)blockIdx.x * SCAN_TILE;
  for (int i = threadIdx.x; i < SCAN_TILE; i += SCAN_THREADS) {
    size_t idx = base + i;
    if (idx < (size_t)n) out[idx] += add;
  }
}

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

static size_t scan_tmp_ints(size_t n) {
  size_t total = 0;
  while (n > 1) {
    size_t nb = (n + SCAN_TILE - 1) / SCAN_TILE;
    total += align256(nb * 4) / 4;
    n = nb;
  }
  return total + 64;
}

static hipError_t scan_exclusive(const int32_t* in, int32_t* out, int n, int32_t* tmp, hipStream_t s) {
  int nb = (n + SCAN_TILE - 1) / SCAN_TILE;
  hipLaunchKernelGGL(k_scan_tile, dim3(nb), dim3(SCAN_THREADS), 0, s, in, out, n, tmp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nb <= 1) return e;
  int32_t* next = tmp + align256((size_t)nb * 4) / 4;
  e = scan_exclusive(tmp, tmp, nb, next, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scan_add, dim3(nb), dim3(SCAN_THREADS), 0, s, out, n, (const int32_t*)tmp);
  return hipGetLastError();
}

// bin_start[k] = number of sorted keys < k, for k in [0, nbins].
__global__ void k_bin_bounds(const uint32_t* __restrict__ skeys, int np, int nbins, int32_t* __restrict__ bin_start) {
  int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k > nbins) return;
  int lo = 0, hi = np;
  while (lo < hi) {
    int mid = lo + ((hi - lo) >> 1);
    if (skeys[mid] < (uint32_t)k)
      lo = mid + 1;
    else
      hi = mid;
  }
  bin_start[k] = lo;
}

__global__ void k_fill_i32(int32_t* p, int n, int v) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

static int digit_passes(int64_t nbins) {
  int bits = 0;
  while (bits < 32 && ((uint64_t)(nbins - 1) >> bits) != 0) ++bits;
  if (bits == 0) bits = 1;
  return (bits + 7) / 8;
}

struct BinWs {
  uint32_t* keysA;
  uint32_t* keysB;
  int32_t* vtmp;
  int32_t* ghist;
  int32_t* scan_tmp;
  size_t bytes;
};

static BinWs bin_layout(void* base, int64_t np, int64_t nbins) {
  (void)nbins;
  BinWs w;
  size_t off = 0;
  char* b = (char*)base;
  size_t nblocks = (size_t)((np + RS_TILE - 1) / RS_TILE);
  size_t nh = 256 * (nblocks > 0 ? nblocks : 1);
  w.keysA = (uint32_t*)(b + off);
  off += align256((size_t)np * 4);
  w.keysB = (uint32_t*)(b + off);
  off += align256((size_t)np * 4);
  w.vtmp = (int32_t*)(b + off);
  off += align256((size_t)np * 4);
  w.ghist = (int32_t*)(b + off);
  off += align256(nh * 4);
  w.scan_tmp = (int32_t*)(b + off);
  off += align256(scan_tmp_ints(nh) * 4);
  w.bytes = off;
  return w;
}

size_t bin_workspace_bytes(int64_t np, int64_t nbins) { return bin_layout(nullptr, np, nbins).bytes; }

template <typename T>
static hipError_t keys_t(const GridDev& g, int order, const void* pos, int np, uint32_t* keys, hipStream_t s) {
  dim3 grid((np + 255) / 256), block(256);
  if (order == 1)
    hipLaunchKernelGGL((k_keys<T, 1>), grid, block, 0, s, g, (const T*)pos, np, keys);
  else
    hipLaunchKernelGGL((k_keys<T, 2>), grid, block, 0, s, g, (const T*)pos, np, keys);
  return hipGetLastError();
}

hipError_t launch_bin(const GridDev& g, int order, bool f32, const void* pos, int np, int nbins, int32_t* bin_start,
                      int32_t* perm, void* ws, hipStream_t s) {
  if (np == 0) {
    hipLaunchKernelGGL(k_fill_i32, dim3((nbins + 1 + 255) / 256), dim3(256), 0, s, bin_start, nbins + 1, 0);
    return hipGetLastError();
  }
  BinWs w = bin_layout(ws, np, nbins);
  hipError_t e = f32 ? keys_t<float>(g, order, pos, np, w.keysA, s) : keys_t<double>(g, order, pos, np, w.keysA, s);
  if (e != hipSuccess) return e;
  const int passes = digit_passes(nbins);
  const int nblocks = (np + RS_TILE - 1) / RS_TILE;
  const int nh = 256 * nblocks;
  uint32_t* kin = w.keysA;
  uint32_t* kout = w.keysB;
  const int32_t* vin = nullptr;
  for (int p = 0; p < passes; ++p) {
    int32_t* vout = ((passes - 1 - p) % 2 == 0) ? perm : w.vtmp;
    hipLaunchKernelGGL(k_radix_hist, dim3(nblocks), dim3(RS_THREADS), 0, s, (const uint32_t*)kin, np, 8 * p, w.ghist,
                       nblocks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = scan_exclusive(w.ghist, w.ghist, nh, w.scan_tmp, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_radix_scatter, dim3(nblocks), dim3(RS_THREADS), 0, s, (const uint32_t*)kin, vin, np, 8 * p,
                       (const int32_t*)w.ghist, nblocks, kout, vout);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    vin = vout;
    uint32_t* t = kin;
    kin = kout;
    kout = t;
  }
  hipLaunchKernelGGL(k_bin_bounds, dim3((nbins + 1 + 255) / 256), dim3(256), 0, s, (const uint32_t*)kin, np, nbins,
                     bin_start);
  return hipGetLastError();
}

}  // namespace mmk
