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
// Pipeline (all on the caller's stream), 8-bit digits, npass = ceil(bits/8):
//   k_keys_hist   key[p] = first support node of particle p, and per tile of
//                 2048 particles the counts of the first digit
//   per pass d:   k_hist (d > 0: per-tile counts of digit d in the order the
//                 previous pass left), k_scan_cols (exclusive scan of each
//                 digit's column over the tiles, plus the column totals),
//                 k_scatter (stable in-tile ranks: each wave ranks its 512
//                 particles in index order with wave-private digit counters;
//                 position = digit base + tile prefix + wave prefix + rank)
//   k_bounds      bin_start[k] = first sorted position whose key is >= k
//
// Particles already stored in key order (e.g. cell by cell for CIC) are
// detected on the device: k_keys_hist records per tile whether a key is below
// its predecessor's and, for a tile in order, already writes its part of the
// identity permutation and of bin_start. The first k_scan_cols reduces the
// tile records into one flag; while it is clear the digit passes and k_bounds
// return at once. Every flag is written before it is read in the same call,
// so the workspace needs no initialisation. The result is the same unique
// stable order either way.
#include "mm_internal.h"

namespace mmk {

namespace {

constexpr int BT = 256;                // threads per block
constexpr int BI = 8;                  // items per thread
constexpr int TILE = BT * BI;          // particles per tile
constexpr int NWV = BT / 64;           // waves per block
constexpr int WITEMS = TILE / NWV;     // particles per wave in the scatter

__device__ __forceinline__ unsigned long long lanemask_lt() { return __lanemask_lt(); }

// Tile of this block in the per-tile kernels (one block per tile). The digit
// counts are stored column by column (ghist[digit][tile]), so every tile
// writes, and the scatter reads, one value in each of 256 columns; chunks of
// 32 consecutive tiles on one XCD let its L2 gather those values into whole
// lines (dealt round the XCDs, tiles are spread one per XCD and every column
// value went to memory as a partial line).
__device__ __forceinline__ int tile_of_block() { return xcd_chunk_remap(blockIdx.x, gridDim.x, 32); }

// Lanes of the wave whose 8-bit digit equals this lane's (among `valid` lanes).
__device__ __forceinline__ unsigned long long match_digit(int d, bool valid) {
  unsigned long long peers = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (d >> b) & 1;
    const unsigned long long m = __ballot(valid && bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

}  // namespace

// Adds this wave's digits to the LDS histogram h. Consecutive lanes hold
// consecutive particles and the valid lanes are a prefix of the wave, so equal
// digits of a cell-sorted input form runs; each run is one LDS atomic.
__device__ __forceinline__ void count_digit_runs(int* h, int d, bool valid, int lane) {
  const int end = __popcll(__ballot(valid));
  const int dprev = __shfl_up(d, 1);
  const bool head = valid && (lane == 0 || d != dprev);
  const unsigned long long heads = __ballot(head);
  if (head) {
    const unsigned long long after = lane == 63 ? 0ull : (heads >> (lane + 1));
    const int next = after ? lane + 1 + __ffsll((long long)after) - 1 : end;
    atomicAdd(&h[d], next - lane);
  }
}

// Keys, and per tile of TILE particles the counts of the first digit. The
// positions of KB items per thread are loaded before any is processed. A
// descent (key below the previous particle's key) is found inside a wave by a
// shuffle, across waves and items through the first and last key of each
// wave's run of 64, and across tiles by recomputing the key of the particle
// before the tile; tile_unsorted[tile] records it. A tile without a descent
// writes perm[p] = p and bin_start[k] = p for k in (key[p-1], key[p]] (the
// tail up to nbins from the last particle): the final values when the whole
// input is in key order, and overwritten by the digit passes and k_bounds
// otherwise.
// T: arithmetic of the key; PT: type of the stored positions (T, or fp32 read into fp64).
template <typename T, int R, typename PT>
__global__ __launch_bounds__(BT) void k_keys_hist(GridDev g, const PT* __restrict__ pos, int64_t ps, int np, int nbins,
                                                  uint32_t* __restrict__ keys, int32_t* __restrict__ ghist,
                                                  int ntiles, int32_t* __restrict__ tile_unsorted,
                                                  int32_t* __restrict__ bin_start, int32_t* __restrict__ perm) {
  static_assert(BI == 8, "one batch of KB = BI loads per thread");
  constexpr int KB = 8;
  __shared__ int h[256];
  __shared__ uint32_t kfirst[BI][NWV], klast[BI][NWV];
  __shared__ int kbefore;  // key of the particle before the tile (-1 for the first tile)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  h[tid] = 0;
  __syncthreads();
  const int tile = tile_of_block();
  const size_t base = (size_t)tile * TILE;
  bool desc = false;
  uint32_t kv[BI];
  {
    T x[KB][3];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      size_t idx = base + (size_t)i * BT + tid;
      idx = idx < (size_t)np ? idx : (size_t)np - 1;  // clamped: loads are unconditional
#pragma unroll
      for (int d = 0; d < 3; ++d) x[i][d] = (T)pos[ps * idx + d];
    }
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const size_t idx = base + (size_t)i * BT + tid;
      const bool valid = idx < (size_t)np;
      const uint32_t key = (uint32_t)particle_key<R>(x[i], g);
      kv[i] = key;
      if (valid) keys[idx] = key;
      count_digit_runs(h, (int)(key & 255u), valid, lane);
      const uint32_t kprev = __shfl_up(key, 1);
      desc |= valid && lane > 0 && key < kprev;
      if (lane == 0) kfirst[i][wave] = key;
      if (lane == 63) klast[i][wave] = key;
    }
  }
  if (tid == 0) {  // key of the last particle of the previous tile
    int kb = -1;
    if (base > 0) {
      const size_t pb = ps * (base - 1);
      const T xb[3] = {(T)pos[pb], (T)pos[pb + 1], (T)pos[pb + 2]};
      kb = particle_key<R>(xb, g);
    }
    kbefore = kb;
  }
  __syncthreads();
  if (tid < BI * NWV) {  // first particle of each wave's run of 64 against its predecessor
    const int i = tid / NWV, wv = tid - i * NWV;
    const size_t idx = base + (size_t)i * BT + 64 * wv;
    if (idx < (size_t)np && idx > 0) {
      uint32_t prev;
      if (wv > 0)
        prev = klast[i][wv - 1];
      else if (i > 0)
        prev = klast[i - 1][NWV - 1];
      else
        prev = (uint32_t)kbefore;
      desc |= kfirst[i][wv] < prev;
    }
  }
  const bool tile_desc = __syncthreads_or(desc);
  if (tid == 0) tile_unsorted[tile] = tile_desc ? 1 : 0;
  ghist[(size_t)tid * ntiles + tile] = h[tid];
  if (tile_desc) return;
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const size_t idx = base + (size_t)i * BT + tid;
    const uint32_t up = __shfl_up(kv[i], 1);
    if (idx >= (size_t)np) continue;
    int lo;
    if (lane > 0)
      lo = (int)up;
    else if (wave > 0)
      lo = (int)klast[i][wave - 1];
    else if (i > 0)
      lo = (int)klast[i - 1][NWV - 1];
    else
      lo = kbefore;
    perm[idx] = (int32_t)idx;
    const int hi = (int)kv[i] < nbins ? (int)kv[i] : nbins;
    for (int k = lo + 1; k <= hi; ++k) bin_start[k] = (int32_t)idx;
    if (idx == (size_t)np - 1)
      for (int k = hi + 1; k <= nbins; ++k) bin_start[k] = np;
  }
}

// Per-tile counts of the digit at `shift` of keys in their current order.
__global__ __launch_bounds__(BT) void k_hist(const uint32_t* __restrict__ keys, int np, int shift,
                                             int32_t* __restrict__ ghist, int ntiles,
                                             const int32_t* __restrict__ unsorted) {
  __shared__ int h[256];
  if (*unsorted == 0) return;  // already in key order
  const int tid = threadIdx.x, lane = tid & 63;
  h[tid] = 0;
  const int tile = tile_of_block();
  const size_t base = (size_t)tile * TILE;
  uint32_t kk[BI];
#pragma unroll
  for (int it = 0; it < BI; ++it) {
    const size_t idx = base + (size_t)it * BT + tid;
    kk[it] = keys[idx < (size_t)np ? idx : (size_t)np - 1];
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < BI; ++it) {
    const size_t idx = base + (size_t)it * BT + tid;
    count_digit_runs(h, (int)((kk[it] >> shift) & 255u), idx < (size_t)np, lane);
  }
  __syncthreads();
  ghist[(size_t)tid * ntiles + tile] = h[tid];
}

// One block per digit column: exclusive scan over the tiles in place, column
// total to totals[digit]. In the first pass (tile_unsorted != NULL) every
// block reduces the per-tile descent records itself and block 0 stores the
// result in *unsorted for the kernels after it. With one block per column
// the latency of each round of loads is exposed, so the loads are
// unconditional (clamped indices; np > 0, so ntiles >= 1), the column is
// taken in batches of SB chunks of 2048 tiles loaded before any is scanned,
// and the first batch is in flight while the order flag is found (in key
// order the values are then not used).
__global__ __launch_bounds__(256) void k_scan_cols(int32_t* __restrict__ ghist, int ntiles,
                                                   int32_t* __restrict__ totals,
                                                   const int32_t* __restrict__ tile_unsorted,
                                                   int32_t* __restrict__ unsorted) {
  constexpr int SI = 8, SB = 4;  // tiles per thread per chunk, chunks per batch
  __shared__ int wsum[SB][4];
  const int col = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* c = ghist + (size_t)col * ntiles;
  int v[SB][SI];
  auto load_batch = [&](int b0) {
#pragma unroll
    for (int k = 0; k < SB; ++k) {
#pragma unroll
      for (int i = 0; i < SI; ++i) {
        const int idx = b0 + k * 256 * SI + tid * SI + i;
        const int x = c[idx < ntiles ? idx : ntiles - 1];
        v[k][i] = idx < ntiles ? x : 0;
      }
    }
  };
  load_batch(0);
  if (tile_unsorted) {
    bool any = false;
    for (int t0 = 0; t0 < ntiles; t0 += 256 * 8) {
      int f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = t0 + i * 256 + tid;
        f[i] = tile_unsorted[t < ntiles ? t : ntiles - 1];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) any |= f[i] != 0;  // a clamped index repeats a real tile's record
    }
    any = __syncthreads_or(any);
    if (col == 0 && tid == 0) *unsorted = any ? 1 : 0;
    if (!any) return;  // already in key order
  } else if (*unsorted == 0) {
    return;
  }
  int carry = 0;
  for (int b0 = 0; b0 < ntiles; b0 += 256 * SI * SB) {
    if (b0 > 0) load_batch(b0);
    int run[SB], incl[SB];
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      run[k] = 0;
#pragma unroll
      for (int i = 0; i < SI; ++i) run[k] += v[k][i];
      incl[k] = run[k];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl[k], off);
        if (lane >= off) incl[k] += y;
      }
      if (lane == 63) wsum[k][wave] = incl[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      int wbase = 0, total = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (w < wave) wbase += wsum[k][w];
        total += wsum[k][w];
      }
      int excl = carry + wbase + incl[k] - run[k];
#pragma unroll
      for (int i = 0; i < SI; ++i) {
        const int idx = b0 + k * 256 * SI + tid * SI + i;
        if (idx < ntiles) c[idx] = excl;
        excl += v[k][i];
      }
      carry += total;
    }
    __syncthreads();
  }
  if (tid == 0) totals[col] = carry;
}

// Stable scatter of one 8-bit digit pass. vals_in == NULL means the identity.
__global__ __launch_bounds__(BT) void k_scatter(const uint32_t* __restrict__ keys_in,
                                                const int32_t* __restrict__ vals_in, int np, int shift,
                                                const int32_t* __restrict__ ghist, const int32_t* __restrict__ totals,
                                                int ntiles, uint32_t* __restrict__ keys_out,
                                                int32_t* __restrict__ vals_out, const int32_t* __restrict__ unsorted) {
  __shared__ int wcnt[NWV][256];
  if (*unsorted == 0) return;  // already in key order
  __shared__ int wpre[NWV][256];
  __shared__ int dsum[4];
  __shared__ int doff[256];          // global position minus tile-local position, per digit
  __shared__ uint32_t sk[TILE];      // the tile's keys and values in digit order
  __shared__ int32_t sv[TILE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = tile_of_block();

  // digit base of this tile: exclusive prefix of the pass totals over digits
  // plus this tile's prefix within the digit's column
  const int tot = totals[tid];
  int incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) dsum[wave] = incl;
#pragma unroll
  for (int w = 0; w < NWV; ++w) wcnt[w][tid] = 0;
  __syncthreads();
  int dbase = incl - tot;
  for (int w = 0; w < wave; ++w) dbase += dsum[w];
  dbase += ghist[(size_t)tid * ntiles + tile];

  // rank this wave's particles in index order
  const size_t base = (size_t)tile * TILE + (size_t)wave * WITEMS;
  const unsigned long long lt = lanemask_lt();
  uint32_t k[BI];
  int32_t v[BI];
  int rk[BI];
#pragma unroll
  for (int r = 0; r < BI; ++r) {  // loads first (clamped index, unconditional)
    const size_t idx = base + (size_t)r * 64 + lane;
    const size_t ci = idx < (size_t)np ? idx : (size_t)np - 1;
    k[r] = keys_in[ci];
    v[r] = vals_in ? vals_in[ci] : (int32_t)idx;
  }
#pragma unroll
  for (int r = 0; r < BI; ++r) {
    // rank = number of this wave's earlier particles with the same digit.
    // The leader of each digit's lanes adds their count to the wave's counter
    // with an LDS fetch-and-add (a wave's LDS atomics complete in order, so
    // the returned value is the count of earlier rounds) and shares it.
    const size_t idx = base + (size_t)r * 64 + lane;
    const bool valid = idx < (size_t)np;  // valid lanes are a prefix of the wave
    const int d = (int)((k[r] >> shift) & 255u);
    const int dprev = __shfl_up(d, 1);
    const int end = __popcll(__ballot(valid));  // all lanes active here: the ballot sees every lane
    int rank, leader, cnt;
    if (__ballot(valid && lane > 0 && d < dprev) == 0) {
      // digits never decrease across the wave (cell-sorted input): each digit
      // is one run of lanes, ranked by position in the run
      const unsigned long long heads = __ballot(valid && (lane == 0 || d != dprev));
      leader = 63 - __clzll(heads & (lt | (1ull << lane)));
      rank = lane - leader;
      const unsigned long long after = lane == 63 ? 0ull : (heads >> (lane + 1));
      cnt = after ? __ffsll((long long)after) : end - lane;
    } else {
      const unsigned long long peers = match_digit(d, valid);
      rank = __popcll(peers & lt);
      leader = __ffsll((long long)peers) - 1;
      cnt = __popcll(peers);
    }
    int old = 0;
    if (valid && rank == 0) old = atomicAdd(&wcnt[wave][d], cnt);
    const int first = __shfl(old, leader < 0 ? 0 : leader);
    rk[r] = valid ? first + rank : -1;
  }
  __syncthreads();
  // Tile-local position of (wave, digit tid): the tile's count of smaller
  // digits plus the counts of digit tid in earlier waves. Where the tile's
  // digits form short runs (fewer than 16 particles per digit on average, as
  // for shuffled input), the particles are placed in LDS in that order and
  // written out by consecutive threads, so that each digit's run is one
  // contiguous stretch of stores. Longer runs are already contiguous enough
  // in the direct stores, and the LDS pass would only add to them.
  const size_t t0 = (size_t)tile * TILE;
  const int nvalid = (size_t)np - t0 < (size_t)TILE ? (int)((size_t)np - t0) : TILE;
  int cnt_d = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) cnt_d += wcnt[w][tid];
  const bool staged = __syncthreads_count(cnt_d > 0) * 16 > nvalid;  // block-uniform
  // wpre[w][d]: output position (direct stores) or tile-local position
  // (staged) of wave w's first particle with digit d
  int run = dbase;
  if (staged) {
    int inc = cnt_d;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(inc, off);
      if (lane >= off) inc += y;
    }
    if (lane == 63) dsum[wave] = inc;  // every thread read dsum for dbase before the barriers above
    __syncthreads();
    int lbase = inc - cnt_d;
    for (int w = 0; w < wave; ++w) lbase += dsum[w];
    doff[tid] = dbase - lbase;
    run = lbase;
  }
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    wpre[w][tid] = run;
    run += wcnt[w][tid];
  }
  __syncthreads();
  if (!staged) {
#pragma unroll
    for (int r = 0; r < BI; ++r) {
      if (rk[r] >= 0) {
        const int d = (int)((k[r] >> shift) & 255u);
        const int dst = wpre[wave][d] + rk[r];
        if ((unsigned)dst < (unsigned)np) {  // always true for consistent inputs; guards the writes
          keys_out[dst] = k[r];
          vals_out[dst] = v[r];
        }
      }
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < BI; ++r) {
    if (rk[r] >= 0) {
      const int d = (int)((k[r] >> shift) & 255u);
      const int lp = wpre[wave][d] + rk[r];
      if ((unsigned)lp < (unsigned)TILE) {  // always true for consistent inputs; guards the LDS
        sk[lp] = k[r];
        sv[lp] = v[r];
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < BI; ++r) {
    const int i = r * BT + tid;
    if (i < nvalid) {
      const uint32_t kk = sk[i];
      const int dst = doff[(kk >> shift) & 255u] + i;
      if ((unsigned)dst < (unsigned)np) {  // always true for consistent inputs; guards the writes
        keys_out[dst] = kk;
        vals_out[dst] = sv[i];
      }
    }
  }
}

// bin_start[k] = lower bound of k in the sorted keys, for k in [0, nbins]:
// thread i (0 <= i <= np) writes i for every k in (skeys[i-1], skeys[i]]
// (with skeys[-1] = -1 and skeys[np] = nbins), so each entry is written once.
// Input already in key order: k_keys_hist has written bin_start and perm.
// Grid-stride over i = 0..np with a capped grid, so that the launch is cheap
// when the input was already in key order; the keys of UB strides are loaded
// before any is used, so that UB loads per thread are in flight at once.
__global__ void k_bounds(const uint32_t* __restrict__ skeys, int np, int nbins, int32_t* __restrict__ bin_start,
                         const int32_t* __restrict__ unsorted) {
  if (*unsorted == 0) return;
  constexpr int UB = 4;
  const int stride = gridDim.x * blockDim.x;
  // 64-bit counter: with np just below 2^31 the last strides pass INT_MAX
  for (long long i0 = (long long)blockIdx.x * blockDim.x + threadIdx.x; i0 <= np; i0 += (long long)UB * stride) {
    int lo[UB], hi[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const long long i = i0 + (long long)u * stride;
      lo[u] = -1;
      hi[u] = -1;  // no entry for i beyond np
      if (i <= np) {
        lo[u] = i == 0 ? -1 : (int)skeys[i - 1];
        hi[u] = i == np ? nbins : (int)skeys[i];
      }
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int i = (int)(i0 + (long long)u * stride);  // used only where i <= np
      const int h = hi[u] > nbins ? nbins : hi[u];
      for (int k = lo[u] + 1; k <= h; ++k) bin_start[k] = i;
    }
  }
}

__global__ void k_fill_i32(int32_t* p, int n, int v) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

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
  int32_t* totals;
  int32_t* tile_unsorted;  // per tile: some key is below its predecessor's
  int32_t* unsorted;       // the same over all tiles
  size_t bytes;
};

static BinWs bin_layout(void* base, int64_t np, int64_t nbins) {
  BinWs w;
  size_t off = 0;
  char* b = (char*)base;
  (void)nbins;
  const size_t ntiles = (size_t)((np + TILE - 1) / TILE);
  w.keysA = (uint32_t*)(b + off);
  off += align256((size_t)np * 4);
  w.keysB = (uint32_t*)(b + off);
  off += align256((size_t)np * 4);
  w.vtmp = (int32_t*)(b + off);
  off += align256((size_t)np * 4);
  w.ghist = (int32_t*)(b + off);
  off += align256((size_t)256 * (ntiles > 0 ? ntiles : 1) * 4);
  w.totals = (int32_t*)(b + off);
  off += align256((size_t)256 * 4);
  w.tile_unsorted = (int32_t*)(b + off);
  off += align256((ntiles > 0 ? ntiles : 1) * 4);
  w.unsorted = (int32_t*)(b + off);
  off += 256;
  w.bytes = off;
  return w;
}

size_t bin_workspace_bytes(int64_t np, int64_t nbins) { return bin_layout(nullptr, np, nbins).bytes; }

template <typename T, typename PT>
static hipError_t keys_t(const GridDev& g, int order, const void* pos, int64_t ps, int np, int nbins, const BinWs& w,
                         int ntiles, int32_t* bin_start, int32_t* perm, hipStream_t s) {
  if (order == 1)
    hipLaunchKernelGGL((k_keys_hist<T, 1, PT>), dim3(ntiles), dim3(BT), 0, s, g, (const PT*)pos, ps, np, nbins,
                       w.keysA, w.ghist, ntiles, w.tile_unsorted, bin_start, perm);
  else
    hipLaunchKernelGGL((k_keys_hist<T, 2, PT>), dim3(ntiles), dim3(BT), 0, s, g, (const PT*)pos, ps, np, nbins,
                       w.keysA, w.ghist, ntiles, w.tile_unsorted, bin_start, perm);
  return hipGetLastError();
}

hipError_t launch_bin(const GridDev& g, int order, bool f32, const void* pos, int np, int nbins, int32_t* bin_start,
                      int32_t* perm, void* ws, hipStream_t s, bool pos32, int64_t ps) {
  if (np == 0) {
    hipLaunchKernelGGL(k_fill_i32, dim3((nbins + 1 + 255) / 256), dim3(256), 0, s, bin_start, nbins + 1, 0);
    return hipGetLastError();
  }
  BinWs w = bin_layout(ws, np, nbins);
  const int npass = digit_passes(nbins);
  const int ntiles = (np + TILE - 1) / TILE;
  // fp32 positions (MM_F32 and the mixed layout) are read exactly into fp64:
  // the key is found in fp64 arithmetic, as every kernel finds the support
  hipError_t e = (f32 || pos32) ? keys_t<double, float>(g, order, pos, ps, np, nbins, w, ntiles, bin_start, perm, s)
                                : keys_t<double, double>(g, order, pos, ps, np, nbins, w, ntiles, bin_start, perm, s);
  if (e != hipSuccess) return e;
  uint32_t* kin = w.keysA;
  uint32_t* kout = w.keysB;
  const int32_t* vin = nullptr;
  for (int p = 0; p < npass; ++p) {
    if (p > 0) {
      hipLaunchKernelGGL(k_hist, dim3(ntiles), dim3(BT), 0, s, (const uint32_t*)kin, np, 8 * p, w.ghist, ntiles,
                         (const int32_t*)w.unsorted);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_scan_cols, dim3(256), dim3(256), 0, s, w.ghist, ntiles, w.totals,
                       p == 0 ? (const int32_t*)w.tile_unsorted : nullptr, w.unsorted);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    int32_t* vout = ((npass - 1 - p) % 2 == 0) ? perm : w.vtmp;
    hipLaunchKernelGGL(k_scatter, dim3(ntiles), dim3(BT), 0, s, (const uint32_t*)kin, vin, np, 8 * p,
                       (const int32_t*)w.ghist, (const int32_t*)w.totals, ntiles, kout, vout,
                       (const int32_t*)w.unsorted);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    vin = vout;
    uint32_t* t = kin;
    kin = kout;
    kout = t;
  }
  const size_t nbb = ((size_t)np + 256) / 256;  // blocks for np + 1 threads
  const int bblocks = nbb < 2048 ? (int)nbb : 2048;
  hipLaunchKernelGGL(k_bounds, dim3(bblocks), dim3(256), 0, s, (const uint32_t*)kin, np, nbins,
                     bin_start, (const int32_t*)w.unsorted);
  return hipGetLastError();
}

}  // namespace mmk
