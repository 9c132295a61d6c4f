// Per-bin matrix-core contraction of the mass matrix (gfx950 MFMA), phase 1.
//
// Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for Implicit
// Particle-In-Cell Methods": within one support group (one bin of particles
// sharing their first support node, Sec. 3.3) the local matrix is
//   Mhat^{c}_{ab} = sum_p t_p^c W_pa W_pb            (Sec. 3.1, Eq. 15)
// i.e. A^c B with A^c = W diag(t^c), B = W^T (Sec. 3.1, Eq. 14), evaluated as
// batched products whose inner dimension is a batch of particles (Sec. 3.2)
// and using the spatial symmetry Mhat_ab = Mhat_ba to skip the lower
// off-diagonal tile (Table 1). t^c = sigma w_p alpha_p^c (Eq. 6).
//
// Wave organisation (one wave owns a bin at a time, persistent over bins):
//  * particle preparation runs one particle per lane: 64 particles are loaded
//    with one gather each, their support weights W_a (Eq. 12) and
//    coefficients t^c are computed once and staged in LDS columns;
//  * the matrix instructions then read their operands from LDS:
//    CIC fp64 - v_mfma_f64_4x4x4, 4 blocks; the 8 support rows split by az into
//      two halves (quadrants Q00, Q01, Q11; Q10 = Q01^T); one instruction is one
//      (component, quadrant) product for four different 4-particle batches
//      (block = batch), so no block is padded; the 4 block partials are summed
//      across lanes once per bin. 16 particles per round.
//    CIC fp32 - v_mfma_f32_4x4x1, 16 blocks, one particle per block.
//    TSC      - (scalar, fp32 and the atomic mode; fp64 ECSIM records: k_tsc64.hip)
//      27 rows padded to 32, tiles (0,0), (0,1), (1,1) of
//      v_mfma_{f64,f32}_16x16x4, 4 particles per batch.
//  * the next chunk's particle index and data are fetched while the current
//    chunk computes.
//
// Output of a bin (MODE):
//  MODE_RECORD - the upper triangle (a <= b) of the local matrix is written as
//    one compact record rec[bin][pair(a,b)][comp], assembled in the wave's LDS
//    region and stored with coalesced 8-byte stores; a second kernel
//    (k_gather) sums records into the stencil matrix (deterministic, every
//    output entry written once, no atomics);
//  MODE_ATOMIC - every local entry is added into the stencil matrix with a
//    hardware atomic ((a,b) and (b,a) for off-diagonal tiles).
#include "mm_contract.h"
#include "mm_run.h"

namespace mmk {

template <int R>
struct Geo {
  static constexpr int NS = R + 1;
  static constexpr int N = NS * NS * NS;
  static constexpr int NPAIR = N * (N + 1) / 2;
  static constexpr int NO = 2 * R + 1;
  static constexpr int NOFF = NO * NO * NO;
};

// Row stride (elements) of the staged weights sW[a][lane]. The rounds read 16
// rows at one column: a stride of 64 would put those 16 reads on one LDS bank;
// 68 spreads them (fp32: 4 i + k covers all 64 banks for 16 rows x 4 columns),
// and the staging stores (one column per lane) stay conflict-free.
constexpr int SWS = 68;

// The fp64 scalar order-2 kernel stages the 3 + 3 + 3 one-dimensional
// weights of each particle (sW[3 d + k][lane], axis d) instead of the 27
// products, and forms W_a = (wx wy) wz in the rounds: 9 instead of 27 staged
// rows per wave, so that the registers rather than the LDS bound the waves
// per SIMD (5 instead of 2; contraction 12% faster on 32^3 cells x 64). In
// fp32 the LDS did not bound them, and the extra products cost 5%.
template <typename T, int R, int NC>
constexpr bool stage_1d() {
  return R == 2 && NC == 1 && sizeof(T) == 8;
}
template <typename T, int R, int NC>
constexpr int staged_rows() {
  return stage_1d<T, R, NC>() ? 9 : Geo<R>::N;
}

// Position of the pair (a, b), a <= b, in the packed upper triangle.
template <int N>
__device__ __forceinline__ int pair_index(int a, int b) {
  return a * N - (a * (a - 1)) / 2 + (b - a);
}

__device__ __forceinline__ size_t support_node(int fx, int fy, int fz, int ax, int ay, int az, const GridDev& g) {
  int x = fx + ax, y = fy + ay, z = fz + az;
  x = x >= g.n0 ? x - g.n0 : x;
  y = y >= g.n1 ? y - g.n1 : y;
  z = z >= g.n2 ? z - g.n2 : z;
  return (size_t)x + (size_t)g.n0 * ((size_t)y + (size_t)g.n1 * (size_t)z);
}

// Bin output for local entry (a, b) of component c (value v). Records are
// assembled in the wave's LDS region `lds` ([pair][comp], the layout of one
// bin's record) and leave with coalesced stores (store_record).
template <typename T, int R, int NC, int MODE>
struct Sink {
  T* out;
  int bin, fx, fy, fz;
  GridDev g;
  T* lds;
  __device__ __forceinline__ void atomic_entry(int a, int b, int c, T v) const {
    constexpr int NS = Geo<R>::NS, NO = Geo<R>::NO, NOFF = Geo<R>::NOFF;
    int ax = a % NS, ay = (a / NS) % NS, az = a / (NS * NS);
    int bx = b % NS, by = (b / NS) % NS, bz = b / (NS * NS);
    size_t node = support_node(fx, fy, fz, ax, ay, az, g);
    int o = (bx - ax + R) + NO * ((by - ay + R) + NO * (bz - az + R));
    atomic_add(out + (node * NOFF + o) * NC + c, v);
  }
  // Diagonal-tile entry: stored once as (a,b) with a <= b (record) or added as is (atomic).
  __device__ __forceinline__ void diag_tile(int a, int b, int c, T v) const {
    if (MODE == MODE_RECORD) {
      if (a <= b) lds[pair_index<Geo<R>::N>(a, b) * NC + c] = v;
    } else {
      atomic_entry(a, b, c, v);
    }
  }
  // Off-diagonal-tile entry with a < b: stands for both (a,b) and (b,a).
  __device__ __forceinline__ void off_tile(int a, int b, int c, T v) const {
    if (MODE == MODE_RECORD) {
      lds[pair_index<Geo<R>::N>(a, b) * NC + c] = v;
    } else {
      atomic_entry(a, b, c, v);
      atomic_entry(b, a, c, v);
    }
  }
  // The bin's record, complete in LDS, to rec[bin] in 8-byte units (every
  // record length is a multiple of 8 bytes and the records start 256-byte
  // aligned). The wave is alone on its LDS region, and its LDS accesses are
  // performed in program order, so no barrier is needed.
  __device__ __forceinline__ void store_record(int lane) const {
    constexpr int LEN = Geo<R>::NPAIR * NC;
    static_assert((LEN * sizeof(T)) % 8 == 0, "record of whole 8-byte units");
    constexpr int N8 = LEN * (int)sizeof(T) / 8;
    const uint2* src = reinterpret_cast<const uint2*>(lds);
    uint2* dst = reinterpret_cast<uint2*>(out + (size_t)bin * LEN);
    for (int i = lane; i < N8; i += 64) dst[i] = src[i];
  }
};

// Raw data of the particle a lane prepares.
template <typename T>
struct Raw {
  T x, y, z, w, bx, by, bz;
  bool valid;
};

// PT: type of the stored positions and field (T, or fp32 read into fp64).
template <typename T, typename PT, int NC>
__device__ __forceinline__ Raw<T> load_raw(const PT* __restrict__ pos, const T* __restrict__ w,
                                           const PT* __restrict__ Bf, int p, int np) {
  Raw<T> r;
  r.valid = (unsigned)p < (unsigned)np;
  r.x = r.y = r.z = r.w = r.bx = r.by = r.bz = T(0);
  if (r.valid) {
    r.x = pos[3 * (size_t)p];
    r.y = pos[3 * (size_t)p + 1];
    r.z = pos[3 * (size_t)p + 2];
    r.w = w[p];
    if (NC == 9) {
      r.bx = Bf[3 * (size_t)p];
      r.by = Bf[3 * (size_t)p + 1];
      r.bz = Bf[3 * (size_t)p + 2];
    }
  }
  return r;
}

// One particle per lane: weights W[a] (a = ax + NS*(ay + NS*az)) into sW[a * SWS + lane]
// (or the one-dimensional weights, stage_1d),
// coefficients t^c into sT[c][lane]; zeros for an empty lane.
template <typename T, int R, int NC>
__device__ __forceinline__ void stage_particle(const Raw<T>& r, const GridDev& g, T beta, T sigma, T* sW, T* sT,
                                               int lane) {
  constexpr int NS = Geo<R>::NS, N = Geo<R>::N;
  T wx[3] = {0, 0, 0}, wy[3] = {0, 0, 0}, wz[3] = {0, 0, 0}, t[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) t[c] = T(0);
  if (r.valid) {
    support_axis<T, R, 0>((double)r.x, g, wx);
    support_axis<T, R, 1>((double)r.y, g, wy);
    support_axis<T, R, 2>((double)r.z, g, wz);
    T f = sigma * r.w;
    if (NC == 9)
      response<T>(r.bx, r.by, r.bz, beta, f, t);
    else
      t[0] = f;
  }
  if (stage_1d<T, R, NC>()) {
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      sW[k * SWS + lane] = wx[k];
      sW[(NS + k) * SWS + lane] = wy[k];
      sW[(2 * NS + k) * SWS + lane] = wz[k];
    }
  } else {
#pragma unroll
    for (int az = 0; az < NS; ++az)
#pragma unroll
      for (int ay = 0; ay < NS; ++ay)
#pragma unroll
        for (int ax = 0; ax < NS; ++ax) sW[(ax + NS * (ay + NS * az)) * SWS + lane] = (wx[ax] * wy[ay]) * wz[az];
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) sT[c * 64 + lane] = t[c];
  static_assert(N == NS * NS * NS, "support size");
}

// ---------------------------------------------------------------- accumulators
// CIC fp64: 3 quadrants x NC components, one double each (4x4x4, 4 blocks).
template <int NC>
struct AccCicF64 {
  double q[NC][3];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int c = 0; c < NC; ++c) q[c][0] = q[c][1] = q[c][2] = 0.0;
  }
  // Rounds of 16 particles from LDS columns [0, cnt).
  __device__ __forceinline__ void accumulate(const double* sW, const double* sT, int cnt, int lane) {
    const int slot = (lane >> 2) & 3, r4 = lane & 3, kq = lane >> 4;
    for (int r0 = 0; r0 < cnt; r0 += 16) {
      const int pl = r0 + 4 * slot + kq;
      const double wlo = sW[r4 * SWS + pl], whi = sW[(4 + r4) * SWS + pl];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const double tc = sT[c * 64 + pl];
        const double alo = tc * wlo, ahi = tc * whi;
        q[c][0] = mfma_f64_4x4x4(alo, wlo, q[c][0]);
        q[c][1] = mfma_f64_4x4x4(alo, whi, q[c][1]);
        q[c][2] = mfma_f64_4x4x4(ahi, whi, q[c][2]);
      }
    }
  }
  template <int MODE>
  __device__ __forceinline__ void finish(const Sink<double, 1, NC, MODE>& sk, int lane) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        double v = q[c][k];
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        q[c][k] = v;
      }
    // D_blk[i][j] at lane (i<<4)|(blk<<2)|j; every block lane now holds the sum.
    const int i = lane >> 4, slot = (lane >> 2) & 3, j = lane & 3;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (slot == 0) sk.diag_tile(i, j, c, q[c][0]);
      if (slot == 1) sk.off_tile(i, 4 + j, c, q[c][1]);
      if (slot == 2) sk.diag_tile(4 + i, 4 + j, c, q[c][2]);
    }
  }
};

// CIC fp32: 3 quadrants x NC components, 4 floats each (4x4x1, 16 blocks).
template <int NC>
struct AccCicF32 {
  v4f q[NC][3];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int k = 0; k < 3; ++k) q[c][k] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void accumulate(const float* sW, const float* sT, int cnt, int lane) {
    const int blk = lane >> 2, r4 = lane & 3;
    for (int r0 = 0; r0 < cnt; r0 += 16) {
      const int pl = r0 + blk;
      const float wlo = sW[r4 * SWS + pl], whi = sW[(4 + r4) * SWS + pl];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float tc = sT[c * 64 + pl];
        const float alo = tc * wlo, ahi = tc * whi;
        q[c][0] = mfma_f32_4x4x1(alo, wlo, q[c][0]);
        q[c][1] = mfma_f32_4x4x1(alo, whi, q[c][1]);
        q[c][2] = mfma_f32_4x4x1(ahi, whi, q[c][2]);
      }
    }
  }
  template <int MODE>
  __device__ __forceinline__ void finish(const Sink<float, 1, NC, MODE>& sk, int lane) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = q[c][k][r];
          v += __shfl_xor(v, 4);
          v += __shfl_xor(v, 8);
          v += __shfl_xor(v, 16);
          v += __shfl_xor(v, 32);
          q[c][k][r] = v;
        }
    // D_blk[i][j] at lane 4 blk + j, register i; all blocks hold the sum.
    const int blk = lane >> 2, j = lane & 3;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (blk == 0) sk.diag_tile(i, j, c, q[c][0][i]);
        if (blk == 1) sk.off_tile(i, 4 + j, c, q[c][1][i]);
        if (blk == 2) sk.diag_tile(4 + i, 4 + j, c, q[c][2][i]);
      }
  }
};

// TSC: tiles (0,0), (0,1), (1,1) of 16x16 per component.
template <typename T>
struct TscOps;
template <>
struct TscOps<double> {
  typedef v4d V;
  static __device__ __forceinline__ V mma(double a, double b, V c) { return mfma_f64_16x16x4(a, b, c); }
  static __device__ __forceinline__ int row(int l, int r) { return 4 * r + (l >> 4); }
};
template <>
struct TscOps<float> {
  typedef v4f V;
  static __device__ __forceinline__ V mma(float a, float b, V c) { return mfma_f32_16x16x4(a, b, c); }
  static __device__ __forceinline__ int row(int l, int r) { return 4 * (l >> 4) + r; }
};

template <typename T, int NC>
struct AccTsc {
  typedef typename TscOps<T>::V V;
  V q[NC][3];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int k = 0; k < 3; ++k) q[c][k] = V{0, 0, 0, 0};
  }
  __device__ __forceinline__ void accumulate(const T* sW, const T* sT, int cnt, int lane) {
    const int i16 = lane & 15, kq = lane >> 4;
    const bool hi_ok = 16 + i16 < 27;
    // one-dimensional staging (scalar): rows of the x, y, z weights of
    // support rows i16 and 16 + i16
    constexpr bool S1 = stage_1d<T, 2, NC>();
    const int a1 = hi_ok ? 16 + i16 : 0;
    const int x0 = (i16 % 3) * SWS, y0 = (3 + (i16 / 3) % 3) * SWS, z0 = (6 + i16 / 9) * SWS;
    const int x1 = (a1 % 3) * SWS, y1 = (3 + (a1 / 3) % 3) * SWS, z1 = (6 + a1 / 9) * SWS;
    for (int b0 = 0; b0 < cnt; b0 += 4) {
      const int pl = b0 + kq;
      T w0, w1;
      if (S1) {
        w0 = (sW[x0 + pl] * sW[y0 + pl]) * sW[z0 + pl];
        w1 = hi_ok ? (sW[x1 + pl] * sW[y1 + pl]) * sW[z1 + pl] : T(0);
      } else {
        w0 = sW[i16 * SWS + pl];
        w1 = hi_ok ? sW[(16 + i16) * SWS + pl] : T(0);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const T tc = sT[c * 64 + pl];
        const T a0 = tc * w0, a1 = tc * w1;
        q[c][0] = TscOps<T>::mma(a0, w0, q[c][0]);
        q[c][1] = TscOps<T>::mma(a0, w1, q[c][1]);
        q[c][2] = TscOps<T>::mma(a1, w1, q[c][2]);
      }
    }
  }
  template <int MODE>
  __device__ __forceinline__ void finish(const Sink<T, 2, NC, MODE>& sk, int lane) {
    const int j = lane & 15;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = TscOps<T>::row(lane, r);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        sk.diag_tile(i, j, c, q[c][0][r]);
        if (16 + j < 27) sk.off_tile(i, 16 + j, c, q[c][1][r]);
        if (16 + i < 27 && 16 + j < 27) sk.diag_tile(16 + i, 16 + j, c, q[c][2][r]);
      }
    }
  }
};

template <typename T, int R, int NC>
struct AccSel;
template <int NC>
struct AccSel<double, 1, NC> {
  typedef AccCicF64<NC> A;
};
template <int NC>
struct AccSel<float, 1, NC> {
  typedef AccCicF32<NC> A;
};
template <typename T, int NC>
struct AccSel<T, 2, NC> {
  typedef AccTsc<T, NC> A;
};

// ---------------------------------------------------------------- kernel
constexpr int CT_WAVES = 4;  // waves per block; each wave works alone

// Waves per SIMD the register allocation must allow: two for the fp32
// tensorial record kernels, whose 108 fp32 accumulators otherwise leave one.
template <typename T, int NC, int MODE>
constexpr int contract_wpe() {
  return sizeof(T) == 4 && NC == 9 && MODE == MODE_RECORD ? 2 : 1;
}

template <typename T, typename PT, int R, int NC, int MODE>
__global__ __launch_bounds__(64 * CT_WAVES) __attribute__((amdgpu_waves_per_eu(contract_wpe<T, NC, MODE>())))
void k_contract(GridDev g, const PT* __restrict__ pos, const T* __restrict__ w, const PT* __restrict__ Bf,
                const int32_t* __restrict__ bin_start, const int32_t* __restrict__ perm, int np, int nbins, T beta,
                T sigma, T* __restrict__ out) {
  constexpr int N = Geo<R>::N;
  // per wave: the staged weights and coefficients, or one bin's record
  constexpr int STG = staged_rows<T, R, NC>() * SWS + NC * 64;
  constexpr int REC = MODE == MODE_RECORD ? Geo<R>::NPAIR * NC : 0;
  constexpr int WSZ = ((STG > REC ? STG : REC) + 3) & ~3;
  __shared__ __attribute__((aligned(16))) T smem[CT_WAVES][WSZ];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  T* sW = smem[wv];
  T* sT = smem[wv] + staged_rows<T, R, NC>() * SWS;
  const int nwaves = gridDim.x * CT_WAVES;
  int b = blockIdx.x * CT_WAVES + wv;
  if (b >= nbins) return;

  typename AccSel<T, R, NC>::A acc;
  acc.zero();

  int s = bin_start[b], e = bin_start[b + 1];
  s = s < 0 ? 0 : s;
  e = e > np ? np : e;
  int c0 = s;
  Raw<T> cur = load_raw<T, PT, NC>(pos, w, Bf, c0 + lane < e ? perm[c0 + lane] : -1, np);

  while (true) {
    // Next chunk: the rest of this bin, else the wave's next bin.
    int nb = b, ns = s, ne = e, nc0 = c0 + 64;
    if (nc0 >= e) {
      nb = b + nwaves;
      if (nb < nbins) {
        ns = bin_start[nb];
        ne = bin_start[nb + 1];
        ns = ns < 0 ? 0 : ns;
        ne = ne > np ? np : ne;
        nc0 = ns;
      }
    }
    const bool more = nb < nbins;
    const int pnext = (more && nc0 + lane < ne) ? perm[nc0 + lane] : -1;

    stage_particle<T, R, NC>(cur, g, beta, sigma, sW, sT, lane);
    Raw<T> nxt = load_raw<T, PT, NC>(pos, w, Bf, pnext, np);
    const int cnt = e - c0 < 64 ? (e - c0 > 0 ? e - c0 : 0) : 64;
    acc.accumulate(sW, sT, cnt, lane);

    if (c0 + 64 >= e) {  // bin complete
      const int fx = b % g.n0, fy = (b / g.n0) % g.n1, fz = b / (g.n0 * g.n1);
      Sink<T, R, NC, MODE> sk{out, b, fx, fy, fz, g, smem[wv]};
      if (MODE == MODE_RECORD || e > s) acc.template finish<MODE>(sk, lane);
      if (MODE == MODE_RECORD) sk.store_record(lane);
      acc.zero();
    }
    if (!more) break;
    b = nb;
    s = ns;
    e = ne;
    c0 = nc0;
    cur = nxt;
  }
}

template <typename T, int R, int NC, int MODE>
static hipError_t contract_launch(const GridDev& g, const Particles& P, const int32_t* bin_start,
                                  const int32_t* perm, double beta, double sigma, void* out, int waves_per_cu,
                                  hipStream_t s) {
  const int nbins = g.n0 * g.n1 * g.n2;
  int blocks = (nbins + CT_WAVES - 1) / CT_WAVES;
  int cap = 256 * waves_per_cu / CT_WAVES;
  if (blocks > cap) blocks = cap;
  if (P.pos32)  // fp32 positions and field into fp64 arithmetic
    hipLaunchKernelGGL((k_contract<T, float, R, NC, MODE>), dim3(blocks), dim3(64 * CT_WAVES), 0, s, g,
                       (const float*)P.pos, (const T*)P.w, (const float*)P.B, bin_start, perm, P.np, nbins, (T)beta,
                       (T)sigma, (T*)out);
  else
    hipLaunchKernelGGL((k_contract<T, T, R, NC, MODE>), dim3(blocks), dim3(64 * CT_WAVES), 0, s, g,
                       (const T*)P.pos, (const T*)P.w, (const T*)P.B, bin_start, perm, P.np, nbins, (T)beta,
                       (T)sigma, (T*)out);
  return hipGetLastError();
}

template <typename T, int MODE>
static hipError_t contract_t(const GridDev& g, int order, const Particles& P, const int32_t* bin_start,
                             const int32_t* perm, double beta, double sigma, void* out, hipStream_t s) {
  const bool ten = P.B != nullptr;
  // resident waves per CU that the register/LDS budget of each variant allows
  if (order == 1)
    return ten ? contract_launch<T, 1, 9, MODE>(g, P, bin_start, perm, beta, sigma, out, 16, s)
               : contract_launch<T, 1, 1, MODE>(g, P, bin_start, perm, beta, sigma, out, 32, s);
  return ten ? contract_launch<T, 2, 9, MODE>(g, P, bin_start, perm, beta, sigma, out,
                                               4 * contract_wpe<T, 9, MODE>(), s)
             : contract_launch<T, 2, 1, MODE>(g, P, bin_start, perm, beta, sigma, out,
                                              stage_1d<T, 2, 1>() ? 20 : 16, s);
}

hipError_t launch_contract(const GridDev& g, int order, bool f32, const Particles& P, const int32_t* bin_start,
                           const int32_t* perm, double beta, double sigma, int mode, void* out, hipStream_t s) {
  if (mode == MODE_RECORD && order == 1 && !f32)
    return launch_cic64(g, P, bin_start, perm, beta, sigma, (double*)out, s);
  if (P.strided()) return hipErrorInvalidValue;  // only the fp64 CIC record kernel reads strided arrays
  if (mode == MODE_RECORD && order == 1 && f32 && !P.Bgrid)
    return launch_cic32(g, P, bin_start, perm, beta, sigma, (float*)out, s);
  if (mode == MODE_RECORD && order == 2 && !f32 && (P.B || P.Bgrid))
    return launch_tsc64(g, P, bin_start, perm, beta, sigma, (double*)out, s);
  if (mode == MODE_RECORD && order == 2 && f32 && P.B && !P.Bgrid && tsc_run_records(g))
    return launch_tsc32(g, P, bin_start, perm, beta, sigma, (float*)out, s);
  if (P.Bgrid) return hipErrorInvalidValue;  // the other kernels take a per-particle field (interp first)
  if (mode == MODE_RECORD)
    return f32 ? contract_t<float, MODE_RECORD>(g, order, P, bin_start, perm, beta, sigma, out, s)
               : contract_t<double, MODE_RECORD>(g, order, P, bin_start, perm, beta, sigma, out, s);
  return f32 ? contract_t<float, MODE_ATOMIC>(g, order, P, bin_start, perm, beta, sigma, out, s)
             : contract_t<double, MODE_ATOMIC>(g, order, P, bin_start, perm, beta, sigma, out, s);
}

bool contract_planes_apply(const GridDev& g, int order, bool f32, const Particles& P) {
  if (order != 2 || !tsc_run_records(g) || P.strided()) return false;
  return f32 ? (P.B && !P.Bgrid && !P.pos32) : (P.B || P.Bgrid);
}

hipError_t launch_contract_planes(const GridDev& g, bool f32, const Particles& P, const int32_t* bin_start,
                                  const int32_t* perm, double beta, double sigma, void* rec, int z0, int z1,
                                  hipStream_t s) {
  if (!contract_planes_apply(g, 2, f32, P)) return hipErrorInvalidValue;
  return f32 ? launch_tsc32(g, P, bin_start, perm, beta, sigma, (float*)rec, s, z0, z1)
             : launch_tsc64(g, P, bin_start, perm, beta, sigma, (double*)rec, s, z0, z1);
}

bool contract_gathers_field(int order, bool f32, int mode) {
  return mode == MODE_RECORD && !f32 && (order == 1 || order == 2);  // k_cic64, k_tsc64
}

size_t record_bytes(int order, bool f32, bool tensorial, const GridDev& g) {
  const int64_t nbins = (int64_t)g.n0 * g.n1 * g.n2;
  if (order == 2 && tensorial && tsc_run_records(g))  // one record per run of four bins
    return (size_t)(nbins / run::RUN) * run::RUNREC * (f32 ? 4 : 8);
  const int npair = order == 1 ? Geo<1>::NPAIR : Geo<2>::NPAIR;
  const size_t recb = (size_t)nbins * npair * (tensorial ? 9 : 1) * (f32 ? 4 : 8);
  if (order == 2 && !f32 && tensorial)  // k_tsc64 keeps its bin order after the records
    return (recb + 255) / 256 * 256 + tsc64_order_bytes(nbins);
  return recb;
}

// ---------------------------------------------------------------- phase 2
// Thread order of the gather (GatherShape::ROWS): rows of offsets at order 2
// (with the mirrored stores, the deposit is 10% faster for the scalar matrix
// and 9% (fp64) to 21% (fp32) for 3x3 blocks than in node-major order) and for
// the mirrored single-set deposit at order 1; node-major otherwise, where
// order 1 stages its contiguous outputs through LDS.

// M[g][o][c] = sum over the bins k = g - a whose support holds both g and
// g + o of rec[k][pair(a, a+o)][c]; the terms are added in a fixed order.
// With several record sets (one per species, NR > 1) each term is the sum of
// the sets' entries in set order, so the species' matrices are added in one
// pass over M.
// One thread per (node, offset, group of CPT components): the CPT values of a
// record entry are contiguous, and the threads of one entry cover it without
// gaps. Each block covers part of one row of nodes (fixed y, z), so the row
// decomposition is wave-uniform and the per-thread index arithmetic divides
// only by compile-time constants. Rows are visited in z-blocks of ZB planes,
// y-major and z-minor within a block, and each XCD takes a contiguous range of
// blocks: the 4 (CIC) or 9 (TSC) bin rows a node row reads were read by the
// XCD a few rows earlier and are still in its L2.
// CANON: only the canonical half of the offsets, o >= centre (Sec. 3.4),
// stored at o - centre.
// Full stencil (SYM): the threads run the canonical half too and each stores
// its sum twice, at M[g][o] and at the mirrored entry M[g + d(o)][-o], equal
// by the spatial symmetry M_gg' = M_g'g. Each record entry is then read
// once: run over all offsets, the two reads of a pair (for o and for -o)
// fall far apart and the second missed the L2 (the order-2 deposit fetched
// 2.2 times its records, the order-1 deposit of two species on 64^3 cells
// 1.7 times). At order 1 with one record set (MIR1) it is taken only on
// small planes, in rows of offsets: 34 against 36.5 us on 32^3 cells, while
// on 64^3 cells the node-major order with its contiguous outputs staged
// through LDS stays ahead (387 against 469 us).
template <int R, bool CANON, int NR, bool MIR1 = false>
struct GatherShape {
  static constexpr int NOFF = Geo<R>::NOFF;
  static constexpr bool SYM = !CANON && (R == 2 || NR > 1 || MIR1);
  static constexpr bool ROWS = R == 2 || (MIR1 && R == 1 && NR == 1 && !CANON);  // rows of offsets
  static constexpr int O0 = (CANON || SYM) ? (NOFF - 1) / 2 : 0;  // first offset computed
  static constexpr int NIT = NOFF - O0;                            // offsets computed per node
  static constexpr int NOUT = CANON ? NIT : NOFF;                  // offsets stored per node
  static constexpr int SO0 = CANON ? O0 : 0;                       // offset o is stored at o - SO0
};

template <typename T, int R, int NC, bool CANON, int NR, bool MIR1>
__global__ __launch_bounds__(256) void k_gather(GridDev g, RecSet<T> recs, int accumulate, T* __restrict__ M,
                                                int blocks_per_row) {
  constexpr int NS = Geo<R>::NS, N = Geo<R>::N, NO = Geo<R>::NO, NOFF = Geo<R>::NOFF, NPAIR = Geo<R>::NPAIR;
  constexpr int CPT = NC == 9 ? 3 : 1;  // components per thread
  constexpr int TPE = NC / CPT;         // threads per (node, offset)
  typedef GatherShape<R, CANON, NR, MIR1> GS;
  constexpr int O0 = GS::O0, NOUT = GS::NOUT, SO0 = GS::SO0;
  constexpr int ROWT = GS::NIT * TPE;              // threads per node
  constexpr bool ROWS_OF_OFFSETS = GS::ROWS;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int rv = blk / blocks_per_row;  // visit order of the row
  const int t0 = (blk - rv * blocks_per_row) * 256;
  const int t = t0 + threadIdx.x;
  const bool active = t < g.n0 * (ROWS_OF_OFFSETS ? (NO * NO - O0 / NO) * NO * TPE : ROWT);
  // order 1 without the mirrored form stages its contiguous outputs through
  // LDS (every thread stays for the block's barrier); the others store directly
  constexpr bool STAGED = R == 1 && !GS::SYM;
  if (!STAGED && !active) return;
  constexpr int ZB = 4;
  const int nfull = g.n2 / ZB;           // complete z-blocks
  const int inb = g.n1 * ZB;             // rows per complete z-block
  int gy, gz;
  if (rv < nfull * inb) {
    const int zb = rv / inb, rem = rv - zb * inb;
    gy = rem / ZB;
    gz = zb * ZB + (rem - gy * ZB);
  } else {                               // last, thinner z-block
    const int zl = g.n2 - nfull * ZB, rem = rv - nfull * inb;
    gy = rem / zl;
    gz = nfull * ZB + (rem - gy * zl);
  }
  const int row = gy + g.n1 * gz;
  int gx, o, c0;
  if (!ROWS_OF_OFFSETS) {  // (node, offset, component group), offset-minor: contiguous outputs
    gx = t / ROWT;
    const int rr = t - gx * ROWT;
    o = O0 + rr / TPE;
    c0 = (rr - (o - O0) * TPE) * CPT;
  } else {
    // (oy, oz), then node, then (ox, component group): a wave shares the y and
    // z parts of its offsets, so the y and z loops below run the same terms on
    // every lane and only the three x terms depend on the lane (in node-major
    // order a wave spans about 21 offsets and runs nearly all 27 terms with
    // few lanes each). Offsets below O0 (the half that is not computed) are
    // idle threads.
    constexpr int OYZ0 = O0 / NO;
    const int per = g.n0 * NO * TPE;  // threads per (oy, oz)
    const int oyz = OYZ0 + t / per;
    const int rem = t - (oyz - OYZ0) * per;
    gx = rem / (NO * TPE);
    const int r2 = rem - gx * (NO * TPE);
    const int oxi = r2 / TPE;
    o = oxi + NO * oyz;
    c0 = (r2 - oxi * TPE) * CPT;
    if (o < O0) return;
  }
  const int ox = o % NO - R, oy = (o / NO) % NO - R, oz = o / (NO * NO) - R;
  const int dlin = ox + NS * (oy + NS * oz);  // b - a in support-linear numbering
  // bin coordinates g - a per axis (wrapped)
  int kx[NS], kyz[NS][NS];
#pragma unroll
  for (int a = 0; a < NS; ++a) kx[a] = gx - a < 0 ? gx - a + g.n0 : gx - a;
#pragma unroll
  for (int az = 0; az < NS; ++az) {
    const int kz = gz - az < 0 ? gz - az + g.n2 : gz - az;
#pragma unroll
    for (int ay = 0; ay < NS; ++ay) {
      const int ky = gy - ay < 0 ? gy - ay + g.n1 : gy - ay;
      kyz[az][ay] = g.n0 * (ky + g.n1 * kz);
    }
  }
  T sum[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) sum[j] = T(0);
  if (active) {
#pragma unroll
  for (int az = 0; az < NS; ++az) {
    if (az + oz < 0 || az + oz > R) continue;
#pragma unroll
    for (int ay = 0; ay < NS; ++ay) {
      if (ay + oy < 0 || ay + oy > R) continue;
#pragma unroll
      for (int ax = 0; ax < NS; ++ax) {
        if (ax + ox < 0 || ax + ox > R) continue;
        const int a = ax + NS * (ay + NS * az);
        const int b = a + dlin;
        // pair(lo, hi) = lo * N - lo (lo - 1) / 2 + hi - lo
        const int lo = a < b ? a : b, hi = a < b ? b : a;
        const int pi = lo * (2 * N - lo - 1) / 2 + hi;
        const unsigned k = (unsigned)(kx[ax] + kyz[az][ay]);
        const size_t off = ((size_t)k * NPAIR + pi) * NC + c0;
#pragma unroll
        for (int q = 0; q < NR; ++q) {
          if (q == 0 || q < recs.n) {  // (wave-uniform)
            const T* src = recs.r[q] + off;
#pragma unroll
            for (int j = 0; j < CPT; ++j) sum[j] += src[j];
          }
        }
      }
    }
  }
  }
  if (STAGED) {
    // The block's outputs are contiguous (thread t holds values CPT t ..
    // CPT t + CPT - 1 of its row): stage them in LDS and store 16 bytes per
    // lane. 10% faster at 64^3 cells.
    __shared__ __attribute__((aligned(16))) T so[256 * CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) so[threadIdx.x * CPT + j] = sum[j];
    __syncthreads();
    const int nval = (g.n0 * ROWT - t0 < 256 ? g.n0 * ROWT - t0 : 256) * CPT;
    T* base = M + (size_t)row * g.n0 * (NOUT * NC) + (size_t)t0 * CPT;
    if (sizeof(T) == 8 && (reinterpret_cast<uintptr_t>(base) & 15) == 0) {
      const int npair = nval / 2;
      for (int i = threadIdx.x; i < npair; i += 256) {
        double2 v = reinterpret_cast<const double2*>(so)[i];
        double2* d = reinterpret_cast<double2*>(base) + i;
        if (accumulate) {
          const double2 old = *d;
          v.x += old.x;
          v.y += old.y;
        }
        *d = v;
      }
      if ((nval & 1) && threadIdx.x == 0) base[nval - 1] = accumulate ? base[nval - 1] + so[nval - 1] : so[nval - 1];
    } else {
      for (int i = threadIdx.x; i < nval; i += 256) base[i] = accumulate ? base[i] + so[i] : so[i];
    }
  } else {
    T* dst = M + ((size_t)row * g.n0 + gx) * (NOUT * NC) + (o - SO0) * NC + c0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) dst[j] = accumulate ? dst[j] + sum[j] : sum[j];
    if (GS::SYM && o != O0) {  // the mirrored entry (O0 is the centre offset here)
      int mx = gx + ox, my = gy + oy, mz = gz + oz;
      mx = mx < 0 ? mx + g.n0 : (mx >= g.n0 ? mx - g.n0 : mx);
      my = my < 0 ? my + g.n1 : (my >= g.n1 ? my - g.n1 : my);
      mz = mz < 0 ? mz + g.n2 : (mz >= g.n2 ? mz - g.n2 : mz);
      T* mdst = M + ((size_t)mx + (size_t)g.n0 * ((size_t)my + (size_t)g.n1 * mz)) * (NOUT * NC) +
                (NOFF - 1 - o) * NC + c0;
#pragma unroll
      for (int j = 0; j < CPT; ++j) mdst[j] = accumulate ? mdst[j] + sum[j] : sum[j];
    }
  }
}

template <typename T, int R, int NC, bool CANON, int NR, bool MIR1 = false>
static hipError_t gather_go(const GridDev& g, const RecSet<T>& rs, int accumulate, void* M, hipStream_t s) {
  typedef GatherShape<R, CANON, NR, MIR1> GS;
  constexpr int NO = Geo<R>::NO;
  // threads per row of nodes (with rows of offsets: whole (oy, oz) rows)
  const size_t row_len =
      (size_t)g.n0 * (GS::ROWS ? (NO * NO - GS::O0 / NO) * NO : GS::NIT) * (NC == 9 ? 3 : 1);
  if (row_len > 0x7fffff00ULL) return hipErrorInvalidValue;
  const int bpr = (int)((row_len + 255) / 256);
  const size_t blocks = (size_t)bpr * g.n1 * g.n2;
  if (blocks > 0x7fffffffULL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gather<T, R, NC, CANON, NR, MIR1>), dim3((unsigned)blocks), dim3(256), 0, s, g, rs,
                     accumulate, (T*)M, bpr);
  return hipGetLastError();
}

template <typename T, int R, int NC, bool CANON>
static hipError_t gather_launch(const GridDev& g, const void* const* rec, int nrec, int accumulate, void* M,
                                hipStream_t s) {
  if (nrec < 1 || nrec > MAX_REC) return hipErrorInvalidValue;
  RecSet<T> rs{};
  for (int q = 0; q < nrec; ++q) rs.r[q] = (const T*)rec[q];
  rs.n = nrec;
  if (nrec > 1) return gather_go<T, R, NC, CANON, MAX_REC>(g, rs, accumulate, M, s);
  // one set at order 1 (full stencil): the mirrored form on planes of at most 32 x 32 nodes
  if constexpr (R == 1 && !CANON) {
    if ((int64_t)g.n0 * g.n1 <= 1024) return gather_go<T, R, NC, CANON, 1, true>(g, rs, accumulate, M, s);
  }
  return gather_go<T, R, NC, CANON, 1>(g, rs, accumulate, M, s);
}

template <bool CANON>
static hipError_t gather_dispatch(const GridDev& g, int order, bool f32, bool tensorial, const void* const* rec,
                                  int nrec, int accumulate, void* M, hipStream_t s) {
  if (f32) {
    if (order == 1)
      return tensorial ? gather_launch<float, 1, 9, CANON>(g, rec, nrec, accumulate, M, s)
                       : gather_launch<float, 1, 1, CANON>(g, rec, nrec, accumulate, M, s);
    return tensorial ? gather_launch<float, 2, 9, CANON>(g, rec, nrec, accumulate, M, s)
                     : gather_launch<float, 2, 1, CANON>(g, rec, nrec, accumulate, M, s);
  }
  if (order == 1)
    return tensorial ? gather_launch<double, 1, 9, CANON>(g, rec, nrec, accumulate, M, s)
                     : gather_launch<double, 1, 1, CANON>(g, rec, nrec, accumulate, M, s);
  return tensorial ? gather_launch<double, 2, 9, CANON>(g, rec, nrec, accumulate, M, s)
                   : gather_launch<double, 2, 1, CANON>(g, rec, nrec, accumulate, M, s);
}

hipError_t launch_gather(const GridDev& g, int order, bool f32, bool tensorial, const void* const* rec, int nrec,
                         int accumulate,
                         void* M, hipStream_t s, bool canonical) {
  if (order == 2 && tensorial && tsc_run_records(g))  // run records of k_tsc64 / k_tsc32
    return launch_gather_run(g, rec, nrec, accumulate, M, s, canonical, f32);
  return canonical ? gather_dispatch<true>(g, order, f32, tensorial, rec, nrec, accumulate, M, s)
                   : gather_dispatch<false>(g, order, f32, tensorial, rec, nrec, accumulate, M, s);
}

}  // namespace mmk
