// First-order (CIC) fp32 per-bin contraction on v_mfma_f32_4x4x1_16b, phase 1
// of the two-phase assembly in single precision.
//
// Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for Implicit
// Particle-In-Cell Methods": every particle of a CIC cell touches the same
// 8 corner nodes (Sec. 2.3), so the cell's local matrix is
//   Mhat^c_ab = sum_p t_p^c W_pa W_pb                       (Sec. 3.1, Eq. 15)
// accumulated particle by particle (Sec. 3.2); the lower off-diagonal
// quadrant is skipped by the spatial symmetry Mhat_ab = Mhat_ba (Table 1).
//
// gfx950 mapping. The fp32 4x4x1 instruction works on 16 independent 4x4
// blocks with one product term each. One wave owns a group of 16 consecutive
// bins and gives each bin one block, so block results are final (no
// cross-block reduction) and every instruction advances all 16 bins by one
// particle. The 8 support rows split by the z corner into two halves; per
// component three instructions form the quadrants Q00, Q01, Q11 (27 per
// particle of each bin for the 3x3 matrix, 3 for the scalar one).
//
//  * Particle preparation runs one particle per lane (4 per bin per chunk):
//    the cell decision in fp64 on the stored position (as the binning), the
//    support weights W_a (Eq. 12) and the coefficients t^c = sigma w alpha^c in
//    fp32, staged in LDS. A lane of a round feeds rows r and 4 + r of its
//    bin, one 8-byte read; slots are padded so that the 16 bins' reads fall
//    on distinct LDS banks.
//  * The particle data of the next chunk, and the permutation entries of the
//    chunk after it, are in flight while the current chunk is contracted.
//  * A finished group stages its packed upper-triangle records in LDS, eight
//    bins at a time, and writes them with 16-byte stores (the records of
//    consecutive bins are contiguous).
#include "mm_contract.h"

namespace mmk {

namespace {

constexpr int NB = 16;      // bins per wave group (= blocks of the instruction)
constexpr int CH = 4;       // particles per bin per chunk (one per lane)
constexpr int NPAIR = 36;   // packed upper triangle of 8 x 8
constexpr int WS = 10;      // floats per staged slot of W: 4 pairs (W_r, W_{4+r}) and one pad pair
constexpr int TS = 12;      // floats per staged slot of t (9 used)
constexpr int WREG = 64 * WS;

template <int NC>
struct Cfg {
  static constexpr int STAGE = WREG + 64 * TS;            // floats of particle staging
  static constexpr int REC = (NB / 2) * NPAIR * NC;       // records of eight bins
  static constexpr int SMEM = STAGE > REC ? STAGE : REC;
};

// A group is bins 16g .. 16g+15. Prep lane l serves bin 16g + (l >> 2): `s`
// and `n` are that bin's start in perm and particle count; `maxn` is the
// largest count of the group (wave-uniform).
struct Group {
  int s, n;
  int maxn;
  int nchunks;
};

__device__ __forceinline__ Group load_group(const int32_t* __restrict__ bin_start, int g, int nbins, int np,
                                            int lane) {
  Group G;
  const int bin = NB * g + (lane >> 2);
  int s = 0, e = 0;
  if (bin < nbins) {
    s = bin_start[bin];
    e = bin_start[bin + 1];
    s = s < 0 ? 0 : (s > np ? np : s);
    e = e < s ? s : (e > np ? np : e);
  }
  G.s = s;
  G.n = e - s;
  int m = G.n;
#pragma unroll
  for (int off = 4; off < 64; off <<= 1) m = max(m, __shfl_xor(m, off));
  G.maxn = __builtin_amdgcn_readfirstlane(m);
  G.nchunks = G.maxn > 0 ? (G.maxn + CH - 1) / CH : 1;  // an empty group still writes zero records
  return G;
}

__device__ __forceinline__ int chunk_perm(const int32_t* __restrict__ perm, const Group& G, int j, int lane) {
  const int q = j * CH + (lane & 3);
  return q < G.n ? perm[G.s + q] : -1;
}

struct Raw {
  float x, y, z, w, bx, by, bz;
  bool valid;
};

template <int NC>
__device__ __forceinline__ Raw load_raw(const float* __restrict__ pos, const float* __restrict__ w,
                                        const float* __restrict__ Bf, int p, int np) {
  Raw r{0, 0, 0, 0, 0, 0, 0, false};
  if ((unsigned)p < (unsigned)np) {
    r.valid = true;
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

// Weights and coefficients of the lane's particle into slot `lane` (zeros for
// a lane without a particle).
template <int NC>
__device__ __forceinline__ void stage(const Raw& r, const GridDev& g, float beta, float sigma, float* sm, int lane) {
  float wx[2] = {0, 0}, wy[2] = {0, 0}, wz[2] = {0, 0}, t[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) t[c] = 0.0f;
  if (r.valid) {
    support_axis<float, 1, 0>((double)r.x, g, wx);
    support_axis<float, 1, 1>((double)r.y, g, wy);
    support_axis<float, 1, 2>((double)r.z, g, wz);
    const float f = sigma * r.w;
    if (NC == 9)
      response<float>(r.bx, r.by, r.bz, beta, f, t);
    else
      t[0] = f;
  }
  float2* sw = reinterpret_cast<float2*>(sm + lane * WS);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float wxy = wx[q & 1] * wy[q >> 1];
    sw[q] = float2{wxy * wz[0], wxy * wz[1]};
  }
  float* st = sm + WREG + lane * TS;
  if (NC == 9) {
    *reinterpret_cast<float4*>(st) = float4{t[0], t[1], t[2], t[3]};
    *reinterpret_cast<float4*>(st + 4) = float4{t[4], t[5], t[6], t[7]};
    st[8] = t[8];
  } else {
    st[0] = t[0];
  }
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace

template <int NC>
__global__ __launch_bounds__(64) void k_cic32(GridDev g, const float* __restrict__ pos, const float* __restrict__ w,
                                              const float* __restrict__ Bf, const int32_t* __restrict__ bin_start,
                                              const int32_t* __restrict__ perm, int np, int nbins, float beta,
                                              float sigma, float* __restrict__ rec) {
  __shared__ __attribute__((aligned(16))) float sm[Cfg<NC>::SMEM];
  const int lane = threadIdx.x;
  const int ngroups = (nbins + NB - 1) / NB;
  const int grp = xcd_chunk_remap(blockIdx.x, gridDim.x, 16);  // chunks of groups dealt round the XCDs
  if (grp >= ngroups) return;
  const Group G = load_group(bin_start, grp, nbins, np, lane);

  // MFMA lane roles: block (= bin) mb, row / column mr of the 4x4 block.
  const int mb = lane >> 2, mr = lane & 3;
  v4f acc[NC][3];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int k = 0; k < 3; ++k) acc[c][k] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  Raw raw = load_raw<NC>(pos, w, Bf, chunk_perm(perm, G, 0, lane), np);
  int pnext = chunk_perm(perm, G, 1, lane);
  for (int j = 0; j < G.nchunks; ++j) {
    stage<NC>(raw, g, beta, sigma, sm, lane);
    wave_sync();
    raw = load_raw<NC>(pos, w, Bf, pnext, np);  // next chunk, in flight during the rounds
    pnext = chunk_perm(perm, G, j + 2, lane);
    const int left = G.maxn - j * CH;
    const int nr = left >= CH ? CH : left;
    for (int rd = 0; rd < nr; ++rd) {
      const int slot = CH * mb + rd;
      const float2 wv = reinterpret_cast<const float2*>(sm + slot * WS)[mr];  // (W_r, W_{4+r})
      const float* st = sm + WREG + slot * TS;
      float tv[NC];
      if (NC == 9) {
        const float4 t0 = *reinterpret_cast<const float4*>(st);
        const float4 t1 = *reinterpret_cast<const float4*>(st + 4);
        tv[0] = t0.x; tv[1] = t0.y; tv[2] = t0.z; tv[3] = t0.w;
        tv[4] = t1.x; tv[5] = t1.y; tv[6] = t1.z; tv[7] = t1.w;
        tv[8] = st[8];
      } else {
        tv[0] = st[0];
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float alo = tv[c] * wv.x, ahi = tv[c] * wv.y;
        acc[c][0] = mfma_f32_4x4x1(alo, wv.x, acc[c][0]);
        acc[c][1] = mfma_f32_4x4x1(alo, wv.y, acc[c][1]);
        acc[c][2] = mfma_f32_4x4x1(ahi, wv.y, acc[c][2]);
      }
    }
    wave_sync();
  }

  // D_blk[i][j] sits in lane 4 blk + j, register i. Stage the packed records
  // rec[bin][pair(a, b)][c] (a <= b, pair(a, b) = 8a - a(a-1)/2 + b - a) of
  // eight bins at a time in LDS and write them with 16-byte stores.
  const int dj = mr;
  const int b0 = NB * grp;
  const int nvalid = nbins - b0 < NB ? nbins - b0 : NB;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((mb >> 3) == half) {
      float* sr = sm + (mb & 7) * NPAIR * NC;
#pragma unroll
      for (int di = 0; di < 4; ++di) {
        const int p00 = di * 8 - (di * (di - 1)) / 2 + (dj - di);
        const int p01 = di * 8 - (di * (di - 1)) / 2 + (4 + dj - di);
        const int a1 = 4 + di;
        const int p11 = a1 * 8 - (a1 * (a1 - 1)) / 2 + (dj - di);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          if (di <= dj) sr[p00 * NC + c] = acc[c][0][di];
          sr[p01 * NC + c] = acc[c][1][di];
          if (di <= dj) sr[p11 * NC + c] = acc[c][2][di];
        }
      }
    }
    wave_sync();
    const int nb = nvalid - 8 * half < 8 ? nvalid - 8 * half : 8;
    const int n4 = nb > 0 ? nb * NPAIR * NC / 4 : 0;  // NPAIR is a multiple of 4: whole 16-byte words
    float4* dst = reinterpret_cast<float4*>(rec + (size_t)(b0 + 8 * half) * NPAIR * NC);
    const float4* src = reinterpret_cast<const float4*>(sm);
    for (int i = lane; i < n4; i += 64) dst[i] = src[i];
    wave_sync();
  }
}

hipError_t launch_cic32(const GridDev& g, const Particles& P, const int32_t* bin_start, const int32_t* perm,
                        double beta, double sigma, float* rec, hipStream_t s) {
  if (P.Bgrid || P.pos32) return hipErrorInvalidValue;  // fp32 particles, field per particle
  const int nbins = g.n0 * g.n1 * g.n2;
  const int ngroups = (nbins + NB - 1) / NB;  // one single-wave workgroup per group of 16 bins
  if (P.B)
    hipLaunchKernelGGL((k_cic32<9>), dim3(ngroups), dim3(64), 0, s, g, (const float*)P.pos, (const float*)P.w,
                       (const float*)P.B, bin_start, perm, P.np, nbins, (float)beta, (float)sigma, rec);
  else
    hipLaunchKernelGGL((k_cic32<1>), dim3(ngroups), dim3(64), 0, s, g, (const float*)P.pos, (const float*)P.w,
                       (const float*)nullptr, bin_start, perm, P.np, nbins, (float)beta, (float)sigma, rec);
  return hipGetLastError();
}

}  // namespace mmk
