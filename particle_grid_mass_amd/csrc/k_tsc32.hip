// Second-order (TSC) fp32 3x3 per-bin contraction on v_mfma_f32_4x4x1_16b,
// writing the records of x-runs of four bins (mm_run.h): phase 1 of the
// two-phase assembly in single precision.
//
// Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for Implicit
// Particle-In-Cell Methods": the particles of one support group share 27
// support nodes (Sec. 3.3; here one bin per first support node), whose local
// matrix Mhat^c_ab = sum_p t_p^c W_pa W_pb (Sec. 3.1, Eq. 15) is accumulated
// particle by particle (Sec. 3.2); blocks below the diagonal are skipped by
// the symmetry Mhat_ab = Mhat_ba (Table 1 and its footnote).
//
// gfx950 mapping. The fp32 4x4x1 instruction works on 16 independent 4x4
// blocks with one product term each, four result values per lane, so a wave
// that gave each of 16 blocks a bin of its own and held all 28 upper blocks
// of the 27 rows (padded to 28) would need 112 registers per component. A
// wave here takes a group of 8 consecutive bins (two runs) and two components:
// block b is bin b & 7 for component c0 (b < 8) or c1 (b >= 8). The 28
// instructions of a step advance the 8 bins by one particle each for both
// components; five waves cover the 9 components of a group (the fifth takes
// component 8 in both halves and keeps one).
//  * Particle preparation runs two particles per lane (16 per bin per chunk): the
//    cell decision in fp64 on the stored position (as the binning), the
//    support weights W_a (Eq. 12) and the response tensor in fp32. A staged
//    slot holds, for each row r of a 4x4 block, W_{4I + r} (I = 0..6) and one
//    coefficient, placed so that neither the staging stores nor the step
//    loads meet an LDS bank conflict (unit_base, unit_swz).
//  * The particle data of the next chunk, and the permutation entries of the
//    chunk after it, are in flight during the current chunk's 16 steps.
//  * End phase, per component and run: the lanes of the run's four blocks
//    park their blocks in LDS (one 16-byte store per block: the transposed
//    block layout of mm_run.h), then every lane sums the one to three bin
//    values of 16 of the run's 999 union entries in bin order (reading the
//    exact zero of a padding entry where an entry has fewer bins) and stores
//    them into the component's line-aligned stretches of the run record.
#include "mm_contract.h"
#include "mm_run.h"

namespace mmk {

namespace {

constexpr int NBW = 8;                   // bins per wave group (two runs)
constexpr int CH = 16;                   // particles per bin per chunk (two per lane)
constexpr int NS = 3;                    // support nodes per axis
constexpr int N = 27;                    // support nodes
constexpr int NBLK = 7;                  // row blocks of 4 (28 rows)
constexpr int NBP = NBLK * (NBLK + 1) / 2;  // upper blocks
constexpr int NQ = 5;                    // waves per group: components (0,1) (2,3) (4,5) (6,7) (8,8)
constexpr int SLOTF = 32;                // floats per staged particle: 4 rows x (7 W + 1 coefficient)
constexpr int STAGEF = NBW * CH * SLOTF;  // staged particles of a chunk
constexpr int PVF = run::RUN * run::BSTRIDE;  // one component's blocks of one run
constexpr int SMEMF = STAGEF > PVF ? STAGEF : PVF;

// Staging layout in 16-byte units: particle p of bin b keeps its 8 units
// (unit 2 r + h: half h of row r) at 8 (16 b + (p ^ (b & 1))) + (u ^ swz(b, p)).
// With this placement the 16 lanes served together meet 16 different bank
// groups both when the lanes stage their slots (two bins, eight particles,
// one unit each) and when a step reads one slot of each of 4 bins (4 rows of
// each): neither the staging stores nor the step loads have bank conflicts.
__device__ __forceinline__ int unit_base(int b, int p) { return 8 * (CH * b + (p ^ (b & 1))); }
__device__ __forceinline__ int unit_swz(int b, int p) {
  return (((b >> 1) ^ (p >> 1)) & 1) | (((p >> 2) & 1) << 1) | ((b & 1) << 2);
}

static __constant__ run::Tables kRun32 = run::make_tables();

// Bins b0 + 8g .. b0 + 8g + 7 below bend. Prep lane l serves bin b0 + 8g +
// (l >> 3) (particles l & 7 and 8 + (l & 7) of each chunk): start in perm and
// count; maxn (the largest count of the group) is wave-uniform.
struct Group {
  int s, n;
  int maxn;
  int nchunks;
};

__device__ __forceinline__ Group load_group(const int32_t* __restrict__ bin_start, int g, int b0, int bend, int np,
                                            int lane) {
  Group G;
  const int bin = b0 + NBW * g + (lane >> 3);
  int s = 0, e = 0;
  if (bin < bend) {
    s = bin_start[bin];
    e = bin_start[bin + 1];
    s = s < 0 ? 0 : (s > np ? np : s);
    e = e < s ? s : (e > np ? np : e);
  }
  G.s = s;
  G.n = e - s;
  int m = G.n;
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) m = max(m, __shfl_xor(m, off));
  G.maxn = __builtin_amdgcn_readfirstlane(m);
  G.nchunks = G.maxn > 0 ? (G.maxn + CH - 1) / CH : 1;  // an empty group still writes zero records
  return G;
}

// The loads below are unconditional (index 0 stands in for a missing
// particle; the kernel loads nothing when np == 0), so that the compiler's
// wait counts stay exact: a load under a branch makes it wait for every load
// in flight.
__device__ __forceinline__ int chunk_perm(const int32_t* __restrict__ perm, const Group& G, int j, int h,
                                          int lane) {
  const int q = j * CH + 8 * h + (lane & 7);
  const int v = perm[q < G.n ? G.s + q : 0];
  return q < G.n ? v : -1;
}

struct Raw {
  float x, y, z, w, bx, by, bz;
  bool valid;
};

__device__ __forceinline__ Raw load_raw(const float* __restrict__ pos, const float* __restrict__ w,
                                        const float* __restrict__ Bf, int p, int np) {
  Raw r;
  r.valid = (unsigned)p < (unsigned)np;
  const size_t i = r.valid ? (size_t)p : 0;
  r.x = pos[3 * i];
  r.y = pos[3 * i + 1];
  r.z = pos[3 * i + 2];
  r.w = w[i];
  r.bx = Bf[3 * i];
  r.by = Bf[3 * i + 1];
  r.bz = Bf[3 * i + 2];
  return r;
}

// Weights and this wave's two coefficients of the lane's particle into its
// slot (zeros for a lane without a particle): row r of the slot holds
// W_{4I + r} for I = 0..6 (zero for the padding row 27) and, in its last
// float, t^{c0} (r = 0), t^{c1} (r = 1) or zero.
__device__ __forceinline__ void stage(const Raw& r, const GridDev& g, float beta, float sigma, int c0, int c1,
                                      float* sm, int lane, int h) {
  float wx[3] = {0, 0, 0}, wy[3] = {0, 0, 0}, wz[3] = {0, 0, 0}, t[9];
#pragma unroll
  for (int c = 0; c < 9; ++c) t[c] = 0.0f;
  if (r.valid) {
    support_axis<float, 2, 0>((double)r.x, g, wx);
    support_axis<float, 2, 1>((double)r.y, g, wy);
    support_axis<float, 2, 2>((double)r.z, g, wz);
    response<float>(r.bx, r.by, r.bz, beta, sigma * r.w, t);
  }
  float wyz[NS * NS];
#pragma unroll
  for (int az = 0; az < NS; ++az)
#pragma unroll
    for (int ay = 0; ay < NS; ++ay) wyz[ay + NS * az] = wy[ay] * wz[az];
  auto wsup = [&](int a) { return a < N ? wx[a % NS] * wyz[a / NS] : 0.0f; };
  // t[c0], t[c1] with wave-uniform c0, c1: selected without indexing registers
  float tc0 = 0.0f, tc1 = 0.0f;
#pragma unroll
  for (int c = 0; c < 9; ++c) {
    tc0 = c == c0 ? t[c] : tc0;
    tc1 = c == c1 ? t[c] : tc1;
  }
  const int b = lane >> 3, p = (lane & 7) + 8 * h;
  float4* su = reinterpret_cast<float4*>(sm) + unit_base(b, p);
  const int x = unit_swz(b, p);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const float e7 = rr == 0 ? tc0 : (rr == 1 ? tc1 : 0.0f);
    su[(2 * rr) ^ x] = float4{wsup(rr), wsup(4 + rr), wsup(8 + rr), wsup(12 + rr)};
    su[(2 * rr + 1) ^ x] = float4{wsup(16 + rr), wsup(20 + rr), wsup(24 + rr), e7};
  }
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace

__global__ __launch_bounds__(64) void k_tsc32(GridDev g, const float* __restrict__ pos, const float* __restrict__ w,
                                              const float* __restrict__ Bf, const int32_t* __restrict__ bin_start,
                                              const int32_t* __restrict__ perm, int np, int b0, int bend,
                                              float beta, float sigma, float* __restrict__ rec, int xch) {
  __shared__ __attribute__((aligned(16))) float sm[SMEMF];
  const int lane = threadIdx.x;
  // the launch covers bins b0 .. bend - 1 (whole runs)
  const int ngroups = (bend - b0 + NBW - 1) / NBW;
  const int r0 = b0 / run::RUN, rend = bend / run::RUN;
  // chunks of xch blocks (whole groups: the NQ waves of a group share an XCD
  // and its L2) dealt round the XCDs
  const int lid = xcd_chunk_remap(blockIdx.x, gridDim.x, xch);
  const int grp = lid / NQ, qw = lid - grp * NQ;
  if (grp >= ngroups) return;
  const int c0 = 2 * qw, c1 = 2 * qw + 1 < 9 ? 2 * qw + 1 : 8;  // this wave's components
  const Group G = load_group(bin_start, grp, b0, bend, np, lane);

  // MFMA lane roles: block blk (bin blk & 7, component slot blk >> 3), row /
  // column mr of the 4x4 block.
  const int blk = lane >> 2, mr = lane & 3, bb = blk & 7, cs = blk >> 3;
  v4f acc[NBP];
#pragma unroll
  for (int k = 0; k < NBP; ++k) acc[k] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  auto steps = [&](int j) {
    const int left = G.maxn - j * CH;
    const int nr = left >= CH ? CH : left;
    for (int rd = 0; rd < nr; ++rd) {
      const float4* su = reinterpret_cast<const float4*>(sm) + unit_base(bb, rd);
      const int x = unit_swz(bb, rd);
      const float4 u0 = su[(2 * mr) ^ x];
      const float4 u1 = su[(2 * mr + 1) ^ x];
      const float tv = reinterpret_cast<const float*>(su + ((2 * cs + 1) ^ x))[3];
      const float wv[NBLK] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z};
      float a[NBLK];
#pragma unroll
      for (int I = 0; I < NBLK; ++I) a[I] = tv * wv[I];
      int k = 0;
#pragma unroll
      for (int I = 0; I < NBLK; ++I)
#pragma unroll
        for (int J = I; J < NBLK; ++J, ++k) acc[k] = mfma_f32_4x4x1(a[I], wv[J], acc[k]);
    }
  };
  // The loads are unconditional at index 0 for a missing particle, which
  // exists only when np > 0: without particles (an empty species) nothing is
  // read and the records stay zero.
  if (np > 0) {
  Raw r0 = load_raw(pos, w, Bf, chunk_perm(perm, G, 0, 0, lane), np);
  Raw r1 = load_raw(pos, w, Bf, chunk_perm(perm, G, 0, 1, lane), np);
  int p0 = chunk_perm(perm, G, 1, 0, lane), p1 = chunk_perm(perm, G, 1, 1, lane);
  for (int j = 0; j < G.nchunks; ++j) {
    stage(r0, g, beta, sigma, c0, c1, sm, lane, 0);
    stage(r1, g, beta, sigma, c0, c1, sm, lane, 1);
    wave_sync();
    r0 = load_raw(pos, w, Bf, p0, np);  // next chunk, in flight during the steps
    r1 = load_raw(pos, w, Bf, p1, np);
    p0 = chunk_perm(perm, G, j + 2, 0, lane);
    p1 = chunk_perm(perm, G, j + 2, 1, lane);
    steps(j);
    wave_sync();
  }
  }

  // D_blk[i][j] sits in lane 4 blk + j, register i: column j of the block, the
  // four rows contiguous in the transposed layout (block_slot_t).
  constexpr int NIT = (run::NENT + 63) / 64;  // entries per lane
  unsigned tb[NIT], ts[NIT];  // the lane's entries: their block slots and where they are stored
#pragma unroll
  for (int q = 0; q < NIT; ++q) {
    const int e = lane + 64 * q < run::NENT ? lane + 64 * q : run::NENT - 1;
    tb[q] = kRun32.contrib_t[e];
    ts[q] = kRun32.store_bytes[e];
  }
#pragma unroll 1
  for (int s2 = 0; s2 < 2; ++s2) {
    if (s2 == 1 && c1 == c0) break;  // the fifth wave keeps component 8 once
    const unsigned comp = s2 == 0 ? c0 : c1;
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
      const int r = r0 + 2 * grp + h;  // the run
      if (r >= rend) break;
      if (cs == s2 && (bb >> 2) == h) {
        float* pl = sm + (bb & 3) * run::BSTRIDE + 4 * mr;
#pragma unroll
        for (int k = 0; k < NBP; ++k) *reinterpret_cast<v4f*>(pl + 16 * k) = acc[k];
      }
      wave_sync();
      char* dst = reinterpret_cast<char*>(rec + (size_t)r * run::RUNREC);
#pragma unroll
      for (int q = 0; q < NIT; ++q) {
        const unsigned t = tb[q];
        const unsigned sb = ts[q];
        const float v = (sm[t & 2047u] + sm[((t >> 11) & 2047u) + run::ZERO0]) + sm[(t >> 22) + run::ZERO1];
        // float offset = half the double offset of the same entry; comp planes of
        // its slice. Nontemporal, as in the fp64 kernel: the records are read
        // again only by the deposit.
        const unsigned o = ((sb & 0x1ffffu) >> 1) + comp * 64u * (sb >> 17);
        if (q < NIT - 1 || lane + 64 * q < run::NENT) __builtin_nontemporal_store(v, reinterpret_cast<float*>(dst + o));
      }
      wave_sync();
    }
  }
}

hipError_t launch_tsc32(const GridDev& g, const Particles& P, const int32_t* bin_start, const int32_t* perm,
                        double beta, double sigma, float* rec, hipStream_t s, int z0, int z1) {
  if (!P.B || P.Bgrid || P.pos32 || !tsc_run_records(g)) return hipErrorInvalidValue;
  if (z1 < 0) z1 = g.n2;
  if (z0 < 0 || z0 > z1 || z1 > g.n2) return hipErrorInvalidValue;
  const int pl = g.n0 * g.n1;  // bins per plane
  const int b0 = z0 * pl, bend = z1 * pl;
  const int ngroups = (bend - b0 + NBW - 1) / NBW;
  if (ngroups == 0) return hipSuccess;
  // XCD chunks of a plane of groups (a launch of fewer than 8 planes: an
  // eighth of its groups per chunk): bins one row apart in y read the same
  // cells' particles from one L2
  int xg = pl / NBW < ngroups / 8 ? pl / NBW : ngroups / 8;
  xg = xg > 1 ? xg : 1;
  hipLaunchKernelGGL(k_tsc32, dim3(ngroups * NQ), dim3(64), 0, s, g, (const float*)P.pos, (const float*)P.w,
                     (const float*)P.B, bin_start, perm, P.np, b0, bend, (float)beta, (float)sigma, rec, NQ * xg);
  return hipGetLastError();
}

}  // namespace mmk
