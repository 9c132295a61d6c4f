// Second-order (TSC) fp64 per-bin contraction on v_mfma_f64_4x4x4_4b, phase 1
// of the two-phase assembly.
//
// Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for Implicit
// Particle-In-Cell Methods": particles with the same 27-node support form one
// support group (Sec. 3.3; here one bin per first support node), whose local
// matrix Mhat^c_ab = sum_p t_p^c W_pa W_pb (Sec. 3.1, Eq. 15) is accumulated
// over batches of K_t particles (Sec. 3.2); blocks below the diagonal are
// skipped by the symmetry Mhat_ab = Mhat_ba (Table 1 and its footnote).
//
// gfx950 mapping.
//  * The 27 support rows are padded to 28 = 7 row blocks of 4. The 4x4x4_4b
//    instruction computes one 4x4 block (I, J) of four bins at once (one bin
//    per block, K_t = 4 particles of each bin); the 28 blocks with I <= J
//    cover the upper triangle: 28 instructions per component per 16
//    particles, against 27 16x16x4 instructions per 4 particles when the
//    rows are padded to 32 (4.3x less matrix-core time per particle).
//  * One single-wave workgroup per (group of four consecutive bins, row i of
//    alpha): the wave keeps the 28 blocks of components 3i .. 3i+2 (84
//    accumulators). The three waves of a group run on one XCD, so the
//    particles all three read come from that XCD's L2 after the first.
//  * Particle preparation runs one particle per lane: the 27 support weights
//    W_a (Eq. 12) and the wave's three coefficients are staged in LDS, W
//    laid out so that staging stores and round loads meet no LDS bank conflict.
//  * Particle data of the next chunk is in flight during the current rounds.
//  * Two waves per SIMD (the accumulators live in VGPRs), so that one wave's
//    preparation and record writes overlap the other's matrix instructions.
//  * Records rec[bin][pair][comp] are staged in LDS one bin at a time; the
//    three components a wave owns per pair are written as one 24-byte piece
//    (the three waves of a group fill the 72 bytes of a pair in the XCD's L2).
//  * The particle arrays may have any element stride (ST), as when each
//    particle is one record of its position, weight and field.
#include "mm_contract.h"
#include "mm_run.h"

namespace mmk {

namespace {

constexpr int NB = 4;       // bins per group (= 4x4x4 blocks)
constexpr int CH = 16;      // particles per bin per chunk
constexpr int NS = 3;       // support nodes per axis
constexpr int N = 27;       // support nodes
constexpr int NBLK = 7;     // row blocks of 4 (28 rows)
constexpr int NBP = NBLK * (NBLK + 1) / 2;  // upper blocks
constexpr int NPAIR = 378;  // packed upper triangle of 27 x 27
constexpr int WSLOT = 32;   // staged doubles per particle: 16 units of 16 bytes (see w_unit)

constexpr int NC = 9;       // components of the tensorial matrix
constexpr int CPW = 3;      // components per wave (one row of alpha)
constexpr int NQ = NC / CPW;  // waves per group of bins
constexpr int SMEM = 64 * WSLOT;
constexpr int FIELD = NB * N * 3;  // grid field at the group's support nodes (field on the grid), after SMEM
static_assert(NPAIR * CPW <= 64 * WSLOT, "record staging fits the W region");

// Bins 4g .. 4g+3. Prep lane l serves bin 4g + (l >> 4): start in perm and
// count; maxn (the largest count of the group) is wave-uniform.
struct Group {
  int s, n;
  int maxn;
  int nchunks;
};

// Bin b (0..3) of group g: order[4g + b] when the groups follow a bin order,
// else 4g + b; nbins or more for a slot past the end.
__device__ __forceinline__ int group_bin(const int32_t* __restrict__ order, int g, int b, int nbins) {
  const int i = NB * g + b;
  return order ? (i < nbins ? order[i] : nbins) : i;
}

__device__ __forceinline__ Group load_group(const int32_t* __restrict__ bin_start, const int32_t* __restrict__ order,
                                            int g, int nbins, int np, int lane) {
  Group G;
  const int bin = group_bin(order, g, lane >> 4, nbins);
  int s = 0, e = 0;
  if (bin < nbins) {
    s = bin_start[bin];
    e = bin_start[bin + 1];
    s = s < 0 ? 0 : (s > np ? np : s);
    e = e < s ? s : (e > np ? np : e);
  }
  G.s = s;
  G.n = e - s;
  int m = __builtin_amdgcn_readlane(G.n, 0);
  m = max(m, __builtin_amdgcn_readlane(G.n, 16));
  m = max(m, __builtin_amdgcn_readlane(G.n, 32));
  m = max(m, __builtin_amdgcn_readlane(G.n, 48));
  G.maxn = m;
  G.nchunks = m > 0 ? (m + CH - 1) / CH : 1;  // an empty group still writes zero records
  return G;
}

__device__ __forceinline__ int chunk_perm(const int32_t* __restrict__ perm, const Group& G, int j, int lane) {
  const int q = j * CH + (lane & 15);
  return q < G.n ? perm[G.s + q] : -1;
}

struct Raw {
  double x, y, z, w, bx, by, bz;
  bool valid;
};

// Element strides of the particle arrays (read when the kernel's ST is set).
struct ArrStrides {
  int64_t ps, wst, bst;
};

// GB: the field is on the grid (gathered in stage), not per particle. PT: type
// of the stored positions and field (fp64, or fp32 read into fp64). ST: the
// particle values st.ps, st.wst and st.bst elements apart instead of 3, 1, 3.
template <typename PT, bool GB, bool ST>
__device__ __forceinline__ Raw load_raw(const PT* __restrict__ pos, const double* __restrict__ w,
                                        const PT* __restrict__ Bf, int p, int np, const ArrStrides& st) {
  Raw r{0, 0, 0, 0, 0, 0, 0, false};
  if ((unsigned)p < (unsigned)np) {
    r.valid = true;
    const size_t qp = ST ? (size_t)st.ps * p : 3 * (size_t)p, qb = ST ? (size_t)st.bst * p : 3 * (size_t)p;
    r.x = pos[qp];
    r.y = pos[qp + 1];
    r.z = pos[qp + 2];
    r.w = w[ST ? (size_t)st.wst * p : (size_t)p];
    if (!GB) {
      r.bx = Bf[qb];
      r.by = Bf[qb + 1];
      r.bz = Bf[qb + 2];
    }
  }
  return r;
}

// Row `row` of t = f alpha, alpha = (I + beta^2 B B^T - beta [B]x) / (1 + beta^2 |B|^2),
// [B]x = [[0,-Bz,By],[Bz,0,-Bx],[-By,Bx,0]]; `row` is wave-uniform.
__device__ __forceinline__ void response_row(double bx, double by, double bz, double beta, double f, int row,
                                             double* t) {
  const double b2 = beta * beta;
  const double den = 1.0 + b2 * (bx * bx + by * by + bz * bz);
  const double gq = f / den;
  const double cx = beta * bx, cy = beta * by, cz = beta * bz;
  if (row == 0) {
    const double s = b2 * bx;
    t[0] = gq * (1.0 + s * bx);
    t[1] = gq * (s * by + cz);
    t[2] = gq * (s * bz - cy);
  } else if (row == 1) {
    const double s = b2 * by;
    t[0] = gq * (s * bx - cz);
    t[1] = gq * (1.0 + s * by);
    t[2] = gq * (s * bz + cx);
  } else {
    const double s = b2 * bz;
    t[0] = gq * (s * bx + cy);
    t[1] = gq * (s * by - cx);
    t[2] = gq * (1.0 + s * bz);
  }
}

// LDS layout, chosen so that neither the staging stores (lane = slot) nor
// the operand loads of a round (lanes = 4 bins x 4 rows, each group of 16
// lanes served together) meet two lanes on one bank.
// W: slot s holds W_{4I + r} (I = 0..6, zero where 4I + r > 26) in logical
// 16-byte unit u = 4r + I/2, half I & 1; the unit is stored at position
// u ^ ((s >> 4) ^ (s & 15)). The half I = 7 of row r < 3 (never a matrix
// operand) holds the coefficient t_r of this wave's row of alpha.
__device__ __forceinline__ int w_unit(int s, int u) { return s * (WSLOT / 2) + (u ^ (((s >> 4) & 3) ^ (s & 15))); }

// Value of v in lane C of each group of four lanes (DPP quad_perm broadcast).
template <int C>
__device__ __forceinline__ double quad_bcast(double v) {
  constexpr int ctrl = C | (C << 2) | (C << 4) | (C << 6);
  const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), ctrl, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), ctrl, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}

// Support weights and this wave's coefficients of the lane's particle into
// slot `lane` (zeros for a lane without a particle). With GB the field at the
// particle is gathered from sF, the grid field at the 27 support nodes of each
// bin of the group (node a = ax + 3 ay + 9 az, 3 components).
template <bool GB>
__device__ __forceinline__ void stage(const Raw& r, const GridDev& g, double beta, double sigma, int row,
                                      double* sW, const double* sF, int lane) {
  double wx[3] = {0, 0, 0}, wy[3] = {0, 0, 0}, wz[3] = {0, 0, 0}, t[3] = {0, 0, 0};
  if (r.valid) {
    support_axis<double, 2, 0>((double)r.x, g, wx);
    support_axis<double, 2, 1>((double)r.y, g, wy);
    support_axis<double, 2, 2>((double)r.z, g, wz);
    double bx = r.bx, by = r.by, bz = r.bz;
    if (GB) {
      const double* fb = sF + (lane >> 4) * (3 * N);
      bx = by = bz = 0.0;
#pragma unroll
      for (int a = 0; a < N; ++a) {
        const double W = (wx[a % NS] * wy[(a / NS) % NS]) * wz[a / (NS * NS)];
        bx += W * fb[3 * a];
        by += W * fb[3 * a + 1];
        bz += W * fb[3 * a + 2];
      }
    }
    response_row(bx, by, bz, beta, sigma * r.w, row, t);
  }
  double wyz[NS * NS];
#pragma unroll
  for (int az = 0; az < NS; ++az)
#pragma unroll
    for (int ay = 0; ay < NS; ++ay) wyz[ay + NS * az] = wy[ay] * wz[az];
  // W_a = wx[a % 3] * wyz[a / 3], zero for the padding rows a >= 27
  auto wsup = [&](int a) { return a < N ? wx[a % NS] * wyz[a / NS] : 0.0; };
  double2* su = reinterpret_cast<double2*>(sW);
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
    for (int h = 0; h < 4; ++h)
      su[w_unit(lane, 4 * r4 + h)] = double2{wsup(8 * h + r4), h < 3 ? wsup(8 * h + 4 + r4) : (r4 < 3 ? t[r4] : 0.0)};
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace

// Run records (RUNS): the group is the run of bins 4 grp .. 4 grp + 3 (consecutive
// x; the launcher passes no bin order). For each of its three components a
// wave stores the four bins' pair values in LDS (one packed triangle per bin,
// each lane its own entries: no conflicts), then every lane sums the one to
// three bin values of its union entries (mm_run.h) in bin order and writes
// the component's nine line-aligned stretches of the run record.
static __constant__ run::Tables kRun = run::make_tables();

template <typename PT, bool GB, bool RUNS, bool ST>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_tsc64(
    GridDev g, const PT* __restrict__ pos, const double* __restrict__ w, const PT* __restrict__ Bf,
    const int32_t* __restrict__ bin_start, const int32_t* __restrict__ perm, int np, int nbins, double beta,
    double sigma, double* __restrict__ rec, const int32_t* __restrict__ order, int xch, int z0, int nz,
    ArrStrides str) {
  __shared__ __attribute__((aligned(16))) double smem[GB ? SMEM + FIELD : SMEM];
  double* sW = smem;
  const int lane = threadIdx.x;
  const int ngroups = (nbins + NB - 1) / NB;
  // chunks of xch blocks (whole groups: the NQ waves of a group share an XCD)
  // dealt round the XCDs: a contiguous range per XCD put 1.3 times the mean
  // work on the XCDs whose range held a cluster of a clustered density
  const int lid = xcd_chunk_remap(blockIdx.x, gridDim.x, xch);
  const int vis = lid / NQ, row = lid - vis * NQ;     // row of alpha: components CPW*row ..
  // Run records: the launch covers the runs of the nz bin planes z0 .. z0 + nz - 1
  if (vis >= (RUNS ? nz * (g.n0 / run::RUN) * g.n1 : ngroups)) return;
  // Run records over an even number of planes: groups are visited by pairs of
  // planes, row by row, the two planes' rows one after the other (the
  // particles of a cell plane are read by the bins of two consecutive planes,
  // which then run on one XCD close in time); otherwise in order.
  int grp = vis;
  if (RUNS) {
    const int R = g.n0 / run::RUN;  // runs per row
    if ((nz & 1) == 0) {
      const int pr = 2 * R * g.n1;  // runs per plane pair
      const int pz = vis / pr, t = vis - pz * pr;
      const int y = t / (2 * R), u = t - y * 2 * R;
      const int zz = u / R, x = u - zz * R;
      grp = x + R * (y + g.n1 * (z0 + 2 * pz + zz));
    } else {
      grp = vis + z0 * R * g.n1;
    }
  }
  const Group G = load_group(bin_start, order, grp, nbins, np, lane);
  double* sF = smem + SMEM;
  if (GB) {
    // Bf is the grid field [nnodes][3]: node a of bin 4 grp + b is the bin's
    // own node (its first support node) shifted by (ax, ay, az).
    for (int i = lane; i < NB * N; i += 64) {
      const int bin = group_bin(order, grp, i / N, nbins), a = i % N;
      double f0 = 0.0, f1 = 0.0, f2 = 0.0;
      if (bin < nbins) {
        const int kx = bin % g.n0, ky = (bin / g.n0) % g.n1, kz = bin / (g.n0 * g.n1);
        int x = kx + a % NS, y = ky + (a / NS) % NS, z = kz + a / (NS * NS);
        x = x < g.n0 ? x : x - g.n0;
        y = y < g.n1 ? y : y - g.n1;
        z = z < g.n2 ? z : z - g.n2;
        const PT* f = Bf + 3 * ((size_t)x + (size_t)g.n0 * ((size_t)y + (size_t)g.n1 * z));
        f0 = f[0];
        f1 = f[1];
        f2 = f[2];
      }
      sF[3 * i] = f0;
      sF[3 * i + 1] = f1;
      sF[3 * i + 2] = f2;
    }
    wave_sync();
  }

  // MFMA lane roles: particle k of the batch, block (= bin) mb, row/column mr.
  const int mk = lane >> 4, mb = (lane >> 2) & 3, mr = lane & 3;
  // slot = 16 mb + 4 rd + mk in round rd: w_unit(slot, 4 mr + h) with the
  // lane's constant part taken out of the loop
  const int wl = (CH * mb + mk) * (WSLOT / 2), wx = mb ^ mk;

  Raw raw = load_raw<PT, GB, ST>(pos, w, Bf, chunk_perm(perm, G, 0, lane), np, str);
  int pnext = chunk_perm(perm, G, 1, lane);
  double acc[CPW][NBP];
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int k = 0; k < NBP; ++k) acc[c][k] = 0.0;

  for (int j = 0; j < G.nchunks; ++j) {
    stage<GB>(raw, g, beta, sigma, row, sW, sF, lane);
    wave_sync();
    raw = load_raw<PT, GB, ST>(pos, w, Bf, pnext, np, str);  // next chunk, in flight during the rounds
    pnext = chunk_perm(perm, G, j + 2, lane);

    const int left = G.maxn - j * CH;
    const int nr = left >= CH ? CH / 4 : (left + 3) / 4;
    for (int rd = 0; rd < nr; ++rd) {
      const double2* su = reinterpret_cast<const double2*>(sW) + wl + 64 * rd;
      const int ux = wx ^ (4 * rd);
      double wv[8];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const double2 v = su[(4 * mr + h) ^ ux];
        wv[2 * h] = v.x;
        wv[2 * h + 1] = v.y;
      }
      // wv[7] of the slot's lane r holds t_r
      const double tv[3] = {quad_bcast<0>(wv[7]), quad_bcast<1>(wv[7]), quad_bcast<2>(wv[7])};
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        double a[NBLK];
#pragma unroll
        for (int I = 0; I < NBLK; ++I) a[I] = tv[c] * wv[I];
        int k = 0;
#pragma unroll
        for (int I = 0; I < NBLK; ++I)
#pragma unroll
          for (int J = I; J < NBLK; ++J, ++k) acc[c][k] = mfma_f64_4x4x4(a[I], wv[J], acc[c][k]);
      }
    }
    wave_sync();
  }

  // D_blk[i][j] of block (I, J) sits in lane (i << 4) | (blk << 2) | j: local
  // entry (4I + i, 4J + j) of bin 4 grp + blk.
  const int di = lane >> 4, db = (lane >> 2) & 3, dj = lane & 3;
  if constexpr (RUNS) {
    static_assert(run::RUN * run::BSTRIDE <= SMEM, "the four bins' blocks of one component fit the W region");
    constexpr int NIT = (run::NENT + 63) / 64;  // entries per lane
    unsigned tb[NIT], ts[NIT];  // the lane's entries: their block slots and where they are stored (read once)
#pragma unroll
    for (int q = 0; q < NIT; ++q) {
      const int e = lane + 64 * q < run::NENT ? lane + 64 * q : run::NENT - 1;
      tb[q] = kRun.contrib[e];
      ts[q] = kRun.store_bytes[e];
    }
    double* pv = sW;                                           // [bin][upper block][i][j] (mm_run.h)
    double* pl = pv + db * run::BSTRIDE + 4 * di + dj;         // this lane's entry of block 0
    char* dst = reinterpret_cast<char*>(rec + (size_t)grp * run::RUNREC);
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
#pragma unroll
      for (int k = 0; k < NBP; ++k) pl[16 * k] = acc[c][k];
      wave_sync();
      // Each entry adds its first bin's value and those of up to two more bins
      // (both nodes one column further left in each), reading an exact zero
      // where it has fewer; no branches, so every lane's reads are in flight
      // together.
      const unsigned comp = CPW * row + c;
      constexpr int HB = NIT / 2;  // entries read before any is summed
#pragma unroll
      for (int h = 0; h < NIT; h += HB) {
        double x[HB][3];
#pragma unroll
        for (int q = 0; q < HB; ++q) {
          const unsigned t = tb[h + q];
          x[q][0] = pv[t & 2047u];
          x[q][1] = pv[((t >> 11) & 2047u) + run::ZERO0];
          x[q][2] = pv[(t >> 22) + run::ZERO1];
        }
#pragma unroll
        for (int q = 0; q < HB; ++q) {
          const double v = (x[q][0] + x[q][1]) + x[q][2];
          const int e = lane + 64 * (h + q);
          // byte offset of the entry's component-0 value plus comp planes of its slice;
          // nontemporal: the records are read again only by the deposit, and
          // kept out of the way in L2 the particle lines that the group's other
          // waves and its y neighbours read stay there (128^3 clustered:
          // FETCH_SIZE 11.0M -> 8.2M KiB per launch, contraction 26.7 -> 26.2 ms)
          const unsigned o = (ts[h + q] & 0x1ffffu) + comp * 128u * (ts[h + q] >> 17);
          if (h + q < NIT - 1 || e < run::NENT) __builtin_nontemporal_store(v, reinterpret_cast<double*>(dst + o));
        }
      }
      wave_sync();
    }
    return;
  }
  // Per-bin records: stage each bin's CPW * NPAIR record values (contiguous in
  // rec) in LDS, then write them with 16-byte stores.
#pragma unroll 1
  for (int b = 0; b < NB; ++b) {
    const int bin = group_bin(order, grp, b, nbins);
    if (bin >= nbins) break;  // wave-uniform (slots past the end come last)
    if (db == b) {
      int k = 0;
#pragma unroll
      for (int I = 0; I < NBLK; ++I)
#pragma unroll
        for (int J = I; J < NBLK; ++J, ++k) {
          const int a = 4 * I + di, bb = 4 * J + dj;
          if (a < N && bb < N && (I < J || di <= dj)) {
            const int pair = a * N - (a * (a - 1)) / 2 + (bb - a);
#pragma unroll
            for (int c = 0; c < CPW; ++c) sW[pair * CPW + c] = acc[c][k];
          }
        }
    }
    wave_sync();
    double* dst = rec + (size_t)bin * NPAIR * NC + CPW * row;
    for (int i = lane; i < NPAIR * CPW; i += 64) {
      const int pair = i / CPW;
      dst[(size_t)pair * NC + (i - pair * CPW)] = sW[i];
    }
    wave_sync();
  }
}

// ---------------------------------------------------------------- bin order
// A group's rounds run to its fullest bin, so bins of different counts in one
// group waste matrix work (about 16% of it for a clustered density). Within
// each window of OWIN consecutive bins the groups take the bins in order of
// decreasing count (ties by index: a stable, deterministic order). Windows
// keep the groups' particles and records close in memory; a global order by
// count was twice as slow for that reason, while windows of 256 bins leave
// about 4% of the work as padding. Each bin's record depends only on its own
// particles, so the records are the same in any order.
constexpr int OWIN = 256;
constexpr int XPLANES = 2;  // planes of runs per XCD chunk (the visit order pairs planes)

__global__ __launch_bounds__(OWIN) void k_order_window(const int32_t* __restrict__ bin_start, int nbins,
                                                       int32_t* __restrict__ order) {
  __shared__ int cnt[OWIN];
  const int w0 = blockIdx.x * OWIN, t = threadIdx.x;
  const int n = nbins - w0 < OWIN ? nbins - w0 : OWIN;
  cnt[t] = t < n ? bin_start[w0 + t + 1] - bin_start[w0 + t] : -1;
  __syncthreads();
  if (t < n) {
    const int c = cnt[t];
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      const int cj = cnt[j];
      rank += (cj > c) || (cj == c && j < t);
    }
    order[w0 + rank] = w0 + t;
  }
}

size_t tsc64_order_bytes(int64_t nbins) { return ((size_t)nbins * 4 + 255) / 256 * 256; }

template <typename PT, bool RUNS>
static hipError_t tsc64_t(const GridDev& g, const Particles& P, const int32_t* bin_start, const int32_t* perm,
                          double beta, double sigma, double* rec, int32_t* order, hipStream_t s, int z0, int z1) {
  const int nbins = g.n0 * g.n1 * g.n2;
  // NQ single-wave workgroups per group of four bins (for run records, the runs of planes z0 .. z1 - 1)
  const int rp = (g.n0 / run::RUN) * g.n1;  // runs per plane
  const int ngroups = RUNS ? (z1 - z0) * rp : (nbins + NB - 1) / NB;
  if (ngroups == 0) return hipSuccess;
  // run records need the groups to be runs of consecutive x: no bin order
  if (!RUNS)
    hipLaunchKernelGGL(k_order_window, dim3((nbins + OWIN - 1) / OWIN), dim3(OWIN), 0, s, bin_start, nbins, order);
  const int32_t* ord = RUNS ? nullptr : (const int32_t*)order;
  // XCD chunks. Runs: a pair of planes of runs per chunk, so that the bins one
  // row and one plane apart, which read the same cells' particles, run on one
  // XCD and find them in its L2 (chunks of 16 runs put them on other XCDs and
  // the particle data was fetched 4.5 times on a 128^3 grid); the plane pairs
  // dealt round the XCDs still balance a clustered density. A launch of fewer
  // than 16 planes (a slab of the overlapped assembly) takes an eighth of its
  // runs per chunk, so that every XCD gets a share. Per-bin records follow the
  // windowed bin order: chunks of 16 groups.
  int xg = 16;
  if (RUNS) {
    xg = ngroups / 8 < XPLANES * rp ? ngroups / 8 : XPLANES * rp;
    xg = xg > 1 ? xg : 1;
  }
  const int xch = NQ * xg;
  const int nz = z1 - z0;
  const ArrStrides str{P.ps, P.wst, P.bst};
  if (P.strided())  // fp64 values with the field per particle (checked by the caller)
    hipLaunchKernelGGL((k_tsc64<PT, false, RUNS, true>), dim3(ngroups * NQ), dim3(64), 0, s, g, (const PT*)P.pos,
                       (const double*)P.w, (const PT*)P.B, bin_start, perm, P.np, nbins, beta, sigma, rec, ord, xch,
                       z0, nz, str);
  else if (P.Bgrid)
    hipLaunchKernelGGL((k_tsc64<PT, true, RUNS, false>), dim3(ngroups * NQ), dim3(64), 0, s, g, (const PT*)P.pos,
                       (const double*)P.w, (const PT*)P.Bgrid, bin_start, perm, P.np, nbins, beta, sigma, rec, ord, xch,
                       z0, nz, str);
  else
    hipLaunchKernelGGL((k_tsc64<PT, false, RUNS, false>), dim3(ngroups * NQ), dim3(64), 0, s, g, (const PT*)P.pos,
                       (const double*)P.w, (const PT*)P.B, bin_start, perm, P.np, nbins, beta, sigma, rec, ord, xch,
                       z0, nz, str);
  return hipGetLastError();
}

bool tsc_run_records(const GridDev& g) { return g.n2 > 1 && g.n0 % run::RUN == 0; }

hipError_t launch_tsc64(const GridDev& g, const Particles& P, const int32_t* bin_start, const int32_t* perm,
                        double beta, double sigma, double* rec, hipStream_t s, int z0, int z1) {
  if (!P.B && !P.Bgrid) return hipErrorInvalidValue;  // tensorial (ECSIM) records only
  if (P.strided() && (P.pos32 || P.Bgrid || !P.B)) return hipErrorInvalidValue;  // strided: fp64, field per particle
  if (z1 < 0) z1 = g.n2;
  if (tsc_run_records(g)) {
    if (z0 < 0 || z0 > z1 || z1 > g.n2) return hipErrorInvalidValue;
    return P.pos32 ? tsc64_t<float, true>(g, P, bin_start, perm, beta, sigma, rec, nullptr, s, z0, z1)
                   : tsc64_t<double, true>(g, P, bin_start, perm, beta, sigma, rec, nullptr, s, z0, z1);
  }
  if (z0 != 0 || z1 != g.n2) return hipErrorInvalidValue;  // plane ranges: run records only
  // per-bin records; the bin order lives after them (record_bytes counts it)
  const int64_t nbins = (int64_t)g.n0 * g.n1 * g.n2;
  const size_t recb = (size_t)nbins * NPAIR * NC * 8;
  int32_t* order = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(rec) + (recb + 255) / 256 * 256);
  return P.pos32 ? tsc64_t<float, false>(g, P, bin_start, perm, beta, sigma, rec, order, s, 0, g.n2)
                 : tsc64_t<double, false>(g, P, bin_start, perm, beta, sigma, rec, order, s, 0, g.n2);
}

}  // namespace mmk
