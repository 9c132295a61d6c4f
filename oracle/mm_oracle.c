/*
 * CPU oracle for particle-to-grid mass-matrix assembly.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU product path
 * never calls it, links it or shares code with it.
 *
 * What it computes (Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores
 * for Implicit Particle-In-Cell Methods"):
 *   M^{ij}_{g g'} = sigma * sum_p s_p^{ij} W_pg W_pg'            (Sec. 2.1, Eq. 6)
 * with the tensor-product B-spline weight W_pg = prod_mu phi^(n)(.)  (Sec. 2.3, Eq. 12),
 * evaluated as a plain direct per-particle scatter: every particle adds its
 * N x N weighted outer product into the compact stencil storage of Sec. 3.4.
 * The paper states that its cell-by-cell matrix-product assembly reaches this
 * same result up to rounding (Sec. 5, "Exactness and precision"), so the plain
 * definition is the oracle.
 *
 * Readings where the page is silent (each is also a test pin):
 *  - phi^(1)(t) = 1 - |t| (CIC) and the quadratic cardinal B-spline (TSC);
 *    the page keeps only their product form and the support rule of Sec. 2.3.
 *  - s_p^{ij} = w_p * alpha_p^{ij}; scalar case s_p = w_p. alpha_p is the
 *    implicit-midpoint magnetic response (I + beta^2 B B^T - beta [B]x) /
 *    (1 + beta^2 |B|^2), [B]x u = B x u (the page cites it as Eq. 5 but the
 *    formula itself did not survive extraction).
 *  - Grid nodes sit at origin + k*h; the domain is periodic with n cells per
 *    dimension and as many nodes. n[2] == 1 is the 2D problem (Sec. 5 reports
 *    2D runs): the z coordinate is ignored, the support is (R+1)^2 nodes in
 *    the x-y plane and the stencil (2R+1)^2 offsets, offset = (dx+R) +
 *    (2R+1)*(dy+R).
 *  - Output layout M[node][offset][comp]: node = x + nx*(y + ny*z);
 *    offset = (dx+R) + (2R+1)*((dy+R) + (2R+1)*(dz+R)) for the node-pair
 *    displacement d = g' - g in [-R, R]^3; comp = 3*i + j (ncomp = 9) or 0.
 *
 * Precision: fp64 throughout, on the values passed in. An fp32 workload is
 * given to the oracle as its fp32-rounded inputs (exact in fp64), so the
 * oracle is fp64 arithmetic on the fp32 inputs, the cell decision included.
 *
 * Determinism: the parallel scatter runs z-slabs of particles in two colours;
 * slabs of one colour touch disjoint node planes, so every entry's summation
 * order is fixed (slab colour, then particle index) for any thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_ERR_ARG 1
#define OR_ERR_MEM 2

typedef struct {
  int order;          /* 1 = CIC, 2 = TSC */
  int32_t n[3];
  double origin[3];
  double h[3];
} or_grid;

/* One particle's support: first node (wrapped) and 1D weights per dimension. */
typedef struct {
  int32_t first[3];
  double w1d[3][3];
} or_support;

static int grid_ok(const or_grid* g) {
  if (g->order != 1 && g->order != 2) return 0;
  for (int d = 0; d < 3; ++d) {
    if (g->n[d] < 2 * g->order + 1 && !(d == 2 && g->n[2] == 1)) return 0;
    if (!(g->h[d] > 0.0) || !isfinite(g->h[d]) || !isfinite(g->origin[d])) return 0;
  }
  return 1;
}

static int32_t wrap_index(int64_t k, int32_t n) {
  int64_t r = k % n;
  return (int32_t)(r < 0 ? r + n : r);
}

/* Cell index j (unwrapped) and fraction xi in [0,1) of one coordinate, in fp64
 * (IEEE division, as Sec. 2.3 reads: u = (x - origin) / h). */
static void cell_and_fraction(const or_grid* g, int d, double x, int64_t* j, double* xi) {
  double u = (x - g->origin[d]) / g->h[d];
  double fl = floor(u);
  *j = (int64_t)fl;
  *xi = u - fl;
}

/* Support rule and 1D B-spline weights (Sec. 2.3). */
/* 2D (n[2] == 1): one node plane, no extent in z. */
static int is2d(const or_grid* g) { return g->n[2] == 1; }
/* support nodes per particle and stencil offsets per node */
static int nsup_of(const or_grid* g) { return (g->order + 1) * (g->order + 1) * (is2d(g) ? 1 : g->order + 1); }
static int noff_of(const or_grid* g) {
  const int NO = 2 * g->order + 1;
  return NO * NO * (is2d(g) ? 1 : NO);
}

static void particle_support(const or_grid* g, const double* x, or_support* s) {
  for (int d = 0; d < 3; ++d) {
    if (d == 2 && is2d(g)) {
      s->first[2] = 0;
      s->w1d[2][0] = 1.0;
      s->w1d[2][1] = 0.0;
      s->w1d[2][2] = 0.0;
      continue;
    }
    int64_t j;
    double xi;
    cell_and_fraction(g, d, x[d], &j, &xi);
    if (g->order == 1) {
      /* CIC: the two corners of the particle's cell; phi(t) = 1 - |t|. */
      s->first[d] = wrap_index(j, g->n[d]);
      s->w1d[d][0] = 1.0 - xi;
      s->w1d[d][1] = xi;
      s->w1d[d][2] = 0.0;
    } else {
      /* TSC: centred on the nearest node m; xi < 1/2 -> m = j, else m = j+1.
       * delta = offset of the particle from m, in [-1/2, 1/2). */
      int64_t m;
      double delta;
      if (xi < 0.5) {
        m = j;
        delta = xi;
      } else {
        m = j + 1;
        delta = xi - 1.0;
      }
      s->first[d] = wrap_index(m - 1, g->n[d]);
      s->w1d[d][0] = 0.5 * (0.5 - delta) * (0.5 - delta);
      s->w1d[d][1] = 0.75 - delta * delta;
      s->w1d[d][2] = 0.5 * (0.5 + delta) * (0.5 + delta);
    }
  }
}

/* alpha = (I + beta^2 B B^T - beta [B]x) / (1 + beta^2 |B|^2), row-major. */
static void response_tensor(const double* B, double beta, double* alpha) {
  double bx = B[0], by = B[1], bz = B[2];
  double den = 1.0 + beta * beta * (bx * bx + by * by + bz * bz);
  /* [B]x = [[0,-bz,by],[bz,0,-bx],[-by,bx,0]] */
  double cross[9] = {0.0, -bz, by, bz, 0.0, -bx, -by, bx, 0.0};
  for (int i = 0; i < 3; ++i)
    for (int k = 0; k < 3; ++k) {
      double v = (i == k ? 1.0 : 0.0) + beta * beta * B[i] * B[k] - beta * cross[3 * i + k];
      alpha[3 * i + k] = v / den;
    }
}

int oracle_alpha(const double* B, double beta, double* alpha) {
  if (!B || !alpha) return OR_ERR_ARG;
  response_tensor(B, beta, alpha);
  return OR_OK;
}

/* Support of one particle, exported for tests: first[3] and w1d[3][3]. */
int oracle_support(int order, const int32_t* n, const double* origin, const double* h,
                   const double* x, int32_t* first, double* w1d) {
  or_grid g;
  g.order = order;
  for (int d = 0; d < 3; ++d) {
    g.n[d] = n[d];
    g.origin[d] = origin[d];
    g.h[d] = h[d];
  }
  if (!grid_ok(&g) || !x || !first || !w1d) return OR_ERR_ARG;
  or_support s;
  particle_support(&g, x, &s);
  for (int d = 0; d < 3; ++d) {
    first[d] = s.first[d];
    for (int a = 0; a < 3; ++a) w1d[3 * d + a] = s.w1d[d][a];
  }
  return OR_OK;
}

/* Add one particle's contribution (Eq. 6) into M. */
static void scatter_particle(const or_grid* g, const double* x, double w, const double* B, double beta,
                             double sigma, double* M) {
  const int R = g->order, NS = R + 1, NO = 2 * R + 1, RZ = is2d(g) ? 0 : R;
  const int noff = noff_of(g);
  const int ncomp = B ? 9 : 1;
  or_support s;
  particle_support(g, x, &s);

  double t[9];
  if (B) {
    double alpha[9];
    response_tensor(B, beta, alpha);
    for (int c = 0; c < 9; ++c) t[c] = sigma * (w * alpha[c]);
  } else {
    t[0] = sigma * w;
  }

  int nsup = nsup_of(g);
  int64_t node[27];
  double W[27];
  int ax[27], ay[27], az[27];
  for (int a = 0; a < nsup; ++a) {
    ax[a] = a % NS;
    ay[a] = (a / NS) % NS;
    az[a] = a / (NS * NS);
    int64_t gx = (s.first[0] + ax[a]) % g->n[0];
    int64_t gy = (s.first[1] + ay[a]) % g->n[1];
    int64_t gz = (s.first[2] + az[a]) % g->n[2];
    node[a] = gx + (int64_t)g->n[0] * (gy + (int64_t)g->n[1] * gz);
    W[a] = (s.w1d[0][ax[a]] * s.w1d[1][ay[a]]) * s.w1d[2][az[a]];
  }
  for (int a = 0; a < nsup; ++a) {
    for (int b = 0; b < nsup; ++b) {
      double ww = W[a] * W[b];
      int o = (ax[b] - ax[a] + R) + NO * ((ay[b] - ay[a] + R) + NO * (az[b] - az[a] + RZ));
      double* dst = M + ((size_t)node[a] * noff + o) * ncomp;
      for (int c = 0; c < ncomp; ++c) dst[c] += t[c] * ww;
    }
  }
}

static int fill_grid(or_grid* g, int order, const int32_t* n, const double* origin,
                     const double* h) {
  if (!n || !origin || !h) return 0;
  g->order = order;
  for (int d = 0; d < 3; ++d) {
    g->n[d] = n[d];
    g->origin[d] = origin[d];
    g->h[d] = h[d];
  }
  return grid_ok(g);
}

/*
 * Direct scatter of Eq. (6). B == NULL selects the scalar mass matrix
 * (ncomp = 1), else the 3x3 tensorial one (ncomp = 9).
 * M has nnodes*noff*ncomp doubles; it is zeroed first unless accumulate != 0.
 * nthreads <= 0 uses the OpenMP default.
 */
int oracle_assemble(int order, const int32_t* n, const double* origin, const double* h,
                    int64_t np, const double* pos, const double* w, const double* B, double beta,
                    double sigma, int accumulate, double* M, int nthreads) {
  or_grid g;
  if (!fill_grid(&g, order, n, origin, h) || !M || np < 0) return OR_ERR_ARG;
  if (np > 0 && (!pos || !w)) return OR_ERR_ARG;
  const int R = order;
  const int64_t nnodes = (int64_t)n[0] * n[1] * n[2];
  const int ncomp = B ? 9 : 1;
  const size_t nel = (size_t)nnodes * noff_of(&g) * ncomp;
  if (!accumulate) memset(M, 0, nel * sizeof(double));
  if (np == 0) return OR_OK;

  /* Bucket particles by the z-slab of their first support node. A slab is at
   * least R+1 node planes thick and the slab count is even, so slabs of one
   * colour write disjoint node planes (including across the periodic wrap). */
  const int nz = n[2];
  int nslab = nz / (R + 1);
  if (nslab % 2) nslab -= 1;
  if (nslab < 2) nslab = 1;
  int64_t* slab_count = (int64_t*)calloc((size_t)nslab + 1, sizeof(int64_t));
  int32_t* slab_of = (int32_t*)malloc((size_t)np * sizeof(int32_t));
  int64_t* order_idx = (int64_t*)malloc((size_t)np * sizeof(int64_t));
  if (!slab_count || !slab_of || !order_idx) {
    free(slab_count);
    free(slab_of);
    free(order_idx);
    return OR_ERR_MEM;
  }
  for (int64_t p = 0; p < np; ++p) {
    or_support s;
    particle_support(&g, pos + 3 * p, &s);
    int sl = (int)(((int64_t)s.first[2] * nslab) / nz);
    slab_of[p] = sl;
    slab_count[sl + 1]++;
  }
  for (int sl = 0; sl < nslab; ++sl) slab_count[sl + 1] += slab_count[sl];
  {
    int64_t* cursor = (int64_t*)malloc((size_t)nslab * sizeof(int64_t));
    if (!cursor) {
      free(slab_count);
      free(slab_of);
      free(order_idx);
      return OR_ERR_MEM;
    }
    for (int sl = 0; sl < nslab; ++sl) cursor[sl] = slab_count[sl];
    for (int64_t p = 0; p < np; ++p) order_idx[cursor[slab_of[p]]++] = p;
    free(cursor);
  }

#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  for (int colour = 0; colour < 2; ++colour) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int sl = colour; sl < nslab; sl += 2) {
      for (int64_t q = slab_count[sl]; q < slab_count[sl + 1]; ++q) {
        int64_t p = order_idx[q];
        scatter_particle(&g, pos + 3 * p, w[p], B ? B + 3 * p : NULL, beta, sigma, M);
      }
    }
    if (nslab == 1) break;
  }
  free(slab_count);
  free(slab_of);
  free(order_idx);
  return OR_OK;
}

/* Number of OpenMP threads the scatter would use (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Particle binning by the linear index of each particle's first support node
 * (one bin per distinct support set, Sec. 3.3), as a stable counting sort:
 * bin_start[k] = number of particles with key < k (nbins+1 entries),
 * perm lists particle indices bin by bin, ascending within a bin.
 */
int oracle_bin(int order, const int32_t* n, const double* origin, const double* h,
               int64_t np, const double* pos, int32_t* bin_start, int32_t* perm) {
  or_grid g;
  if (!fill_grid(&g, order, n, origin, h) || !bin_start || np < 0) return OR_ERR_ARG;
  if (np > 0 && (!pos || !perm)) return OR_ERR_ARG;
  const int64_t nbins = (int64_t)n[0] * n[1] * n[2];
  int32_t* key = (int32_t*)malloc((size_t)(np > 0 ? np : 1) * sizeof(int32_t));
  int64_t* cnt = (int64_t*)calloc((size_t)nbins + 1, sizeof(int64_t));
  if (!key || !cnt) {
    free(key);
    free(cnt);
    return OR_ERR_MEM;
  }
  for (int64_t p = 0; p < np; ++p) {
    or_support s;
    particle_support(&g, pos + 3 * p, &s);
    key[p] = (int32_t)(s.first[0] + (int64_t)n[0] * (s.first[1] + (int64_t)n[1] * s.first[2]));
    cnt[key[p] + 1]++;
  }
  for (int64_t k = 0; k < nbins; ++k) cnt[k + 1] += cnt[k];
  for (int64_t k = 0; k <= nbins; ++k) bin_start[k] = (int32_t)cnt[k];
  for (int64_t p = 0; p < np; ++p) perm[cnt[key[p]]++] = (int32_t)p;
  free(key);
  free(cnt);
  return OR_OK;
}

/*
 * Matrix-free bilinear form of Eq. (6):
 *   out = sigma * sum_p (W_p u)^T s_p (W_p v),   (W_p u)_i = sum_a W_pa u[g_a][i]
 * u, v hold nnodes*ncomp_vec values (ncomp_vec = 3 tensorial, 1 scalar).
 */
int oracle_bilinear(int order, const int32_t* n, const double* origin, const double* h,
                    int64_t np, const double* pos, const double* w, const double* B, double beta,
                    double sigma, const double* u, const double* v, double* out) {
  or_grid g;
  if (!fill_grid(&g, order, n, origin, h) || !u || !v || !out || np < 0) return OR_ERR_ARG;
  if (np > 0 && (!pos || !w)) return OR_ERR_ARG;
  const int NS = order + 1, nsup = nsup_of(&g);
  const int nv = B ? 3 : 1;
  double total = 0.0;
#pragma omp parallel for reduction(+ : total) schedule(static)
  for (int64_t p = 0; p < np; ++p) {
    or_support s;
    particle_support(&g, pos + 3 * p, &s);
    double wu[3] = {0, 0, 0}, wv[3] = {0, 0, 0};
    for (int a = 0; a < nsup; ++a) {
      int ax = a % NS, ay = (a / NS) % NS, az = a / (NS * NS);
      int64_t gx = (s.first[0] + ax) % n[0], gy = (s.first[1] + ay) % n[1], gz = (s.first[2] + az) % n[2];
      int64_t node = gx + (int64_t)n[0] * (gy + (int64_t)n[1] * gz);
      double W = (s.w1d[0][ax] * s.w1d[1][ay]) * s.w1d[2][az];
      for (int i = 0; i < nv; ++i) {
        wu[i] += W * u[node * nv + i];
        wv[i] += W * v[node * nv + i];
      }
    }
    double acc = 0.0;
    if (B) {
      double alpha[9];
      response_tensor(B + 3 * p, beta, alpha);
      for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) acc += wu[i] * (w[p] * alpha[3 * i + j]) * wv[j];
    } else {
      acc = wu[0] * w[p] * wv[0];
    }
    total += sigma * acc;
  }
  *out = total;
  return OR_OK;
}

/*
 * Exact stencil rows of Eq. (6) for a set of nodes, by scanning every
 * particle: rows[s][offset][comp] for node sel[s]. Used where the full output
 * is too large to hold on the host.
 */
int oracle_rows(int order, const int32_t* n, const double* origin, const double* h,
                int64_t np, const double* pos, const double* w, const double* B, double beta,
                double sigma, int64_t nsel, const int64_t* sel, double* rows) {
  or_grid g;
  if (!fill_grid(&g, order, n, origin, h) || !rows || np < 0 || nsel < 0) return OR_ERR_ARG;
  if (nsel > 0 && !sel) return OR_ERR_ARG;
  if (np > 0 && (!pos || !w)) return OR_ERR_ARG;
  const int R = order, NS = R + 1, NO = 2 * R + 1, nsup = nsup_of(&g), noff = noff_of(&g), RZ = is2d(&g) ? 0 : R;
  const int ncomp = B ? 9 : 1;
  const int64_t nnodes = (int64_t)n[0] * n[1] * n[2];
  memset(rows, 0, (size_t)nsel * noff * ncomp * sizeof(double));
  /* node -> list of selected row slots (a node may be selected more than once) */
  int64_t* head = (int64_t*)malloc((size_t)nnodes * sizeof(int64_t));
  int64_t* next = (int64_t*)malloc((size_t)(nsel > 0 ? nsel : 1) * sizeof(int64_t));
  if (!head || !next) {
    free(head);
    free(next);
    return OR_ERR_MEM;
  }
  for (int64_t k = 0; k < nnodes; ++k) head[k] = -1;
  for (int64_t s = 0; s < nsel; ++s) {
    if (sel[s] < 0 || sel[s] >= nnodes) {
      free(head);
      free(next);
      return OR_ERR_ARG;
    }
    next[s] = head[sel[s]];
    head[sel[s]] = s;
  }
  for (int64_t p = 0; p < np; ++p) {
    or_support s;
    particle_support(&g, pos + 3 * p, &s);
    int64_t node[27];
    double W[27];
    int hit = 0;
    for (int a = 0; a < nsup; ++a) {
      int ax = a % NS, ay = (a / NS) % NS, az = a / (NS * NS);
      int64_t gx = (s.first[0] + ax) % n[0], gy = (s.first[1] + ay) % n[1], gz = (s.first[2] + az) % n[2];
      node[a] = gx + (int64_t)n[0] * (gy + (int64_t)n[1] * gz);
      W[a] = (s.w1d[0][ax] * s.w1d[1][ay]) * s.w1d[2][az];
      if (head[node[a]] >= 0) hit = 1;
    }
    if (!hit) continue;
    double t[9];
    if (B) {
      double alpha[9];
      response_tensor(B + 3 * p, beta, alpha);
      for (int c = 0; c < 9; ++c) t[c] = sigma * (w[p] * alpha[c]);
    } else {
      t[0] = sigma * w[p];
    }
    for (int a = 0; a < nsup; ++a) {
      for (int64_t slot = head[node[a]]; slot >= 0; slot = next[slot]) {
        int ax = a % NS, ay = (a / NS) % NS, az = a / (NS * NS);
        for (int b = 0; b < nsup; ++b) {
          int bx = b % NS, by = (b / NS) % NS, bz = b / (NS * NS);
          int o = (bx - ax + R) + NO * ((by - ay + R) + NO * (bz - az + RZ));
          double ww = W[a] * W[b];
          double* dst = rows + ((size_t)slot * noff + o) * ncomp;
          for (int c = 0; c < ncomp; ++c) dst[c] += t[c] * ww;
        }
      }
    }
  }
  free(head);
  free(next);
  return OR_OK;
}

/*
 * Particle values of a nodal vector field, gathered with the particle's own
 * support weights (the same W_pa that enter Eq. 6):
 *   out[p][i] = sum_a W_pa F[g_a][i],   i = 0..2
 * F holds nnodes*3 values (node-major). This is how the magnetic field of the
 * grid reaches each particle before its response tensor alpha_p is formed
 * (Sec. 4.1 names loading the field values and precomputing alpha_p as the
 * non-matrix work of the tensorial kernel); that the field lives on the same
 * nodes as M and is gathered with the same weights is a reading, the plainest
 * one the page supports.
 */
int oracle_interp_field(int order, const int32_t* n, const double* origin, const double* h,
                        int64_t np, const double* pos, const double* F, double* out) {
  or_grid g;
  if (!fill_grid(&g, order, n, origin, h) || np < 0) return OR_ERR_ARG;
  if (np > 0 && (!pos || !F || !out)) return OR_ERR_ARG;
  const int NS = order + 1, nsup = nsup_of(&g);
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < np; ++p) {
    or_support s;
    particle_support(&g, pos + 3 * p, &s);
    double acc[3] = {0.0, 0.0, 0.0};
    for (int a = 0; a < nsup; ++a) {
      int ax = a % NS, ay = (a / NS) % NS, az = a / (NS * NS);
      int64_t gx = (s.first[0] + ax) % n[0], gy = (s.first[1] + ay) % n[1], gz = (s.first[2] + az) % n[2];
      int64_t node = gx + (int64_t)n[0] * (gy + (int64_t)n[1] * gz);
      double W = (s.w1d[0][ax] * s.w1d[1][ay]) * s.w1d[2][az];
      for (int i = 0; i < 3; ++i) acc[i] += W * F[node * 3 + i];
    }
    for (int i = 0; i < 3; ++i) out[3 * p + i] = acc[i];
  }
  return OR_OK;
}

/*
 * Particle-to-grid deposition of per-particle quantities with the same
 * weights, m[g][k] = sum_p W_pg Q_p[k] for k < nq: charge and current (four
 * quantities per particle in 3D) or the ten of the implicit moment method,
 * the other scatters the page's Sec. 6 (Conclusion) names for the same
 * contraction, one operand holding the quantities and the other the weights.
 * Q holds np*nq values (particle-major), m holds nnodes*nq and is zeroed
 * first unless accumulate != 0. Serial, particle by particle.
 */
int oracle_moments(int order, const int32_t* n, const double* origin, const double* h, int64_t np,
                   const double* pos, int nq, const double* Q, int accumulate, double* m) {
  or_grid g;
  if (!fill_grid(&g, order, n, origin, h) || !m || np < 0 || nq < 1) return OR_ERR_ARG;
  if (np > 0 && (!pos || !Q)) return OR_ERR_ARG;
  const int NS = order + 1, nsup = nsup_of(&g);
  const int64_t nnodes = (int64_t)n[0] * n[1] * n[2];
  if (!accumulate) memset(m, 0, (size_t)nnodes * nq * sizeof(double));
  for (int64_t p = 0; p < np; ++p) {
    or_support s;
    particle_support(&g, pos + 3 * p, &s);
    for (int a = 0; a < nsup; ++a) {
      int ax = a % NS, ay = (a / NS) % NS, az = a / (NS * NS);
      int64_t gx = (s.first[0] + ax) % n[0], gy = (s.first[1] + ay) % n[1], gz = (s.first[2] + az) % n[2];
      int64_t node = gx + (int64_t)n[0] * (gy + (int64_t)n[1] * gz);
      double W = (s.w1d[0][ax] * s.w1d[1][ay]) * s.w1d[2][az];
      for (int k = 0; k < nq; ++k) m[node * nq + k] += W * Q[p * nq + k];
    }
  }
  return OR_OK;
}
