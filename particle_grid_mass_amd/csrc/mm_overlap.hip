// The two phases of the second-order tensorial assembly on run records,
// overlapped by slabs of planes.
//
// Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for Implicit
// Particle-In-Cell Methods", Sec. 3 assembles in two phases: the local
// matrices of every support group (Sec. 3.1-3.3), then the sparse stencil
// deposition that sums them per matrix entry (Sec. 3.4). On gfx950 the first
// phase of a TSC workload is bound by the matrix cores and the second by HBM,
// so the two run side by side better than in turn. A stencil entry of node
// plane z reads the records of bin planes z - 2 .. z (periodic), so once bin
// planes 0 .. b - 1 are contracted the node planes 2 .. b - 1 can be
// deposited, and node planes 0 and 1 once the last bin planes are done.
//
// Schedule: slabs of kSlabPlanes bin planes are contracted in order on the
// caller's stream; after each, an event lets a second stream of the device
// deposit the node planes that slab completed, while the caller's stream
// goes on with the next slab. The caller's stream finally waits for the
// second stream, so the call is ordered on the caller's stream like any other
// entry point. Each record and each stencil entry is computed by the same
// kernels, in the same order of summation, as in the unsplit phases: the
// results are bit-identical.
//
// Slab thickness (TSC ECSIM fp64 on the clustered 128^3 workload, two boxes
// on which contraction then deposition in turn took 40.6 and 41.4 ms): slabs
// of 2 planes -/43.4 ms, 4 planes 37.5/38.5, 8 planes 38.0/39.3, 16 planes
// 42.4/- (each XCD then takes one chunk of two whole planes per slab, and the
// clustered density leaves some XCDs with far more work than others before
// the next slab may start), 64 planes 39.2/-. Slabs of 4 planes deal every
// XCD a stretch of rows of the same few planes. On a 32^3 grid the slabs lose
// (0.69 ms in turn, 0.72-0.77 overlapped): kernels of a few thousand waves
// end before the other stream's work can fill the chip, so small grids keep
// the two phases in turn.
#include "mm_contract.h"

#include <mutex>

namespace mmk {

namespace {

constexpr int kSlabPlanes = 4;  // bin planes per slab (even: the fp64 kernel pairs planes)
constexpr int kMaxSlabs = 256;
constexpr int kMinPlaneBins = 8192;  // bins per plane below which the phases run in turn
constexpr int kMaxDev = 64;

// The second stream of a device and the events of one call (default
// priority; non-blocking, so that work on the legacy null stream does not
// serialise it; the events carry no timing).
struct Side {
  hipStream_t st = nullptr;
  hipEvent_t ev[kMaxSlabs + 2] = {};
  bool ready = false;
};
Side sides[kMaxDev];
// Held while a call enqueues: the calls on one device share its events.
std::mutex side_mu;

hipError_t side_of(hipStream_t s, Side** out) {
  int dev = -1;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  Side& sd = sides[dev];
  if (!sd.ready) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    Side nw;
    int nev = 0;
    e = hipStreamCreateWithFlags(&nw.st, hipStreamNonBlocking);
    for (; e == hipSuccess && nev < kMaxSlabs + 2; ++nev) e = hipEventCreateWithFlags(&nw.ev[nev], hipEventDisableTiming);
    if (e != hipSuccess) {  // release what was created; a later call tries again
      for (int i = 0; i < nev; ++i)
        if (nw.ev[i]) (void)hipEventDestroy(nw.ev[i]);
      if (nw.st) (void)hipStreamDestroy(nw.st);
    }
    if (e == hipSuccess) {
      nw.ready = true;
      sd = nw;
    }
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
  }
  *out = &sd;
  return hipSuccess;
}

// Planes per slab: kSlabPlanes, more on grids of more than kMaxSlabs slabs (kept even).
int slab_planes(const GridDev& g) {
  int p = (g.n2 + kMaxSlabs - 1) / kMaxSlabs;
  p = p < kSlabPlanes ? kSlabPlanes : p;
  return p + (p & 1);
}

}  // namespace

int overlap_slabs(const GridDev& g) {
  if (!tsc_run_records(g) || g.n0 * g.n1 < kMinPlaneBins) return 0;
  const int p = slab_planes(g);
  const int n = (g.n2 + p - 1) / p;
  return n >= 4 ? n : 0;
}

int overlap_slab_planes(const GridDev& g) { return overlap_slabs(g) > 0 ? slab_planes(g) : 0; }

hipError_t launch_assemble_overlapped(const GridDev& g, bool f32, const Particles& P, const int32_t* bin_start,
                                      const int32_t* perm, double beta, double sigma, void* rec, int accumulate,
                                      void* M, hipStream_t s) {
  const int nslab = overlap_slabs(g);
  if (nslab < 2 || nslab > kMaxSlabs || !contract_planes_apply(g, 2, f32, P)) return hipErrorInvalidValue;
  const int pz = slab_planes(g);
  std::lock_guard<std::mutex> lock(side_mu);
  Side* sd = nullptr;
  hipError_t e = side_of(s, &sd);
  if (e != hipSuccess) return e;
  // the second stream starts after everything enqueued on s so far
  if ((e = hipEventRecord(sd->ev[0], s)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(sd->st, sd->ev[0], 0)) != hipSuccess) return e;
  const void* recs[1] = {rec};
  hipError_t err = hipSuccess;
  for (int k = 0; k < nslab && err == hipSuccess; ++k) {
    const int z0 = k * pz, z1 = (k + 1) * pz < g.n2 ? (k + 1) * pz : g.n2;
    err = launch_contract_planes(g, f32, P, bin_start, perm, beta, sigma, rec, z0, z1, s);
    if (err != hipSuccess) break;
    if ((err = hipEventRecord(sd->ev[k + 1], s)) != hipSuccess) break;
    if ((err = hipStreamWaitEvent(sd->st, sd->ev[k + 1], 0)) != hipSuccess) break;
    // node planes completed by this slab (2 .. z1 - 1 after the first)
    err = launch_gather_run(g, recs, 1, accumulate, M, sd->st, false, f32, k == 0 ? 2 : z0, z1);
    if (err == hipSuccess && k == nslab - 1)  // node planes 0 and 1 read the last bin planes
      err = launch_gather_run(g, recs, 1, accumulate, M, sd->st, false, f32, 0, 2);
  }
  // the caller's stream waits for the second one, also after an error
  if ((e = hipEventRecord(sd->ev[kMaxSlabs + 1], sd->st)) == hipSuccess)
    e = hipStreamWaitEvent(s, sd->ev[kMaxSlabs + 1], 0);
  return err != hipSuccess ? err : e;
}

}  // namespace mmk
