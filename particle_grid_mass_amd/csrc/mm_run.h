// Records of x-runs of four second-order bins: the layout shared by the TSC
// contraction that writes them (k_tsc64.hip) and the deposit that reads them
// (k_gather_run.hip).
//
// Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for Implicit
// Particle-In-Cell Methods": each support group's local matrix (Sec. 3.1,
// Eq. 15) is scattered into the stencil storage (Sec. 3.4), and the matrix is
// symmetric node pair by node pair (Table 1 and its footnote), so only the
// canonical half of the pairs is kept.
//
// A run is four bins with consecutive x (first support nodes kx = 4r .. 4r+3,
// same y and z). Their supports cover the 6 x 3 x 3 union nodes (X, Y, Z),
// X in [0, 6) relative to node 4r. A run record holds, for every canonical
// node pair of the union that some bin of the run covers, the sum of the
// bins' local matrices: 999 entries instead of 4 x 378 pair records, a third
// fewer bytes to write and to read back.
//
// Entry numbering: by the row node's Z and Y, then the (dY, dZ) row of the
// canonical offset d = (dX, dY, dZ) >= 0 ((dZ, dY, dX) lexicographic; 13 rows,
// the first, d = (dX, 0, 0), holding dX >= 0 only), then X, then dX. For
// fixed (Z, Y, row) the valid (X, dX) (X and X + dX in [0, 6)) form one
// segment. A deposit wave shares the (dY, dZ) row and covers nodes x times
// the five dX, so each term it reads is one contiguous stretch.
//
// Storage (doubles): the entries of one row node position (Z, Y) form a
// slice; slice s = 3 Z + Y keeps its nine component planes one after the
// other, rec[run][slice][comp][entry in slice], each plane padded to a
// multiple of 16 values (a 128-byte line) so that every plane starts a cache
// line. A contraction wave owning row i writes its three components, each as
// nine line-aligned stretches; a deposit block reads, for a node row, the
// slice of each record row it needs, and no line is shared with the slice of
// another node row (slices that shared lines were fetched about 1.2 times).
#pragma once

#include <stdint.h>

namespace mmk {
namespace run {

constexpr int RUN = 4;                 // bins per run (consecutive x)
constexpr int UX = RUN + 2;            // node columns of the union support
constexpr int NENT = 999;              // canonical union entries per run
// entries of slice s = 3 Z + Y (the canonical offsets whose partner node
// stays in the union: 24 per full (dY, dZ) row, 15 in the d = (dX, 0, 0) row)
constexpr int slice_len(int s) {
  const int Z = s / 3, Y = s % 3;
  int n = 0;
  for (int row = 12; row < 25; ++row) {
    const int dy = row % 5 - 2, dz = row / 5 - 2;
    if (Z + dz >= 0 && Z + dz < 3 && Y + dy >= 0 && Y + dy < 3) n += row == 12 ? 15 : 24;
  }
  return n;
}
constexpr int slice_pad(int s) { return (slice_len(s) + 15) / 16 * 16; }  // plane stride in the slice
constexpr int slice_start(int s) { return s == 0 ? 0 : slice_start(s - 1) + slice_len(s - 1); }  // first entry
constexpr int slice_base(int s) { return s == 0 ? 0 : slice_base(s - 1) + 9 * slice_pad(s - 1); }  // storage
constexpr int RUNREC = slice_base(9);  // doubles per run record (9 x 1040)
constexpr int CENTRE = 62;             // full offset index of d = 0
constexpr int ROW0 = CENTRE / 5;       // (dY, dZ) row of d = (dX, 0, 0): full offset index / 5
constexpr int NROW = 25 - ROW0;        // (dY, dZ) rows holding canonical offsets
constexpr int NPAIR = 378;             // packed upper triangle of one bin's 27 x 27 matrix

// Packed upper triangle of a bin's 27 support rows: pair(a, b), a <= b.
constexpr int pair_index(int a, int b) { return a * 27 - (a * (a - 1)) / 2 + (b - a); }

// Where the contraction parks one component of the four bins' local matrices
// for the summation over bins: the 4x4 blocks (I, J), I <= J, of the 27 rows
// padded to 28, as the matrix instruction leaves them, block k (row-major over
// the upper blocks) of bin b at b * BSTRIDE + 16 k, entry (i, j) of the block
// at 4 i + j. Each lane then stores its 28 accumulators at one base address
// plus constant offsets. Entry (27, 27), the padding row against the padding
// column, is an exact zero: it is the slot read for a bin that does not hold
// an entry. BSTRIDE = 448 + 16 puts the four bins of one store on alternate
// halves of the LDS banks.
constexpr int NBLKR = 7;                              // row blocks of 4
constexpr int BSTRIDE = 464;                          // slots per bin
constexpr int ZERO0 = 27 * 16 + 15;                   // bin 0's (27, 27)
constexpr int ZERO1 = BSTRIDE + ZERO0;                // bin 1's (27, 27)
constexpr int upper_block(int I, int J) { return I * NBLKR - (I * (I - 1)) / 2 + (J - I); }
constexpr int block_slot(int bin, int a, int b) {
  return bin * BSTRIDE + 16 * upper_block(a / 4, b / 4) + 4 * (a % 4) + b % 4;
}
// The same with each block stored transposed (entry (i, j) at 4 j + i): the
// layout in which the fp32 4x4x1 instruction leaves a lane's four values of a
// block (one column) contiguous, so a lane parks a block with one 16-byte store.
constexpr int block_slot_t(int bin, int a, int b) {
  return bin * BSTRIDE + 16 * upper_block(a / 4, b / 4) + 4 * (b % 4) + a % 4;
}
static_assert(upper_block(6, 6) == 27 && block_slot(0, 27, 27) == ZERO0 && block_slot(1, 27, 27) == ZERO1 &&
                  block_slot_t(0, 27, 27) == ZERO0 && block_slot_t(1, 27, 27) == ZERO1,
              "the padding entries serve as zero slots");

// Smallest dX of node column X (X + dX >= 0; dX >= 0 in the first row).
constexpr int dx_min(int X, bool first_row) { return first_row ? 0 : (X < 2 ? -X : -2); }
// Largest dX of node column X (X + dX < 6).
constexpr int dx_max(int X) { return 5 - X < 2 ? 5 - X : 2; }

struct Tables {
  short seg_start[9 * NROW];  // first entry of segment (Z, Y, row): [(3 Z + Y) * NROW + row - ROW0]; -1: none
  unsigned char col_start[2][UX + 1];  // entries before column X in a segment: [first row?][X]
  // per entry: the block slots (block_slot) of its value in the bins b0 ..
  // b0 + n - 1 of the run that hold both nodes, both nodes one column further
  // left in each next bin: q0 (bits 0..10), q1 - ZERO0 (bits 11..21) and
  // q2 - ZERO1 (bits 22..31), q1 = ZERO0 when n < 2 and q2 = ZERO1 when n < 3
  unsigned contrib[NENT];
  unsigned contrib_t[NENT];  // the same slots in the transposed block layout (block_slot_t)
  // per entry: the byte offset of its component 0 in the run record (bits
  // 0..16) and the plane stride of its slice in 128-byte lines (bits 17..21);
  // component c is stored c plane strides further on
  unsigned store_bytes[NENT];
  unsigned char nbins[NENT];  // n of each entry (1 to 3)
  int slice_off[9];  // storage offset of slice s minus its first entry index
  int slice_stride[9];  // plane stride of slice s (slice_pad)
  int count;  // entries numbered
};

constexpr Tables make_tables() {
  Tables t{};
  for (int f = 0; f < 2; ++f) {
    int c = 0;
    for (int X = 0; X < UX; ++X) {
      t.col_start[f][X] = (unsigned char)c;
      c += dx_max(X) - dx_min(X, f == 1) + 1;
    }
    t.col_start[f][UX] = (unsigned char)c;
  }
  int e = 0;
  for (int Z = 0; Z < 3; ++Z)
    for (int Y = 0; Y < 3; ++Y)
      for (int row = ROW0; row < 25; ++row) {
        const int dy = row % 5 - 2, dz = row / 5 - 2;
        const bool ok = Z + dz >= 0 && Z + dz < 3 && Y + dy >= 0 && Y + dy < 3;
        t.seg_start[(3 * Z + Y) * NROW + row - ROW0] = ok ? (short)e : (short)-1;
        if (!ok) continue;
        for (int X = 0; X < UX; ++X)
          for (int dx = dx_min(X, row == ROW0); dx <= dx_max(X); ++dx, ++e) {
            int q[3] = {0, ZERO0, ZERO1}, qt[3] = {0, ZERO0, ZERO1}, n = 0;
            for (int b = 0; b < RUN; ++b) {
              const int ax = X - b, bx = X + dx - b;
              if (ax < 0 || ax > 2 || bx < 0 || bx > 2) continue;
              const int na = ax + 3 * Y + 9 * Z, nb = bx + 3 * (Y + dy) + 9 * (Z + dz);
              qt[n] = block_slot_t(b, na, nb);
              q[n++] = block_slot(b, na, nb);
            }
            t.contrib[e] = (unsigned)q[0] | ((unsigned)(q[1] - ZERO0) << 11) | ((unsigned)(q[2] - ZERO1) << 22);
            t.contrib_t[e] =
                (unsigned)qt[0] | ((unsigned)(qt[1] - ZERO0) << 11) | ((unsigned)(qt[2] - ZERO1) << 22);
            t.nbins[e] = (unsigned char)n;
            const int sl = 3 * Z + Y;
            t.store_bytes[e] = (unsigned)(8 * (slice_base(sl) + e - slice_start(sl))) | ((unsigned)(slice_pad(sl) / 16) << 17);
          }
      }
  for (int sl = 0; sl < 9; ++sl) {
    t.slice_off[sl] = slice_base(sl) - slice_start(sl);
    t.slice_stride[sl] = slice_pad(sl);
  }
  t.count = e;
  return t;
}

static_assert(make_tables().count == NENT, "canonical union entries of a run of four bins");

// Every encoded slot fits its field, and every entry gathers the first slot
// of its bins in the upper triangle of a block (i <= j on the diagonal).
constexpr bool contrib_fits() {
  const Tables t = make_tables();
  int total = 0;
  for (int e = 0; e < NENT; ++e) {
    const unsigned c = t.contrib[e];
    const int q0 = (int)(c & 2047u), q1 = (int)((c >> 11) & 2047u) + ZERO0, q2 = (int)(c >> 22) + ZERO1;
    const int n = t.nbins[e];
    if (n < 1 || n > 3 || q0 >= RUN * BSTRIDE || q1 >= RUN * BSTRIDE || q2 >= RUN * BSTRIDE) return false;
    if ((n < 2) != (q1 == ZERO0) || (n < 3) != (q2 == ZERO1)) return false;
    if (q0 % 16 / 4 > q0 % 4 && (q0 % BSTRIDE) / 16 < NBLKR * (NBLKR + 1) / 2) {
      // a slot left of the diagonal inside a diagonal block is never read
      const int k = (q0 % BSTRIDE) / 16;
      for (int I = 0; I < NBLKR; ++I)
        if (upper_block(I, I) == k) return false;
    }
    total += n;
  }
  return total == RUN * NPAIR;  // each bin value is read exactly once
}
static_assert(contrib_fits(), "run table encoding");
static_assert(slice_start(9) == NENT && RUNREC == 9 * 1040 && RUNREC % 2 == 0, "slices of a run record");
static_assert(8 * RUNREC < (1 << 17), "record byte offsets fit the store table's field");
static_assert(make_tables().col_start[0][UX] == 24 && make_tables().col_start[1][UX] == 15, "segment lengths");

}  // namespace run
}  // namespace mmk
