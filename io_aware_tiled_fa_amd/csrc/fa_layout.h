// LDS tile layouts of the attention kernels and the per-lane offsets the
// kernels read and copy them with.  Integer arithmetic only, with no HIP
// include, so the host-side layout checks can compile this file as plain
// C++ (defining __device__ and __forceinline__ away).
//
// Facts of gfx950 these layouts are built for:
//  * v_mfma_f32_32x32x16_bf16 (wave64): lane l holds A[l % 32][8 (l / 32) + e]
//    and B[8 (l / 32) + e][l % 32], e = 0..7; only the pairing of A's and B's
//    contraction index matters, so both may relabel it the same way.
//  * ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element
//    i % 4 of the 8-byte chunks read by lanes i / 4, i / 4 + 4, i / 4 + 8 and
//    i / 4 + 12 of its group.
//  * The LDS serves 16-byte accesses 8 lanes per cycle and 8-byte accesses 16
//    lanes per cycle, over 32 banks of 4 bytes (measured: a layout that is
//    conflict free only for 32 lanes over 64 banks shows 2-way conflicts).
#pragma once

namespace fa {

// Row-group layout of a [rows][D] bf16 tile.  The tile is cut into 128-byte
// blocks of 4 consecutive rows by 2 consecutive 16-byte pieces (16
// columns): block (rg, pp) of row group rg = row / 4 and piece pair pp sits
// at (rg D/16 + (pp ^ ((rg >> 1) & 1))) * 128, the rows of a block 32 bytes
// apart, and the two pieces of a pair swapped when rg is odd.  Then
//  * the 4 rows x 16 columns that a 16-lane group reads with
//    ds_read_b64_tr_b16 form one block, 128 contiguous bytes;
//  * one 16-byte piece of 8 consecutive rows lands in 8 different groups
//    of 4 of 32 banks (16 rows in 16 groups of 64 banks), so 16-byte reads
//    of a column of pieces are conflict free;
//  * offsets split into a per-lane base plus compile-time steps: 256 bytes
//    per 32 columns, 32 ROWB per 32 rows (ROWB = 2 D bytes per row), and for
//    the pieces 2 kk + h of one row a base per parity of kk plus 256 (kk / 2).
template <int D>
__device__ __forceinline__ int rg_off(int row, int piece) {
  const int rg = row >> 2;
  const int pp = (piece >> 1) ^ ((rg >> 1) & 1);
  return (rg * (D / 16) + pp) * 128 + (row & 3) * 32 + (((piece & 1) ^ (rg & 1)) << 4);
}
// the row and piece stored at 16-byte slot `slot` of the tile (the inverse);
// slot s + r D / 8 holds the piece of slot s, r rows further down, whenever
// r is a multiple of 16
template <int D>
__device__ __forceinline__ void rg_slot(int slot, int& row, int& piece) {
  const int blk = slot >> 3, w = slot & 7;
  const int rg = blk / (D / 16), pp = (blk % (D / 16)) ^ ((rg >> 1) & 1);
  row = 4 * rg + (w >> 1);
  piece = 2 * pp + ((w & 1) ^ (rg & 1));
}

// 16-byte row reads of the A (or B) operand, lane l = row l % 32: piece
// 2 kk + l / 32 of that row at rg_row_base(l, kk & 1) + 256 (kk / 2) (+ 32 ROWB
// per further 32 rows)
template <int D>
__device__ __forceinline__ int rg_row_base(int lane, int parity) {
  return rg_off<D>(lane & 31, 2 * parity + (lane >> 5));
}

// Transpose reads of a 16-row step: lane l (group g = l / 16, j = l % 16,
// h = l / 32) reads the 8-byte chunk of row 4 h + j / 4 + 8 r at columns
// 32 db + 16 (g % 2) + 4 (j % 4), at rg_tr_base(l, r) + 256 db + 16 t ROWB for
// the rows 16 t ..  Reads r = 0 and 1 together hand lane l the column
// 32 db + l % 32 at rows 16 t + 4 h + (0..3) and 16 t + 8 + 4 h + (0..3): a B
// operand whose contraction index e = 4 r + i stands for row 8 r + 4 h + i.
template <int D>
__device__ __forceinline__ int rg_tr_base(int lane, int r) {
  const int g = lane >> 4, j = lane & 15, h = lane >> 5;
  return rg_off<D>(4 * h + (j >> 2) + 8 * r, 2 * (g & 1) + ((j & 3) >> 1)) + 8 * (j & 1);
}

// P^T / dS^T tiles of the dK / dV kernel: 128 key rows of 32 queries (64 B),
// in 8-byte chunks of 4 queries, chunk c of row r at c ^ s(r) with
// s(r) = 4 r3 + 2 r2 + (r1 ^ r4) (r_i the bits of r).  Producers and
// consumers move whole chunks, one key row per lane: any 16 consecutive rows
// then hit 16 distinct bank pairs.  Byte offset of query q of row r; the
// chunk of queries q0 + 4 k (q0 a multiple of 4, k and q0 / 4 with no set
// bit in common) is at pt_off(r, q0) ^ 8 k.
__device__ __forceinline__ int pt_off(int row, int q) {
  const int s = ((row >> 1) & 6) | (((row >> 1) ^ (row >> 4)) & 1);
  return row * 64 + (((q >> 2) ^ s) << 3) + 2 * (q & 3);
}

// Staging of 32 output rows (2 D bytes each) in the epilogues: lane l of a
// wave holds four consecutive d = 32 db + 8 g4 + 4 (l / 32) .. of row
// l % 32 and writes them as 8-byte half l / 32 of the row's 16-byte piece
// 4 db + g4; D / 8 lanes then read each row back a piece apiece.  Piece p
// of row r sits at slot stage_slot(r, p) of the row, its two halves swapped
// when stage_swap(r) is set (the reader swaps them back): the 8-byte writes
// of 16 (32) lanes then land in distinct banks of 32 (64), and so do the
// 16-byte reads of 8 (16) lanes.
template <int D>
__device__ __forceinline__ int stage_slot(int row, int piece) {
  static_assert(D == 64 || D == 128, "head dimension 64 or 128");
  return D == 128 ? piece ^ (row & 15) : piece ^ ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int stage_swap(int row) {
  return D == 128 ? ((row >> 3) ^ (row >> 4)) & 1 : (row ^ (row >> 4)) & 1;
}
template <int D>
__device__ __forceinline__ int stage_off(int row, int piece, int half) {
  return row * 2 * D + (stage_slot<D>(row, piece) << 4) + 8 * (half ^ stage_swap<D>(row));
}

}  // namespace fa
