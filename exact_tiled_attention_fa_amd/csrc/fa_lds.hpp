// LDS layouts of the attention kernels' tiles: the XOR each kernel applies to
// a tile row's 16-byte chunk index.  Plain integer code with no HIP
// dependency, so that host-side checks replay the kernels' LDS accesses with
// the same functions.
//
// Bank model: gfx950's LDS has 64 banks of 4 bytes, and an access is served
// 256 bytes at a time (16 lanes of a 16-byte access, 32 lanes of an 8-byte
// one, 64 of a 4-byte one).  Lanes of one such group that touch the same bank
// at different addresses serialise.  Every XOR below is a bijection on the
// chunk indices of a row, so a tile holds each element exactly once.
#pragma once

#if defined(__HIP__)
#define FA_HD __host__ __device__
#else
#define FA_HD
#endif

namespace fa {

// Rows of N chunks read 16 consecutive rows at one logical chunk (the decode
// kernel's K tile, its merge rows): rows that share a 256-byte bank row
// (16 / N of them when N < 16) get distinct chunks.
template <int N> FA_HD inline int row_xor(int r) {
  return N >= 16 ? (r & 15) : ((r / (16 / N)) & (N - 1));
}

// The decode kernel's 16-bit V tile ([16][D]).  A transpose read of 32 lanes
// touches chunks 2m, 2m+1 of 8 consecutive rows, so the bits above bit 0
// spread the rows' chunk pairs; bit 0 alternates between the rows that a
// 16-lane store of widened int8 codes covers together (its first store writes
// chunk 2c of each row), so those rows land on even and odd chunks.
template <int D> FA_HD inline int swz_dv(int r) {
  return D == 64 ? (2 * ((r >> 1) & 3) | ((r >> 1) & 1)) : (2 * (r & 7) | (r & 1));
}

// The backward kernels' Q / dO / K tiles ([32][D]), read two ways: by rows
// (16 lanes read one logical chunk of 16 consecutive rows) and by transpose
// reads (32 lanes read logical chunks 4m .. 4m+3 of 4 consecutive rows, 8
// bytes each).  At D >= 128 a row spans all 64 banks, so the 16 rows need 16
// distinct values, and the 4 rows' values must differ above bit 1 so that
// their chunk quads are disjoint: the value swaps the two 2-bit halves of the
// row's low four bits.  At D = 64 two rows share the banks (odd rows on the
// upper half), so the value is a permutation of r >> 1 whose bit 2 separates
// rows 2 apart.
template <int D> FA_HD inline int swz_b(int r) {
  if (D >= 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  const int x = (r >> 1) & 7;
  return ((x & 1) << 2) | (x >> 1);
}

// The FP8 forward's K tile (rows of D bytes, D/16 chunks).  The 16 lanes of an
// A-operand read take rows {0..7} + {0, 16} (+8, +32) at one logical chunk,
// and rows that share a 256-byte bank row (256 / D of them) must get distinct
// chunks: the XOR takes the row bits above those (within 0..7) and bit 4.
template <int D> FA_HD inline int swz_k8(int r) {
  if (D == 64) return ((r >> 2) & 1) | (((r >> 4) & 1) << 1);
  if (D == 128) return ((r >> 1) & 3) | (((r >> 4) & 1) << 2);
  return (r & 7) | (((r >> 4) & 1) << 3);
}

// The FP8 forward's V^T tile: rows of 64 bytes (4 chunks, four rows per bank
// row); a read takes 16 consecutive rows at one logical chunk, so rows 4
// apart get distinct chunks.
FA_HD inline int swz_v8(int d) { return (d >> 2) & 3; }

}  // namespace fa
