// gdn_tiles.h -- LDS tile layouts for 16-bit operand tiles without padding.
//
// A tile is rows x COLS elements of 2 bytes, row-major, with the 16-byte "octets" of each row
// permuted by an XOR so that the accesses the kernels make touch distinct LDS banks:
//
//  * Matrix-core operand reads take, in one instruction, one octet from each of 16 rows.
//    With the pair-row mapping (rows 32G + 8(i/4) + 4t + i%4 for lane row i) the swizzles
//    below give those 16 rows 16 distinct bank groups (256-byte rows: distinct octets;
//    128-byte rows: distinct (row parity, octet) pairs, since two such rows share one pass
//    over the banks).
//  * Transposed stores (one token per lane, the same tile row for the whole wave) write one
//    full row per instruction, which is conflict-free under any permutation of its octets.
//  * Row-wise 16-byte stores (16 lanes per row) write a permutation of one row.
#pragma once

namespace gdn {

// octet permutation for tiles whose rows are read 16 at a time in pair-row order
template <int COLS>
__device__ __forceinline__ int swz_pair(int r) {
  if constexpr (COLS == 128) return (r & 3) | (((r >> 3) & 3) << 2);   // 16 octets per row
  else return ((r >> 1) & 1) | (((r >> 3) & 3) << 1);                  // 8 octets per row
}

// octet permutation for 128-byte-row tiles whose rows are read 16 consecutive at a time
__device__ __forceinline__ int swz_seq(int r) { return (r >> 1) & 7; }

template <int COLS>
__device__ __forceinline__ int tix_pair(int r, int c) {
  return r * COLS + ((((c >> 3) ^ swz_pair<COLS>(r))) << 3) + (c & 7);
}

__device__ __forceinline__ int tix_seq64(int r, int c) {
  return r * 64 + (((c >> 3) ^ swz_seq(r)) << 3) + (c & 7);
}

// Octet permutation of row r in the column-split tiles below.  Measured on gfx950 with the
// LDS bank-conflict counter (a 16-byte read serves 16 lanes per cycle, an 8-byte read 32):
// 16-byte reads of one octet from 16 consecutive rows, or from the pair rows
// 32G + 8(i/4) + 4t + i%4, run conflict-free with this permutation.  Transposed 8-byte reads
// of eight rows x four octets at one 8-byte half take two cycles per pass under any octet
// permutation (their 32 lanes cover half of the bank slots).
__device__ __forceinline__ int swz64(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// Column-split tile: [R rows][W columns] kept as W/32 sub-tiles of [R][32] (64-byte rows),
// sub-tile s at element s*R*32; octet o (0..3) of row r inside a sub-tile is stored at
// o ^ swz64(r).  A sub-tile offset is then a constant (an instruction immediate).
template <int R>
__device__ __forceinline__ int tix_s32(int r, int c) {
  return (c >> 5) * (R * 32) + r * 32 + ((((c >> 3) & 3) ^ swz64(r)) << 3) + (c & 7);
}

// Column-split [64][W] tile (W a multiple of 32) whose octets are permuted by
// ((r >> 2) ^ (r >> 3)) & 3.  16-byte reads of one octet from 16 consecutive rows or from the
// pair rows 32G + 8i + 4t + j hit 16 distinct bank groups, and transposed 8-byte reads of four
// consecutive rows x four octets hit 16 distinct 8-byte slots.
__device__ __forceinline__ int tix_x64(int r, int c) {
  return (c >> 5) * (64 * 32) + r * 32 + ((((c >> 3) & 3) ^ (((r >> 2) ^ (r >> 3)) & 3)) << 3) + (c & 7);
}

}  // namespace gdn
