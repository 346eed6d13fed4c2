// gemm_dl_index.hpp -- index maps of the direct-to-LDS bf16 GEMM (plain C++,
// usable on the host: the layout is checked exhaustively by a CPU test).
//
// Tile of one operand per pipeline stage: 256 rows (the M or N index) x 32 k
// of bf16 = 16 KB, written by 16 wave-wide global_load_lds_dwordx4
// instructions (each puts lane i's 16 bytes at the instruction's LDS base +
// 16 i) and read back as v_mfma_f32_32x32x16_bf16 operands: lane l needs the
// 8 values (row l % 32, k = 8 (l / 32) .. + 7) of its 32-row block.
//
// K-contiguous operand (X[r][k], k fastest): LDS tile [256 rows][4 chunks of
// 8 k] (64 bytes a row).  Chunk c of row r sits in slot c ^ ((r >> 2) & 3),
// which spreads the 16 rows read together by a quarter-wave over all 64
// banks.  Operand fetch: one ds_read_b128 per 8 values.
//
// K-outer operand (X[k][r], r fastest): LDS tile [32 k-rows][32 chunks of
// 8 r] (512 bytes a k-row).  Chunk c of k-row p sits in slot c ^ (4 (p & 3)).
// Operand fetch: two ds_read_b64_tr_b16 per 8 values.  That instruction
// works on 16-lane groups: lane j of a group receives element j % 4 of the
// 8-byte pieces addressed by lanes j / 4, j / 4 + 4, j / 4 + 8, j / 4 + 12 of
// its group, in that order.  So in group g (lanes 16 g .. 16 g + 15) lane
// s supplies the address of the 4 values (k-row kb + s / 4, r = 16 (g % 2) +
// 4 (s % 4) .. + 3), where kb = 8 (g / 2) + 4 h for the two halves h; lane
// l then holds (r = l % 32, k = 8 (l / 32) + 4 h .. + 3).  An 8-byte LDS read
// is served 32 lanes at a time over the 64 banks: those lanes read the same
// four k-rows, 64 bytes of each; the swizzle moves each k-row's 64 bytes to
// its own quarter of the 256-byte bank window.
#pragma once

#include <stdint.h>

namespace gdl {

constexpr int kRows = 256;        // rows of an operand tile
constexpr int kBK = 32;           // k per pipeline stage
constexpr int kTileBytes = kRows * kBK * 2;
constexpr int kInstrPerTile = kTileBytes / 1024;  // wave-wide 16-byte loads

// ---- K-contiguous tiles ------------------------------------------------

// Slot of chunk c (8 k) in LDS row r.
constexpr int kc_slot(int r, int c) { return c ^ ((r >> 2) & 3); }

// Load instruction gi (0..15), lane i: the tile row and the k-chunk it fetches.
constexpr int kc_load_row(int gi, int i) { return 16 * gi + i / 4; }
constexpr int kc_load_chunk(int gi, int i) { return kc_slot(kc_load_row(gi, i), i % 4); }

// Byte offset, within the tile, of lane l's 16-byte operand piece for row
// block `rb` (a multiple of 32 rows, given in rows) and k sub-step q (0, 1:
// k = 16 q .. 16 q + 15).
constexpr int kc_read_off(int l, int rb, int q) {
  return (rb + (l & 31)) * 64 + 16 * kc_slot(rb + (l & 31), 2 * q + (l >> 5));
}

// ---- K-outer tiles -----------------------------------------------------

// Slot of chunk c (8 r) in LDS k-row p.
constexpr int ko_slot(int p, int c) { return c ^ (4 * (p & 3)); }

// Load instruction gi (0..15), lane i: the k-row and the r-chunk it fetches.
constexpr int ko_load_krow(int gi, int i) { return 2 * gi + i / 32; }
constexpr int ko_load_chunk(int gi, int i) { return ko_slot(ko_load_krow(gi, i), i % 32); }

// Byte offset, within the tile, of the 8-byte piece lane l supplies to the
// h-th transposed read of row block `rb` (multiple of 32, in rows) and k
// sub-step q.
constexpr int ko_read_off(int l, int rb, int q, int h) {
  const int g = l >> 4, s = l & 15;
  const int p = 16 * q + 8 * (g >> 1) + 4 * h + (s >> 2);
  const int r = rb + 16 * (g & 1) + 4 * (s & 3);
  return p * 512 + 16 * ko_slot(p, r >> 3) + 2 * (r & 7);
}

}  // namespace gdl
