// red_layout.hpp -- placement of the per-wavefront transpose buffer through
// which the reverse walk sums db_n = sum_p mu x and dc_n = sum_p g h over a
// wavefront's channels (plain C++, usable on the host: the placement is
// checked exhaustively by a CPU test).
//
// Logical buffer: OUT = 2 NN rows (db of state n, then dc of state n) by CH
// columns (the wavefront's channels).  Writes: for state j of its group, lane
// (grp, pl) stores one float at row grp NL + j (and NN + grp NL + j), column
// pl -- one ds_write_b32 per row, all 64 lanes.  Reads: lane l sums row
// l / LPO, columns (l % LPO) V .. + V - 1, LPO = 64 / OUT lanes per row.
//
// Every address is a per-lane base plus a per-instruction constant
// (row_off(part, j) + lane_base(grp, pl) for writes, row_start(o) + 4 c for
// reads), so the kernel keeps one address register per access kind and the
// constants become instruction offsets.
//
// General shapes pad each row to CH + 1 floats (rows start on every bank).
// For NL = 8, G = 2 (CH = 32, OUT = 32, V = 16) the lane's 16 values are read
// as four 16-byte pieces, and all accesses are kept free of bank conflicts
// (64 banks of 4 bytes; a 16-byte read is served 16 lanes per pass, a 4-byte
// write 64 lanes per pass, and a two-address ds_write2_b32 -- into which the
// compiler merges the writes of rows 2i and 2i + 1 -- 32 lanes per pass):
//   * rows are 32 floats, row j of a group starting at row_j(j) floats, whose
//     bank quads (row_j / 4 mod 16 = 0, 8, 1, 9, 2, 10, 3, 11) and the same
//     plus 4 (the second half of a row) are 16 distinct quads: the 8 rows one
//     read pass covers (one group, one part) never share a quad;
//   * rows 2i and 2i + 1 start 32 banks apart, so a merged write of both by
//     one group's 32 lanes covers all 64 banks;
//   * the second group's rows sit 288 floats (32 banks mod 64) after the
//     first's, so a single write instruction (rows j and 8 + j) covers all 64
//     banks.
#pragma once

namespace redl {

// floats of the buffer for NL states per lane and G lane groups
constexpr int floats(int NL, int G) { return (NL == 8 && G == 2) ? 4 * 288 : 2 * NL * G * (64 / G + 1); }

template <int NL, int G>
struct Layout {
  static constexpr int CH = 64 / G;
  static constexpr int NN = NL * G;
  static constexpr int OUT = 2 * NN;
  static constexpr bool kSwz = (NL == 8 && G == 2);
  static constexpr int kRS = CH + 1;  // padded layout: floats per row
  static constexpr int kGroup = 288;  // unpadded layout: floats per group block
  static constexpr int kFloats = floats(NL, G);
  static_assert(kFloats == (kSwz ? 4 * kGroup : OUT * kRS), "buffer size");

  // row j of a group starts at 0, 32, 68, 100, 136, 168, 204, 236 floats
  // (written as arithmetic: a table indexed by a lane-dependent row would be
  // placed in global memory and read back with a load)
  static constexpr int row_j(int j) { return 68 * (j >> 1) + 32 * (j & 1); }
  // constant part of a write address: state j of a group, part 0 (db) or 1 (dc)
  static constexpr int row_off(int part, int j) { return kSwz ? part * 2 * kGroup + row_j(j) : (part * NN + j) * kRS; }
  // per-lane part of a write address
  static constexpr int lane_base(int grp, int pl) { return kSwz ? grp * kGroup + pl : grp * NL * kRS + pl; }
  // start of logical row `row`
  static constexpr int row_start(int row) {
    return row_off(row / NN, row % NL) + lane_base((row % NN) / NL, 0);
  }
  // float index of (row, col)
  static constexpr int at(int row, int col) { return row_start(row) + col; }
  // float index of 4-float chunk c (columns 4 c .. 4 c + 3) of a row
  static constexpr int chunk(int row, int c) { return row_start(row) + 4 * c; }
};

}  // namespace redl
