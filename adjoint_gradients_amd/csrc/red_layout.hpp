// red_layout.hpp -- placement of the per-wavefront transpose buffer through
// which the reverse walk sums db_n = sum_p mu x and dc_n = sum_p g h over a
// wavefront's channels (plain C++, usable on the host: the placement is
// checked exhaustively by a CPU test).
//
// Logical buffer: OUT = 2 NN rows (db of state n, then dc of state n) by CH
// columns (the wavefront's channels).  Writes: for state j of its group, lane
// (grp, pl) stores one float at row grp NL + j (and NN + grp NL + j), column
// pl -- one ds_write_b32 per row pair, all 64 lanes.  Reads: lane l sums row
// l / LPO, columns (l % LPO) V .. + V - 1, LPO = 64 / OUT lanes per row.
//
// General shapes pad each row to CH + 1 floats (rows start on every bank).
// For NL = 8, G = 2 (CH = 32, OUT = 32, V = 16) rows are unpadded and the
// lane's 16 values are fetched as four 16-byte reads, so the placement must
// keep both access kinds free of bank conflicts (64 banks of 4 bytes; a
// 16-byte read is served 16 lanes per pass, a 4-byte write 64 lanes):
//   * physical row pr = row ^ ((row >> 3) & 1): the two groups' rows j and
//     8 + j get opposite parity, so one write instruction covers all 64 banks;
//   * 4-float chunk c of a row sits in slot c ^ ((pr >> 1) & 3): the 8 rows read
//     in one pass (4 of each parity) put their chunks on 16 distinct bank quads.
#pragma once

namespace redl {

template <int NL, int G>
struct Layout {
  static constexpr int CH = 64 / G;
  static constexpr int NN = NL * G;
  static constexpr int OUT = 2 * NN;
  static constexpr bool kSwz = (NL == 8 && G == 2);
  static constexpr int kRS = kSwz ? CH : CH + 1;  // floats per row
  static constexpr int kFloats = OUT * kRS;

  static constexpr int prow(int row) { return kSwz ? (row ^ ((row >> 3) & 1)) : row; }
  static constexpr int slot(int pr, int c) { return c ^ ((pr >> 1) & 3); }

  // float index of (row, col)
  static constexpr int at(int row, int col) {
    return kSwz ? prow(row) * kRS + 4 * slot(prow(row), col >> 2) + (col & 3) : row * kRS + col;
  }
  // float index of 4-float chunk c (columns 4 c .. 4 c + 3) of a row (swizzled layout)
  static constexpr int chunk(int row, int c) { return prow(row) * kRS + 4 * slot(prow(row), c); }
};

}  // namespace redl
