// grid_order.hpp -- workgroup order of the chunked scans (plain C++, usable
// on the host: a CPU test checks it exhaustively).
//
// A launch over nk chunks x ng channel groups runs one workgroup per (chunk,
// group).  With nk a multiple of 8 its grid is (8 ng, nk / 8): workgroup ids,
// taken x fastest, go round-robin over the 8 XCDs, and chunk c's groups all
// land on XCD c % 8, one after another, so the chunk's rows (b, c: shared by
// every channel) reach that XCD's L2 once.  Otherwise the grid is (nk, ng).
// Both keep each grid dimension's work-item count within 32 bits.
#pragma once

#include <stdint.h>

namespace ssm {

// Grid dimensions (x, y) of the launch.
constexpr void chunk_group_dims(int64_t nk, int64_t ng, uint32_t* gx, uint32_t* gy) {
  *gx = static_cast<uint32_t>(nk % 8 == 0 ? 8 * ng : nk);
  *gy = static_cast<uint32_t>(nk % 8 == 0 ? nk / 8 : ng);
}

// (chunk, group) of workgroup (bx, by) in a grid whose x dimension is gx.
constexpr void chunk_group_of(uint32_t bx, uint32_t by, uint32_t gx, uint32_t* c, uint32_t* g) {
  if (gx % 8 == 0) {
    *c = 8 * by + bx % 8;
    *g = bx / 8;
  } else {
    *c = bx;
    *g = by;
  }
}

}  // namespace ssm
