// Exhaustive host check of the direct-to-LDS GEMM tile layouts
// (adjoint_gradients_amd/csrc/gemm_dl_index.hpp): simulates the 16 DMA load
// instructions of a tile, then every MFMA operand fetch of every lane, and
// compares with the values the v_mfma_f32_32x32x16_bf16 operand layout
// requires (lane l: row l % 32, k = 8 (l / 32) .. + 7 of its 32-row block).
// The transposed LDS read is modelled as measured on gfx950: in each 16-lane
// group, lane j receives element j % 4 of the 8-byte pieces addressed by
// lanes j / 4 + 4 r (r = 0..3) of the group.  Also checks that the loads
// write every LDS byte exactly once and that the operand fetches served in
// one LDS pass touch distinct banks (64 banks of 4 bytes; 16-byte reads are
// served 16 lanes per pass, 8-byte reads 32 lanes per pass, as the bank
// conflict counters on gfx950 show).
#include <cstdio>
#include <cstring>
#include <set>
#include <vector>

#include "gemm_dl_index.hpp"
#include "grid_order.hpp"

using namespace gdl;

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { if (fails < 20) { printf(__VA_ARGS__); printf("\n"); } fails++; } } while (0)

int main() {
  // global operands: value = unique id of (row, k)
  auto kc_val = [](int r, int k) { return (uint16_t)(r * 32 + k); };  // X[r][k]
  auto ko_val = [](int k, int r) { return (uint16_t)(k * 256 + r); }; // X[k][r]
  for (int kind = 0; kind < 2; kind++) {
    std::vector<uint16_t> lds(kTileBytes / 2, 0xFFFF);
    std::vector<int> writes(kTileBytes / 2, 0);
    for (int gi = 0; gi < kInstrPerTile; gi++)
      for (int i = 0; i < 64; i++)
        for (int e = 0; e < 8; e++) {
          const int dst = gi * 512 + i * 8 + e;  // in bf16 elements
          uint16_t v;
          if (kind == 0) v = kc_val(kc_load_row(gi, i), 8 * kc_load_chunk(gi, i) + e);
          else v = ko_val(ko_load_krow(gi, i), 8 * ko_load_chunk(gi, i) + e);
          lds[dst] = v;
          writes[dst]++;
        }
    for (size_t j = 0; j < writes.size(); j++) CHECK(writes[j] == 1, "kind %d: LDS element %zu written %d times", kind, j, writes[j]);
    for (int rb = 0; rb < 256; rb += 32)
      for (int q = 0; q < 2; q++) {
        if (kind == 0) {
          for (int quarter = 0; quarter < 4; quarter++) {
            std::set<int> units;
            for (int l = 16 * quarter; l < 16 * quarter + 16; l++) {
              const int off = kc_read_off(l, rb, q);
              CHECK(off % 16 == 0 && off >= 0 && off + 16 <= kTileBytes, "kc offset %d", off);
              units.insert((off / 16) % 16);
              for (int e = 0; e < 8; e++)
                CHECK(lds[off / 2 + e] == kc_val(rb + (l & 31), 16 * q + 8 * (l >> 5) + e),
                      "kc rb %d q %d lane %d e %d: got %d", rb, q, l, e, lds[off / 2 + e]);
            }
            CHECK(units.size() == 16, "kc rb %d q %d quarter %d: bank conflict (%zu units)", rb, q, quarter, units.size());
          }
        } else {
          for (int h = 0; h < 2; h++) {
            int off[64];
            for (int l = 0; l < 64; l++) {
              off[l] = ko_read_off(l, rb, q, h);
              CHECK(off[l] % 8 == 0 && off[l] >= 0 && off[l] + 8 <= kTileBytes, "ko offset %d", off[l]);
            }
            for (int half = 0; half < 2; half++) {
              std::set<int> banks;
              for (int s = 0; s < 32; s++) {
                banks.insert((off[32 * half + s] / 4) % 64);
                banks.insert((off[32 * half + s] / 4 + 1) % 64);
              }
              CHECK(banks.size() == 64, "ko rb %d q %d h %d half %d: bank conflict (%zu banks)", rb, q, h, half, banks.size());
            }
            for (int g = 0; g < 4; g++) {
              for (int j = 0; j < 16; j++) {
                const int l = 16 * g + j;
                for (int r = 0; r < 4; r++) {
                  const int src = 16 * g + j / 4 + 4 * r;
                  const uint16_t got = lds[off[src] / 2 + j % 4];
                  const uint16_t want = ko_val(16 * q + 8 * (l >> 5) + 4 * h + r, rb + (l & 31));
                  CHECK(got == want, "ko rb %d q %d h %d lane %d r %d: got %d want %d", rb, q, h, l, r, got, want);
                }
              }
            }
          }
        }
      }
  }
  // offsets the kernel derives instead of recomputing: K-contiguous fetches
  // move by 2048 bytes per 32-row block; K-outer fetches (one base per block)
  // by 8192 per k sub-step and 2048 for the second transposed half
  for (int l = 0; l < 64; l++)
    for (int rb = 0; rb <= 128; rb += 128)
      for (int i = 0; i < 4; i++)
        for (int q = 0; q < 2; q++) {
          CHECK(kc_read_off(l, rb + 32 * i, q) == kc_read_off(l, rb, q) + 2048 * i, "kc linear l %d rb %d i %d q %d", l, rb, i, q);
          for (int h = 0; h < 2; h++)
            CHECK(ko_read_off(l, rb + 32 * i, q, h) == ko_read_off(l, rb + 32 * i, 0, 0) + 8192 * q + 2048 * h,
                  "ko linear l %d rb %d i %d q %d h %d", l, rb, i, q, h);
        }
  // workgroup order of the chunked scans: a bijection of the grid onto
  // (chunk, group); with nk a multiple of 8 the ids that the 8 XCDs take
  // round-robin (x fastest) put all of a chunk's groups on XCD chunk % 8,
  // consecutively; each grid dimension's work items fit 32 bits at the
  // largest sizes (2^31 tokens in chunks of 1, 2^20 channels)
  for (int64_t nk = 1; nk <= 70; nk++)
    for (int64_t ng = 1; ng <= 20; ng++) {
      uint32_t gx = 0, gy = 0;
      ssm::chunk_group_dims(nk, ng, &gx, &gy);
      CHECK((int64_t)gx * gy == nk * ng, "order nk %ld ng %ld: grid %u x %u", (long)nk, (long)ng, gx, gy);
      std::vector<int> seen(nk * ng, 0);
      std::vector<int> last_loc(nk, -1);
      for (uint32_t by = 0; by < gy; by++)
        for (uint32_t bx = 0; bx < gx; bx++) {
          uint32_t c = 0, g = 0;
          ssm::chunk_group_of(bx, by, gx, &c, &g);
          CHECK(c < nk && g < ng, "order nk %ld ng %ld: (%u, %u) -> (%u, %u)", (long)nk, (long)ng, bx, by, c, g);
          if (c >= nk || g >= ng) continue;
          seen[c * ng + g]++;
          if (nk % 8 == 0) {
            const int64_t id = (int64_t)by * gx + bx;
            CHECK(id % 8 == c % 8, "order nk %ld ng %ld: chunk %u on XCD %ld", (long)nk, (long)ng, c, (long)(id % 8));
            const int loc = (int)(id / 8);
            CHECK(last_loc[c] < 0 || loc == last_loc[c] + 1, "order nk %ld ng %ld: chunk %u not consecutive", (long)nk,
                  (long)ng, c);
            last_loc[c] = loc;
          }
        }
      for (int64_t v = 0; v < nk * ng; v++)
        CHECK(seen[v] == 1, "order nk %ld ng %ld: pair %ld taken %d times", (long)nk, (long)ng, (long)v, seen[v]);
    }
  {
    const int64_t T = int64_t(1) << 31, P = int64_t(1) << 20;
    for (int64_t C : {1, 2, 7, 8, 256}) {
      const int64_t nk = (T + C - 1) / C, ng = (P / 32 + 3) / 4;  // 4 wavefronts of >= 32 channels
      uint32_t gx = 0, gy = 0;
      ssm::chunk_group_dims(nk, ng, &gx, &gy);
      CHECK((int64_t)gx * 256 < (int64_t(1) << 32) || nk % 8 != 0, "order: x work items overflow at C %ld", (long)C);
      CHECK((int64_t)gy * 1 < (int64_t(1) << 32), "order: y overflow at C %ld", (long)C);
    }
  }
  printf(fails ? "FAILED (%d)\n" : "layout OK\n", fails);
  return fails ? 1 : 0;
}
