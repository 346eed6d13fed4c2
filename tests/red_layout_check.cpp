// Exhaustive host check of the transpose buffer placement of the reverse walk
// (adjoint_gradients_amd/csrc/red_layout.hpp), for every lane layout the
// kernels instantiate: the placement is a bijection onto the buffer; every
// lane's reads return exactly the logical row segment it sums; and, for the
// unpadded layout, each write instruction (64 lanes, 4 bytes each), each
// merged write of rows 2i and 2i + 1 (32 lanes, 8 bytes each) and each
// 16-byte read pass (16 lanes) touches distinct banks (64 banks of 4 bytes).
#include <cstdio>
#include <set>
#include <vector>

#include "red_layout.hpp"

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { if (fails < 20) { printf(__VA_ARGS__); printf("\n"); } fails++; } } while (0)

template <int NL, int G>
void check() {
  using L = redl::Layout<NL, G>;
  constexpr int CH = L::CH, NN = L::NN, OUT = L::OUT;
  std::vector<int> owner(L::kFloats, -1);
  for (int row = 0; row < OUT; row++)
    for (int col = 0; col < CH; col++) {
      const int i = L::at(row, col);
      CHECK(i >= 0 && i < L::kFloats, "NL %d G %d: (%d,%d) -> %d out of range", NL, G, row, col, i);
      if (i < 0 || i >= L::kFloats) continue;
      CHECK(owner[i] < 0, "NL %d G %d: (%d,%d) collides", NL, G, row, col);
      owner[i] = row * CH + col;
    }
  // merged writes of rows 2i and 2i + 1 (ds_write2_b32): 32 lanes of one group per pass
  if (L::kSwz)
    for (int part = 0; part < 2; part++)
      for (int grp = 0; grp < G; grp++)
        for (int j = 0; j + 1 < NL; j += 2) {
          std::set<int> banks;
          for (int pl = 0; pl < CH; pl++) {
            banks.insert(L::at(part * NN + grp * NL + j, pl) % 64);
            banks.insert(L::at(part * NN + grp * NL + j + 1, pl) % 64);
          }
          CHECK(banks.size() == 64, "NL %d G %d: merged write part %d grp %d rows %d,%d conflict (%zu banks)", NL, G,
                part, grp, j, j + 1, banks.size());
        }
  // writes: instruction (part, j), lane (grp, pl)
  for (int part = 0; part < 2; part++)
    for (int j = 0; j < NL; j++) {
      std::set<int> banks;
      for (int lane = 0; lane < 64; lane++) {
        const int grp = lane / CH, pl = lane % CH;
        banks.insert(L::at(part * NN + grp * NL + j, pl) % 64);
      }
      if (L::kSwz) CHECK(banks.size() == 64, "NL %d G %d: write part %d j %d conflicts (%zu banks)", NL, G, part, j, banks.size());
    }
  if constexpr (L::kSwz) {
    constexpr int LPO = 64 / OUT, V = CH / LPO;
    static_assert(V == 16, "four 16-byte reads per lane");
    for (int q = 0; q < 4; q++) {
      for (int pass = 0; pass < 4; pass++) {
        std::set<int> quads;
        for (int lane = 16 * pass; lane < 16 * pass + 16; lane++) {
          const int o = lane / LPO, r = lane % LPO;
          const int base = L::chunk(o, 4 * r + q);
          CHECK(base % 4 == 0, "unaligned chunk");
          quads.insert((base / 4) % 16);
          for (int e = 0; e < 4; e++)
            CHECK(owner[base + e] == o * CH + V * r + 4 * q + e, "lane %d q %d e %d reads the wrong element", lane, q, e);
        }
        CHECK(quads.size() == 16, "read q %d pass %d conflicts (%zu quads)", q, pass, quads.size());
      }
    }
  }
}

int main() {
  check<1, 1>(); check<2, 1>(); check<4, 1>(); check<8, 1>();
  check<8, 2>(); check<8, 4>(); check<8, 8>();
  if (fails) { printf("%d failures\n", fails); return 1; }
  printf("layout OK\n");
  return 0;
}
