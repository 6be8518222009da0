// Host-side checks of the LDS tile layouts in fa_layout.h (built with g++ by
// test_layout.py; no GPU).  For D = 64 and 128 it checks that
//  * the row-group layout is a bijection of (row, piece) onto the tile's
//    16-byte slots, that rg_slot inverts it, and that the slot and row steps
//    the direct copies and the reads rely on hold;
//  * the row reads and the transpose reads address what the kernels use,
//    each 16-lane transpose group reads one aligned 128-byte block, and a
//    simulated ds_read_b64_tr_b16 hands every lane the B-operand elements of
//    the matrix-core layout, in the contraction order of the accumulator
//    (C) layout;
//  * the P^T / dS^T tile layout is a bijection, its XOR steps hold, and the
//    chunks a producer writes reach the consumer as an A operand in the same
//    contraction order as the transpose-read B operand;
//  * the epilogues' staging layout covers its 32 rows exactly once and
//    hands every reader its piece's halves in order;
//  * every one of those accesses is free of bank conflicts when the LDS
//    serves 16-byte accesses 8 lanes (8-byte accesses 16 lanes) per cycle
//    over 32 banks, and 16 (32) lanes over 64 banks.
#define __device__
#define __forceinline__ inline
#include "fa_layout.h"

#include <cstdio>
#include <map>
#include <set>
#include <vector>

using namespace fa;

static int fails = 0;
#define CHECK(cond, ...)                                           \
  do {                                                             \
    if (!(cond)) {                                                 \
      if (fails < 20) {                                            \
        std::printf("FAIL line %d: ", __LINE__);                   \
        std::printf(__VA_ARGS__);                                  \
        std::printf("\n");                                         \
      }                                                            \
      ++fails;                                                     \
    }                                                              \
  } while (0)

// Worst number of distinct 4-byte words that one bank must serve for the
// lanes [g0, g0 + n) of an access of `bytes` bytes per lane (lanes reading
// the same word share it).
static int degree(const std::vector<int>& addr, int g0, int n, int bytes, int banks) {
  std::map<int, std::set<int>> words;
  for (int l = g0; l < g0 + n; ++l)
    for (int b = 0; b < bytes; b += 4) {
      const int wd = (addr[l] + b) / 4;
      words[wd % banks].insert(wd);
    }
  size_t worst = 0;
  for (auto& kv : words) worst = kv.second.size() > worst ? kv.second.size() : worst;
  return (int)worst;
}

// conflict free under both bank models for a wave64 access
static bool conflict_free(const std::vector<int>& addr, int bytes) {
  const int per32 = 128 / bytes, per64 = 256 / bytes;  // lanes per cycle
  for (int g0 = 0; g0 < 64; g0 += per32)
    if (degree(addr, g0, per32, bytes, 32) != 1) return false;
  for (int g0 = 0; g0 < 64; g0 += per64)
    if (degree(addr, g0, per64, bytes, 64) != 1) return false;
  return true;
}

template <int D>
static void check_row_groups() {
  constexpr int NP = D / 8;  // 16-byte pieces per row
  constexpr int ROWB = 2 * D;
  for (int R : {32, 64, 128}) {
    std::vector<int> seen(R * NP, 0);
    for (int row = 0; row < R; ++row)
      for (int piece = 0; piece < NP; ++piece) {
        const int off = rg_off<D>(row, piece);
        CHECK(off % 16 == 0 && off >= 0 && off < R * ROWB, "D=%d rg_off(%d,%d)=%d outside the tile", D, row, piece,
              off);
        if (off % 16 || off < 0 || off >= R * ROWB) continue;
        ++seen[off / 16];
        int r2, p2;
        rg_slot<D>(off / 16, r2, p2);
        CHECK(r2 == row && p2 == piece, "D=%d rg_slot does not invert rg_off at (%d,%d)", D, row, piece);
      }
    for (int s = 0; s < R * NP; ++s) CHECK(seen[s] == 1, "D=%d R=%d slot %d used %d times", D, R, s, seen[s]);
  }
  // slot s + r D / 8 is slot s, r rows down, for r a multiple of 16
  for (int s = 0; s < 16 * NP; ++s)
    for (int r = 16; r < 128; r += 16) {
      int r0, p0, r1, p1;
      rg_slot<D>(s, r0, p0);
      rg_slot<D>(s + r * NP, r1, p1);
      CHECK(r1 == r0 + r && p1 == p0, "D=%d slot step: slot %d + %d rows", D, s, r);
    }
  // row reads: piece 2 kk + l / 32 of row 32 t + l % 32
  for (int t = 0; t < 2; ++t)
    for (int kk = 0; kk < D / 16; ++kk) {
      std::vector<int> addr(64);
      for (int l = 0; l < 64; ++l) {
        addr[l] = rg_row_base<D>(l, kk & 1) + 256 * (kk >> 1) + 32 * ROWB * t;
        CHECK(addr[l] == rg_off<D>(32 * t + (l & 31), 2 * kk + (l >> 5)), "D=%d row read kk=%d lane %d", D, kk, l);
      }
      CHECK(conflict_free(addr, 16), "D=%d row reads kk=%d conflict", D, kk);
    }
  // transpose reads: tile element (row, col) holds the value row * D + col
  constexpr int R = 64;
  std::vector<int> tile(R * ROWB / 2, -1);
  for (int row = 0; row < R; ++row)
    for (int col = 0; col < D; ++col) tile[(rg_off<D>(row, col / 8) + 2 * (col % 8)) / 2] = row * D + col;
  for (int t = 0; t < R / 16; ++t)
    for (int db = 0; db < D / 32; ++db) {
      int got[64][8];
      for (int r = 0; r < 2; ++r) {
        std::vector<int> addr(64);
        for (int l = 0; l < 64; ++l) addr[l] = rg_tr_base<D>(l, r) + 256 * db + 16 * t * ROWB;
        CHECK(conflict_free(addr, 8), "D=%d transpose reads t=%d db=%d r=%d conflict", D, t, db, r);
        for (int g = 0; g < 4; ++g) {
          int lo = addr[16 * g];
          for (int i = 0; i < 16; ++i) lo = addr[16 * g + i] < lo ? addr[16 * g + i] : lo;
          std::set<int> chunks;
          for (int i = 0; i < 16; ++i) chunks.insert(addr[16 * g + i] - lo);
          CHECK(lo % 128 == 0 && chunks.size() == 16 && *chunks.rbegin() == 120,
                "D=%d transpose group %d is not one 128-byte block", D, g);
          // lane i of the group: element i % 4 of the chunks of lanes i / 4 + 4 m
          for (int i = 0; i < 16; ++i)
            for (int m = 0; m < 4; ++m) got[16 * g + i][4 * r + m] = tile[(addr[16 * g + i / 4 + 4 * m] + 2 * (i % 4)) / 2];
        }
      }
      for (int l = 0; l < 64; ++l)
        for (int e = 0; e < 8; ++e) {
          // B operand: column 32 db + l % 32; contraction index e stands for
          // row 8 (e / 4) + 4 (l / 32) + e % 4 of the 16-row step, the row an
          // accumulator element e of lane l holds in the C layout
          const int row = 16 * t + 8 * (e / 4) + 4 * (l >> 5) + (e % 4);
          CHECK(got[l][e] == row * D + 32 * db + (l & 31), "D=%d transpose read lane %d e=%d", D, l, e);
        }
    }
}

static void check_pt() {
  // bijection of (key row, query) onto the 8 KiB tile, 2 bytes each
  std::vector<int> seen(4096, 0);
  for (int row = 0; row < 128; ++row)
    for (int q = 0; q < 32; ++q) {
      const int off = pt_off(row, q);
      CHECK(off % 2 == 0 && off >= 0 && off < 8192, "pt_off(%d,%d)=%d outside", row, q, off);
      if (off % 2 || off < 0 || off >= 8192) continue;
      ++seen[off / 2];
      if (q % 4) CHECK(off == pt_off(row, q & ~3) + 2 * (q & 3), "pt_off chunk not contiguous");
    }
  for (int s = 0; s < 4096; ++s) CHECK(seen[s] == 1, "P^T element slot %d used %d times", s, seen[s]);
  // producer writes: key group kg, lane l = key 32 kg + l % 32, half h = l / 32;
  // accumulator elements e = 4 g4 .. 4 g4 + 3 are queries 8 g4 + 4 h + (0..3)
  // (C layout), written as one chunk at pt_off(key, 4 h) ^ 16 g4
  std::vector<int> tile(4096, -1);
  for (int kg = 0; kg < 4; ++kg)
    for (int g4 = 0; g4 < 4; ++g4) {
      std::vector<int> addr(64);
      for (int l = 0; l < 64; ++l) {
        const int key = 32 * kg + (l & 31), h = l >> 5;
        addr[l] = pt_off(key, 4 * h) ^ (16 * g4);
        CHECK(addr[l] == pt_off(key, 8 * g4 + 4 * h), "producer chunk step g4=%d", g4);
        for (int i = 0; i < 4; ++i) tile[(addr[l] + 2 * i) / 2] = key * 32 + 8 * g4 + 4 * h + i;
      }
      CHECK(conflict_free(addr, 8), "producer writes kg=%d g4=%d conflict", kg, g4);
    }
  // consumer reads: lane l = key row 32 (2 kh + g) + l % 32, half h; for the
  // 16 queries of step tq the chunks at pt_off(key, 4 h) ^ 32 tq and ^ 32 tq + 16
  // are A-operand elements 0-3 and 4-7, which must be the queries the
  // transpose-read B operand pairs them with: 16 tq + 8 (e / 4) + 4 h + e % 4
  for (int kg = 0; kg < 4; ++kg)
    for (int tq = 0; tq < 2; ++tq)
      for (int half = 0; half < 2; ++half) {
        std::vector<int> addr(64);
        for (int l = 0; l < 64; ++l) {
          const int key = 32 * kg + (l & 31), h = l >> 5;
          addr[l] = pt_off(key, 4 * h) ^ (32 * tq + 16 * half);
          for (int i = 0; i < 4; ++i) {
            const int e = 4 * half + i;
            const int q = 16 * tq + 8 * (e / 4) + 4 * h + e % 4;
            CHECK(tile[(addr[l] + 2 * i) / 2] == key * 32 + q, "consumer read key %d tq=%d e=%d", key, tq, e);
          }
        }
        CHECK(conflict_free(addr, 8), "consumer reads kg=%d tq=%d conflict", kg, tq);
      }
}

// Epilogue staging of 32 rows of D bf16: the 8-byte halves the lanes write
// and the 16-byte pieces read back cover each row exactly once, the read
// hands the halves back in order once stage_swap undoes the swap, and both
// access kinds are conflict free.
template <int D>
static void check_stage() {
  constexpr int NCH = D / 8, ROWB = 2 * D, RPI = 64 / NCH;
  std::vector<int> seen(32 * ROWB / 8, 0);
  for (int r = 0; r < 32; ++r)
    for (int p = 0; p < NCH; ++p)
      for (int h = 0; h < 2; ++h) {
        const int off = stage_off<D>(r, p, h);
        CHECK(off % 8 == 0 && off >= r * ROWB && off < (r + 1) * ROWB, "D=%d stage_off(%d,%d,%d)=%d outside its row", D,
              r, p, h, off);
        if (off % 8 || off < 0 || off >= 32 * ROWB) continue;
        ++seen[off / 8];
      }
  for (size_t w = 0; w < seen.size(); ++w) CHECK(seen[w] == 1, "D=%d staging word %zu used %d times", D, w, seen[w]);
  // writes: lane l, row l % 32, half l / 32 of piece 4 db + g4
  for (int db = 0; db < D / 32; ++db)
    for (int g4 = 0; g4 < 4; ++g4) {
      std::vector<int> addr(64);
      for (int l = 0; l < 64; ++l) addr[l] = stage_off<D>(l & 31, 4 * db + g4, l >> 5);
      CHECK(conflict_free(addr, 8), "D=%d staging writes db=%d g4=%d conflict", D, db, g4);
    }
  // reads: lane l, piece l % NCH of row RPI i + l / NCH, as one aligned
  // 16-byte access whose halves come back in order after the swap
  for (int i = 0; i < 32 / RPI; ++i) {
    std::vector<int> addr(64);
    for (int l = 0; l < 64; ++l) {
      const int r = RPI * i + l / NCH, pc = l % NCH;
      addr[l] = stage_off<D>(r, pc, 0) & ~15;
      const int first = stage_swap<D>(r) ? 1 : 0;  // the half at the lower address
      CHECK(stage_off<D>(r, pc, first) == addr[l] && stage_off<D>(r, pc, 1 - first) == addr[l] + 8,
            "D=%d staging read row %d piece %d", D, r, pc);
    }
    CHECK(conflict_free(addr, 16), "D=%d staging reads i=%d conflict", D, i);
  }
}

int main() {
  check_row_groups<64>();
  check_row_groups<128>();
  check_pt();
  check_stage<64>();
  check_stage<128>();
  if (fails) {
    std::printf("%d layout checks failed\n", fails);
    return 1;
  }
  std::printf("all layout checks passed\n");
  return 0;
}
