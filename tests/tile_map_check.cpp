// Exhaustive host-side check of the scheduler's tile mapping (moe_grouped_gemm_nt_amd/
// csrc/tile_map.h, the same functions the kernel decodes its tiles with). For seeded
// random layouts it enumerates every logical tile index a launch walks and checks, by
// brute force against the set of outputs the layout defines:
//   - masked / prefix-sum: every (expert, m-tile, output column) with m-tile below
//     ceil(rows_g / BM) and column below N is covered by exactly one tile or piece, no
//     tile starts at or past its expert's rows, and pieces stay inside [0, N];
//   - contiguous: every (valid row block, sub-tile, column) exactly once;
//   - K-grouped: the order is a bijection onto (m-tile, n-tile), and 32 consecutive
//     tiles of a full group cover 8 m-tiles x 4 n-tiles;
//   - the XCD-aware first-tile order is a permutation of the workgroups.
// Prints "ok" and exits 0, or prints the first failing case and exits 1.
#include <cstdio>
#include <cstdlib>
#include <set>
#include <vector>

#include "tile_map.h"

using namespace mgg;

namespace {

unsigned long long rng_state = 0x9E3779B97F4A7C15ULL;
int rnd(int lo, int hi) {  // uniform integer in [lo, hi]
  rng_state = rng_state * 6364136223846793005ULL + 1442695040888963407ULL;
  return lo + (int)((rng_state >> 33) % (unsigned long long)(hi - lo + 1));
}

int fails = 0;
void fail(const char* what, int a, int b, int c, int d) {
  if (fails++ < 5) std::printf("FAIL %s (%d %d %d %d)\n", what, a, b, c, d);
}

struct Shape {
  int bm, bn, wtn;
};
// the tile shapes the library launches: rows x weight rows, columns per MFMA wave
const Shape kShapes[] = {{32, 64, 32}, {32, 128, 32}, {64, 128, 64}, {128, 256, 64},
                         {128, 256, 128}};
const int kGrids[] = {8, 64, 256, 512, 1024};

// masked and prefix-sum layouts share the mapping: per-expert row counts -> tiles
void check_expert_layout(int trial) {
  const Shape sh = kShapes[rnd(0, 4)];
  const int G = rnd(1, 40), N = 8 * rnd(1, 90), grid = kGrids[rnd(0, 4)];
  const int cap = rnd(1, 700);
  std::vector<int> rows(G), prefix(G);
  const int ntn = (N + sh.bn - 1) / sh.bn;
  int tiles = 0;
  for (int g = 0; g < G; ++g) {
    rows[g] = rnd(0, 5) == 0 ? 0 : rnd(0, cap);
    prefix[g] = tiles;
    tiles += (rows[g] + sh.bm - 1) / sh.bm * ntn;
  }
  const SplitRound sr = split_last_round(tiles, grid, sh.bn, sh.wtn);
  if (sr.pieces > 1 && (sr.total - sr.base) > grid) fail("split round exceeds the grid", trial, sr.total, sr.base, grid);
  const int mt_max = (cap + sh.bm - 1) / sh.bm;
  std::vector<unsigned char> hits((size_t)G * mt_max * N, 0);  // times each output is covered
  for (long L = 0; L < sr.total; ++L) {
    const Piece q = piece_of(L, sr.base, sr.pieces);
    const int g = expert_of_tile(q.tile, prefix.data(), G);
    const int mt_g = (rows[g] + sh.bm - 1) / sh.bm;
    if (mt_g == 0 || q.tile < prefix[g] || q.tile >= prefix[g] + mt_g * ntn) {
      fail("tile outside its expert", trial, (int)L, g, mt_g);
      continue;
    }
    int mt, nt, n0, n_end;
    expert_tile((int)(q.tile - prefix[g]), mt_g, &mt, &nt);
    if (mt < 0 || mt * sh.bm >= rows[g] || nt < 0 || nt >= ntn) {
      fail("tile past the expert's rows", trial, g, mt, nt);
      continue;
    }
    piece_columns(nt, sh.bn, q.piece, q.pieces, N, &n0, &n_end);
    if (n_end < n0 || n0 < nt * sh.bn || n_end > (nt + 1) * sh.bn ||
        (n_end > N && n_end != n0) || n_end - n0 > sh.bn / q.pieces)
      fail("piece columns", trial, nt, n0, n_end);
    if (q.pieces > 1 && (sh.bn / q.pieces) % sh.wtn != 0) fail("piece not whole wave columns", trial, sh.bn, q.pieces, sh.wtn);
    for (int n = n0 < 0 ? 0 : n0; n < n_end && n < N; ++n)
      if (hits[((size_t)g * mt_max + mt) * N + n]++) fail("output covered twice", trial, g, mt, n);
  }
  for (int g = 0; g < G; ++g)
    for (int mt = 0; mt < (rows[g] + sh.bm - 1) / sh.bm; ++mt)
      for (int n = 0; n < N; ++n)
        if (!hits[((size_t)g * mt_max + mt) * N + n]) fail("output missed", trial, g, mt, n);
}

// contiguous layout: valid 128-row blocks split into sub-tiles of BM rows; the last round
// is split only for 128-row tiles (no padding sub-tiles)
void check_contiguous(int trial) {
  const Shape sh = kShapes[rnd(0, 4)];
  const int sub_per_block = 128 / sh.bm;
  const int blocks = rnd(1, 700), N = 8 * rnd(1, 90), grid = kGrids[rnd(0, 4)];
  const int ntn = (N + sh.bn - 1) / sh.bn;
  const int tiles = blocks * sub_per_block * ntn;
  const SplitRound sr = sub_per_block == 1 ? split_last_round(tiles, grid, sh.bn, sh.wtn)
                                           : SplitRound{tiles, 1, tiles};
  std::vector<unsigned char> hits((size_t)blocks * sub_per_block * N, 0);
  for (long L = 0; L < sr.total; ++L) {
    const Piece q = piece_of(L, sr.base, sr.pieces);
    int block, sub, nt, n0, n_end;
    contiguous_tile(q.tile, ntn, sub_per_block, &block, &sub, &nt);
    if (block < 0 || block >= blocks || sub < 0 || sub >= sub_per_block || nt < 0 || nt >= ntn) {
      fail("contiguous tile out of range", trial, block, sub, nt);
      continue;
    }
    piece_columns(nt, sh.bn, q.piece, q.pieces, N, &n0, &n_end);
    if (n_end > N && n_end != n0) fail("contiguous piece past N", trial, nt, n0, n_end);
    for (int n = n0 < 0 ? 0 : n0; n < n_end && n < N; ++n)
      if (hits[((size_t)block * sub_per_block + sub) * N + n]++) fail("contiguous output twice", trial, block, sub, n);
  }
  for (size_t i = 0; i < hits.size(); ++i)
    if (!hits[i]) {
      fail("contiguous output missed", trial, (int)(i / N), (int)(i % N), 0);
      break;
    }
}

void check_kgrouped(int trial) {
  const int mtn = rnd(1, 70), ntn = rnd(1, 40), group_m = 8;
  std::set<std::pair<int, int>> seen;
  std::vector<int> mts(mtn * ntn), nts(mtn * ntn);
  for (int local = 0; local < mtn * ntn; ++local) {
    int mt, nt;
    kgrouped_tile(local, mtn, ntn, group_m, &mt, &nt);
    mts[local] = mt;
    nts[local] = nt;
    if (mt < 0 || mt >= mtn || nt < 0 || nt >= ntn || !seen.insert({mt, nt}).second)
      fail("K-grouped order not a bijection", trial, local, mt, nt);
  }
  // 32 consecutive tiles of a full group (8 m-tiles, n-tiles a multiple of 4): 8 x 4
  if (ntn % 4 == 0) {
    for (int g0 = 0; g0 + group_m <= mtn; g0 += group_m)
      for (int r = 0; r < ntn / 4; ++r) {
        std::set<int> ms, ns;
        const int start = g0 * ntn + 32 * r;
        for (int k = 0; k < 32; ++k) {
          ms.insert(mts[start + k]);
          ns.insert(nts[start + k]);
        }
        if (ms.size() != 8 || ns.size() != 4) fail("XCD footprint", trial, g0, r, (int)ms.size());
      }
  }
}

void check_first_tile() {
  for (int grid = 1; grid <= 1024; ++grid) {
    std::vector<char> hit(grid, 0);
    for (int b = 0; b < grid; ++b) {
      const long L = first_tile_of(b, grid, 8);
      if (L < 0 || L >= grid || hit[L]) {
        fail("first tiles not a permutation", grid, b, (int)L, 0);
        break;
      }
      hit[L] = 1;
    }
  }
}

}  // namespace

int main() {
  for (int t = 0; t < 3000; ++t) check_expert_layout(t);
  for (int t = 0; t < 1500; ++t) check_contiguous(t);
  for (int t = 0; t < 500; ++t) check_kgrouped(t);
  check_first_tile();
  if (fails) {
    std::printf("%d failures\n", fails);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
