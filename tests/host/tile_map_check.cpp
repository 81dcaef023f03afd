// Host check of the grouped GEMM's device tile list (tile_map.h): for many
// random expert-count vectors, empty groups included, every workgroup of
// each launch the library makes is decoded on the CPU, and every
// (row, column) of every group's output must be covered exactly once, by a
// tile of that group, over the same launches the library issues (one
// big-tile launch, or its full rounds plus the quarter-tile launch of a
// split last round). Exit status 0 and "OK" on success.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../../ragged_grouped_gemm_router_amd/csrc/tile_map.h"

using namespace moe;

namespace {

constexpr int CW = 32;  // column granularity of the coverage map
long g_checked = 0;

[[noreturn]] void fail(const char* what, int a, int b, int c) {
  std::printf("FAIL %s (%d, %d, %d)\n", what, a, b, c);
  std::exit(1);
}

// tile_off[e] = sum_{e' < e} ceil(count_e' / bm), the prefix the permute
// step publishes for row tiles of height bm
std::vector<int32_t> tile_prefix(const std::vector<int32_t>& counts, int bm) {
  std::vector<int32_t> t(counts.size() + 1, 0);
  for (size_t e = 0; e < counts.size(); ++e)
    t[e + 1] = t[e] + (counts[e] + bm - 1) / bm;
  return t;
}

struct Problem {
  std::vector<int32_t> counts, off;
  int M, N;
};

// Decode every workgroup of one launch and add its tile to the coverage
// map [M rows x N / CW column pieces].
template <int BM, int BN, int TAIL>
void run_launch(const GemmParams& p, const Problem& pr, std::vector<int>& cover) {
  const long grid = launch_grid<BM, BN, kSchedM, TAIL>(p);
  if (grid % kNumXcd) fail("grid not a multiple of the XCD count", (int)grid, 0, 0);
  const int nch = pr.N / CW;
  for (long b = 0; b < grid; ++b) {
    Tile t;
    if (!decode_tile<BM, BN, kSchedM, TAIL>(p, (int)b, (int)grid, t)) continue;
    if (t.n0 % BN || t.n0 < 0 || t.n0 >= pr.N) fail("column tile", t.n0, BN, (int)b);
    if (p.off) {
      if (t.g < 0 || t.g >= p.G) fail("group", t.g, p.G, (int)b);
      if (t.m_end != pr.off[t.g + 1]) fail("group end", t.m_end, t.g, (int)b);
      if (t.m0 < pr.off[t.g] || t.m0 >= t.m_end) fail("row tile outside group", t.m0, t.g, (int)b);
      if ((t.m0 - pr.off[t.g]) % BM) fail("row tile alignment", t.m0, t.g, (int)b);
    } else {
      if (t.m_end != pr.M || t.m0 % BM || t.m0 >= pr.M) fail("dense row tile", t.m0, pr.M, (int)b);
    }
    const int r1 = t.m0 + BM < t.m_end ? t.m0 + BM : t.m_end;
    const int c1 = t.n0 + BN < pr.N ? t.n0 + BN : pr.N;
    for (int r = t.m0; r < r1; ++r)
      for (int c = t.n0 / CW; c < (c1 + CW - 1) / CW; ++c) ++cover[(long)r * nch + c];
  }
}

void expect_once(const std::vector<int>& cover, const char* what, int a) {
  for (size_t i = 0; i < cover.size(); ++i)
    if (cover[i] != 1) fail(what, a, (int)i, cover[i]);
  g_checked += (long)cover.size();
}

// One row-grouped product in every launch form the library uses for its
// tile size: a single launch (TAIL 0), and the big-tile launch followed by
// the quarter-tile launch (TAIL 1 + TAIL 2) for CU counts `slots`.
template <int BM, int BN>
void check_row_grouped(const Problem& pr, int group_n, int slots, bool grouped) {
  GemmParams p{};
  p.M = pr.M;
  p.N = pr.N;
  p.K = 64;
  p.G = grouped ? (int)pr.counts.size() : 1;
  std::vector<int32_t> tb = tile_prefix(pr.counts, BM);
  std::vector<int32_t> tq = tile_prefix(pr.counts, BM / 2);
  if (grouped) {
    p.off = pr.off.data();
    p.tile_off = tb.data();
    p.tiles_m_max = (pr.M + BM - 1) / BM + (p.G < pr.M ? p.G : pr.M);
  } else {
    p.tiles_m_max = (pr.M + BM - 1) / BM;
  }
  const int tiles_n = (pr.N + BN - 1) / BN;
  p.group_n = group_n > 0 ? group_n : tiles_n;
  std::vector<int> cover((long)pr.M * (pr.N / CW), 0);
  run_launch<BM, BN, 0>(p, pr, cover);
  expect_once(cover, "single launch coverage", BM);
  if (!grouped) return;
  std::fill(cover.begin(), cover.end(), 0);
  p.slots = slots;
  run_launch<BM, BN, 1>(p, pr, cover);
  // the quarter launch decodes from the big tile's prefix and grid bound
  run_launch<BM / 2, BN / 2, 2>(p, pr, cover);
  expect_once(cover, "split launches coverage", slots);
  (void)tq;
}

// Contraction-grouped products: each (group, row tile, column tile) of G
// [M, N] outputs once, contracting over that group's own range.
template <int BM, int BN>
void check_k_grouped(int M, int N, const std::vector<int32_t>& off, int kmul) {
  GemmParams p{};
  p.M = M;
  p.N = N;
  p.G = (int)off.size() - 1;
  p.off = off.data();
  p.kmul = kmul;
  const long grid = launch_grid<BM, BN, kSchedK>(p);
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  std::vector<int> seen((long)p.G * tm * tn, 0);
  for (long b = 0; b < grid; ++b) {
    Tile t;
    if (!decode_tile<BM, BN, kSchedK>(p, (int)b, (int)grid, t)) continue;
    if (t.g < 0 || t.g >= p.G || t.m0 % BM || t.n0 % BN || t.m0 >= M || t.n0 >= N)
      fail("k-grouped tile", t.g, t.m0, t.n0);
    if (t.k_beg != off[t.g] * kmul || t.k_end != off[t.g + 1] * kmul)
      fail("k-grouped range", t.g, t.k_beg, t.k_end);
    ++seen[((long)t.g * tm + t.m0 / BM) * tn + t.n0 / BN];
  }
  expect_once(seen, "k-grouped coverage", p.G);
}

// A split contraction (no offsets): G partial products of one [M, N]
// output, split g over [g * kmul, min(K, (g + 1) * kmul)); together the
// splits cover [0, K) once, and every (split, row tile, column tile) is
// decoded once.
template <int BM, int BN>
void check_k_split(int M, int N, int K, int G, int kmul) {
  GemmParams p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.G = G;
  p.kmul = kmul;
  const long grid = launch_grid<BM, BN, kSchedK>(p);
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  std::vector<int> seen((long)G * tm * tn, 0);
  std::vector<int> kcover(K, 0);
  for (long b = 0; b < grid; ++b) {
    Tile t;
    if (!decode_tile<BM, BN, kSchedK>(p, (int)b, (int)grid, t)) continue;
    if (t.g < 0 || t.g >= G || t.m0 % BM || t.n0 % BN || t.m0 >= M || t.n0 >= N)
      fail("split tile", t.g, t.m0, t.n0);
    if (t.k_beg < 0 || t.k_end > K || t.k_beg > t.k_end)
      fail("split range", t.g, t.k_beg, t.k_end);
    if (++seen[((long)t.g * tm + t.m0 / BM) * tn + t.n0 / BN] == 1 &&
        t.m0 == 0 && t.n0 == 0)
      for (int k = t.k_beg; k < t.k_end; ++k) ++kcover[k];
  }
  expect_once(seen, "split coverage", G);
  expect_once(kcover, "split contraction coverage", G);
}

}  // namespace

int main(int argc, char** argv) {
  const int n_cases = argc > 1 ? std::atoi(argv[1]) : 1500;
  std::mt19937 rng(12345);
  auto uni = [&](int lo, int hi) {  // [lo, hi]
    return std::uniform_int_distribution<int>(lo, hi)(rng);
  };
  // xcd_remap_n is a bijection that gives each XCD a contiguous range
  for (int n = 1; n < 3000; n += (n < 64 ? 1 : 37)) {
    std::vector<int> hit(n, 0);
    for (int b = 0; b < n; ++b) {
      const int l = xcd_remap_n(b, n);
      if (l < 0 || l >= n) fail("xcd_remap_n range", n, b, l);
      ++hit[l];
    }
    for (int l = 0; l < n; ++l)
      if (hit[l] != 1) fail("xcd_remap_n bijection", n, l, hit[l]);
  }
  for (int it = 0; it < n_cases; ++it) {
    Problem pr;
    const int E = it % 7 == 0 ? uni(1, 4) : uni(1, 300);
    const int shape = uni(0, 4);
    pr.counts.resize(E);
    for (int e = 0; e < E; ++e) {
      int c;
      switch (shape) {
        case 0: c = uni(0, 40); break;                      // tiny groups
        case 1: c = uni(0, 1) ? 0 : uni(1, 700); break;     // half empty
        case 2: c = 256 * uni(0, 3) + uni(-1, 1); break;    // tile edges
        case 3: c = e == 0 ? uni(2000, 6000) : uni(0, 9); break;  // one big
        default: c = uni(90, 200); break;                   // ~half a tile
      }
      pr.counts[e] = c < 0 ? 0 : c;
    }
    if (it % 11 == 0) std::fill(pr.counts.begin(), pr.counts.end(), 0);
    pr.off.assign(E + 1, 0);
    for (int e = 0; e < E; ++e) pr.off[e + 1] = pr.off[e] + pr.counts[e];
    pr.M = pr.off[E];
    if (pr.M == 0) {
      // nothing to cover, but no workgroup may claim a tile
      GemmParams p{};
      p.M = 0; p.N = 256; p.K = 64; p.G = E; p.off = pr.off.data();
      std::vector<int32_t> tb = tile_prefix(pr.counts, 256);
      p.tile_off = tb.data();
      p.tiles_m_max = E;
      p.group_n = 4;
      p.slots = 256;
      const long grid = launch_grid<256, 128, kSchedM, 1>(p);
      for (long b = 0; b < grid; ++b) {
        Tile t;
        if (decode_tile<256, 128, kSchedM, 1>(p, (int)b, (int)grid, t))
          fail("tile with no rows", (int)b, 0, 0);
      }
      continue;
    }
    pr.N = CW * uni(1, 40);
    const int gsel = uni(0, 3);
    const int group_n = gsel == 0 ? 0 : gsel == 1 ? 4 : uni(1, 9);
    const int slots = uni(0, 1) ? 256 : uni(1, 64);
    check_row_grouped<256, 128>(pr, group_n, slots, true);  // dual GEMM 1
    check_row_grouped<256, 256>(pr, group_n, slots, true);  // GEMM 2, MX
    check_row_grouped<128, 64>(pr, group_n, slots, true);   // small dual
    check_row_grouped<128, 128>(pr, group_n, slots, true);  // small single
    if (it % 5 == 0) check_row_grouped<32, 32>(pr, 0, slots, false);  // router
    // weight gradients: G groups of [M, N] over ragged row ranges (kmul 1)
    // or over 64-padded k-tiles (kmul 64)
    const int Mk = 64 * uni(1, 8) + (uni(0, 1) ? 0 : 32);
    check_k_grouped<256, 256>(Mk, pr.N, pr.off, 1);
    check_k_grouped<128, 128>(Mk, pr.N, tile_prefix(pr.counts, 64), 64);
    // the router GEMM split over its contraction, in the library's tiles
    // (k-tiles of 64 shared out evenly; some splits may be empty)
    const int Mr = uni(1, 3000), Nr = uni(1, 300), Kr = 64 * uni(1, 120);
    const int G = uni(1, 8), kmul = 64 * ((Kr / 64 + G - 1) / G);
    check_k_split<32, 32>(Mr, Nr, Kr, G, kmul);
    check_k_split<64, 64>(Mr, Nr, Kr, G, kmul);
    check_k_split<64, 256>(Mr, Nr, Kr, G, kmul);
  }
  std::printf("OK %d cases, %ld cells checked\n", n_cases, g_checked);
  return 0;
}
