// Output-tile decode of the ragged grouped GEMM: which (group, rows,
// columns, contraction range) a workgroup computes. Pure integer logic,
// callable on the host too, so that a host program can enumerate every
// workgroup of a launch and check the tile list against its definition.
#pragma once

#include "common.h"

namespace moe {

struct Tile {
  int g, m0, m_end, n0, k_beg, k_end;
};

// Decode workgroup `block` of a grid of `grid` workgroups. Returns false
// for surplus workgroups (beyond the device-side tile count).
//
// Row-grouped products (kSchedM): the grid is sized by an upper bound, and
// the real row tiles (mt, from the device tile prefix) are enumerated
// densely in n-group-major order (GN column tiles, every row tile of every
// group, then the GN column tiles within), so that consecutive tiles share
// weight and row panels. The first mt * tiles_n workgroups take them, each
// XCD a contiguous share of equal size; the rest exit.
//
// Split last round (TAIL, row-grouped only). With S = p.slots big tiles
// running at once, n_tiles big tiles take full rounds plus a last round of
// r = n_tiles mod S tiles. When 0 < 4 r <= S and there is a full round,
// the big-tile launch (TAIL 1) runs only the full rounds, and a second
// launch of half-size tiles (TAIL 2: BM x BN = half the big tile each
// way) runs the last round's tiles as four quarters each, so that round
// spreads over 4 r CUs instead of r. Both launches decide from the same
// device tile prefix; otherwise TAIL 1 runs every tile and TAIL 2 nothing.
//
// Contraction-grouped products (kSchedK): every (group, row tile, column
// tile) of G fixed-size [M, N] outputs; group g contracts over
// [off[g] * kmul, off[g + 1] * kmul), or, with no offsets (a split of one
// contraction into G partial products), over [g * kmul, min(K, (g + 1) *
// kmul)), empty past K.
template <int BM, int BN, int SCHED, int TAIL = 0>
__host__ __device__ inline bool decode_tile(const GemmParams& p, int block,
                                            int grid, Tile& t) {
  // tile size of the enumeration: the big tile in the quarter launch
  constexpr int DM = TAIL == 2 ? 2 * BM : BM, DN = TAIL == 2 ? 2 * BN : BN;
  const int tiles_n = (p.N + DN - 1) / DN;
  t.g = 0;
  t.k_beg = 0;
  t.k_end = p.K;
  if (SCHED == kSchedM) {
    const int mt = p.off ? p.tile_off[p.G] : (p.M + DM - 1) / DM;
    const int n_tiles = mt * tiles_n;
    // this launch's logical tiles: [lo, lo + n) (quarters: 4 per tile)
    int lo = 0, n = n_tiles;
    if (TAIL != 0) {
      const int full = n_tiles / p.slots * p.slots, r = n_tiles - full;
      const bool split = full > 0 && r > 0 && 4 * r <= p.slots;
      if (TAIL == 1 && split) n = full;
      if (TAIL == 2) {
        if (!split) return false;
        lo = full;
        n = 4 * r;
      }
    }
    if (block >= n) return false;
    const int li = xcd_remap_n(block, n);
    const int idx = lo + (TAIL == 2 ? li / 4 : li), q = li % 4;
    const int GN = p.group_n;
    const int ng = idx / (mt * GN), within = idx % (mt * GN);
    const int rest = tiles_n - ng * GN;
    const int gsz = GN < rest ? GN : rest;
    const int m = within / gsz;
    t.n0 = (ng * GN + within % gsz) * DN;
    if (p.off == nullptr) {
      t.m0 = m * DM;
      t.m_end = p.M;
    } else {
      t.g = upper_group(p.tile_off, p.G, m);
      t.m0 = p.off[t.g] + (m - p.tile_off[t.g]) * DM;
      t.m_end = p.off[t.g + 1];
    }
    if (TAIL == 2) {  // quarter q of the big tile; none past its rows
      t.m0 += (q / 2) * BM;
      t.n0 += (q % 2) * BN;
      if (t.m0 >= t.m_end || t.n0 >= p.N) return false;
    }
    return true;
  }
  const int L = xcd_remap(block, grid);
  const int tiles_m = (p.M + BM - 1) / BM;
  if (L >= p.G * tiles_m * tiles_n) return false;
  t.g = L / (tiles_m * tiles_n);
  const int rem = L % (tiles_m * tiles_n);
  t.m0 = (rem / tiles_n) * BM;
  t.n0 = (rem % tiles_n) * BN;
  t.m_end = p.M;
  const int km = p.kmul > 0 ? p.kmul : 1;
  if (p.off) {
    t.k_beg = p.off[t.g] * km;
    t.k_end = p.off[t.g + 1] * km;
  } else {
    t.k_beg = t.g * km < p.K ? t.g * km : p.K;
    t.k_end = t.k_beg + km < p.K ? t.k_beg + km : p.K;
  }
  return true;
}

// Grid of a launch, in workgroups, as the launchers size it: for kSchedM
// an upper bound (tiles_m_max row tiles of every column group; the quarter
// launch at most p.slots tiles), rounded up to a multiple of the XCD count.
template <int BM, int BN, int SCHED, int TAIL = 0>
__host__ __device__ inline long launch_grid(const GemmParams& p) {
  const long tiles_n = (p.N + BN - 1) / BN;
  long tiles = SCHED == kSchedK
                   ? (long)p.G * ((p.M + BM - 1) / BM) * tiles_n
                   : (tiles_n + p.group_n - 1) / p.group_n * p.tiles_m_max *
                         p.group_n;
  if (TAIL == 2) tiles = p.slots;  // at most 4 r <= slots quarter tiles
  if (tiles <= 0) return 0;
  return (tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
}

}  // namespace moe
