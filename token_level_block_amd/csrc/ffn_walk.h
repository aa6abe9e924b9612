// Tile walk of the FFN GEMM kernel: which 256 x 256 output tile a workgroup
// computes, and how many workgroups a launch takes.  Plain C++ (constexpr
// functions, usable in device code as well), so host tests can check that
// every tile is computed exactly once.
//
// Workgroups are dealt to the 8 XCDs round-robin (XCD x = id mod 8 runs the
// ones with id / 8 = 0, 1, 2, ... in turn).  With 8 or more weight panels the
// XCDs form an xi x (8 / xi) grid: XCD x takes the (x mod xi)-th of xi equal
// runs of weight panels and every (8 / xi)-th group of kFfnGroupJ token panels,
// starting at group x / xi, and walks them group by group.  The 32 workgroups
// an XCD runs together then cover at least 4 weight panels times a group of
// token panels (xi is the largest of 8, 4, 2 that leaves each XCD 4 weight
// panels or more), which they share in its L2; the XCDs of one column walk the
// same token groups at once, so a token panel leaves HBM once and their other
// L2 misses on it hit the MALL.  Otherwise XCD x walks tiles [x T/8, (x+1) T/8)
// in order.  32-bit arithmetic: the host keeps every tile count, and the grid,
// below 2^32.
#pragma once

#include <stdint.h>

namespace up {

constexpr uint32_t kFfnGroupJ = 8;   // token panels walked together

// rows of the XCD grid (8, 4 or 2) for tiles_i >= 8 weight panels
constexpr uint32_t ffn_xcd_rows(uint32_t tiles_i) { return tiles_i >= 32 ? 8u : (tiles_i >= 16 ? 4u : 2u); }

// workgroups a launch takes: 8 times the most tiles any XCD can get (ids past
// an XCD's share find no tile)
constexpr int64_t ffn_gemm_grid(int64_t tiles_i, int64_t tiles_j) {
  if (tiles_i < 8) return (tiles_i * tiles_j + 7) / 8 * 8;
  const int64_t xi = ffn_xcd_rows((uint32_t)(tiles_i < 32 ? tiles_i : 32)), xj = 8 / xi;
  const int64_t groups = (tiles_j + kFfnGroupJ - 1) / kFfnGroupJ;
  return 8 * ((tiles_i + xi - 1) / xi) * kFfnGroupJ * ((groups + xj - 1) / xj);
}

// Tile (weight panel *ti, token panel *tj) of workgroup id = 8 q + x; false
// when that workgroup has none.
constexpr bool ffn_tile_of(uint32_t x, uint32_t q, uint32_t tiles_i, uint32_t tiles_j, int* ti, int* tj) {
  uint32_t wgi = 0, grp = 0, ti0 = 0;
  if (tiles_i >= 8) {
    const uint32_t xi = ffn_xcd_rows(tiles_i), xj = 8 / xi;
    const uint32_t gi = x % xi;
    ti0 = gi * tiles_i / xi;
    const uint32_t nti = (gi + 1) * tiles_i / xi - ti0;
    grp = (q / (nti * kFfnGroupJ)) * xj + x / xi;
    wgi = q % (nti * kFfnGroupJ);
    if (grp * kFfnGroupJ >= tiles_j) return false;
    const uint32_t left = tiles_j - grp * kFfnGroupJ;
    if (wgi >= nti * (left < kFfnGroupJ ? left : kFfnGroupJ)) return false;
  } else {
    const uint32_t ntiles = tiles_i * tiles_j;
    const uint32_t t = x * ((ntiles + 7) / 8) + q;
    if (t >= ntiles) return false;
    grp = t / (kFfnGroupJ * tiles_i);
    wgi = t % (kFfnGroupJ * tiles_i);
  }
  const uint32_t left = tiles_j - grp * kFfnGroupJ;
  const uint32_t gj = left < kFfnGroupJ ? left : kFfnGroupJ;
  *ti = (int)(ti0 + wgi / gj);
  *tj = (int)(grp * kFfnGroupJ + wgi % gj);
  return true;
}

}  // namespace up
