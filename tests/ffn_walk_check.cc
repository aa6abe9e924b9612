// Host-side checks of the FFN GEMM's tile walk (ffn_walk.h): over many panel
// counts, the workgroups of ffn_gemm_grid compute every tile exactly once and
// no tile out of range; with 8 or more weight panels, the first workgroups
// an XCD runs together cover at least 4 weight panels (or all of its share)
// and one group of token panels.  Built with g++ by tests/test_abi.py;
// prints "ok N" after N checked workgroups.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "../token_level_block_amd/csrc/ffn_walk.h"

static int failures = 0;
static long long checked = 0;

static void check_walk(uint32_t tiles_i, uint32_t tiles_j) {
  const int64_t grid = up::ffn_gemm_grid(tiles_i, tiles_j);
  if (grid % 8 != 0) {
    std::fprintf(stderr, "FAIL grid %lld not a multiple of 8 (%u x %u)\n", (long long)grid, tiles_i, tiles_j);
    ++failures;
    return;
  }
  std::vector<int> seen((size_t)tiles_i * tiles_j, 0);
  for (int64_t id = 0; id < grid; ++id) {
    int ti = -1, tj = -1;
    ++checked;
    if (!up::ffn_tile_of((uint32_t)(id & 7), (uint32_t)(id >> 3), tiles_i, tiles_j, &ti, &tj)) continue;
    if (ti < 0 || tj < 0 || (uint32_t)ti >= tiles_i || (uint32_t)tj >= tiles_j) {
      std::fprintf(stderr, "FAIL %u x %u: workgroup %lld got tile (%d, %d)\n", tiles_i, tiles_j, (long long)id, ti, tj);
      ++failures;
      return;
    }
    ++seen[(size_t)ti * tiles_j + tj];
  }
  for (uint32_t i = 0; i < tiles_i; ++i)
    for (uint32_t j = 0; j < tiles_j; ++j)
      if (seen[(size_t)i * tiles_j + j] != 1) {
        std::fprintf(stderr, "FAIL %u x %u: tile (%u, %u) computed %d times\n", tiles_i, tiles_j, i, j,
                     seen[(size_t)i * tiles_j + j]);
        ++failures;
        return;
      }
  // sharing: the first min(32, its tiles) workgroups of each XCD
  if (tiles_i >= 8 && tiles_j >= up::kFfnGroupJ)
    for (uint32_t x = 0; x < 8; ++x) {
      std::vector<int> wi(tiles_i, 0), wj(tiles_j, 0);
      int n = 0;
      for (uint32_t q = 0; q < 32; ++q) {
        int ti = -1, tj = -1;
        if (!up::ffn_tile_of(x, q, tiles_i, tiles_j, &ti, &tj)) break;
        wi[ti] = 1;
        wj[tj] = 1;
        ++n;
      }
      int ni = 0, nj = 0;
      for (int v : wi) ni += v;
      for (int v : wj) nj += v;
      const uint32_t xi = up::ffn_xcd_rows(tiles_i);
      const int share = (int)((x % xi + 1) * tiles_i / xi - (x % xi) * tiles_i / xi);
      const int want_i = share < 4 ? share : 4;
      if (n == 32 && (ni < want_i || nj > (int)up::kFfnGroupJ)) {
        std::fprintf(stderr, "FAIL %u x %u: XCD %u's first 32 workgroups cover %d weight and %d token panels\n",
                     tiles_i, tiles_j, x, ni, nj);
        ++failures;
        return;
      }
    }
}

int main() {
  for (uint32_t ti = 1; ti <= 72; ++ti)
    for (uint32_t tj = 1; tj <= 70; ++tj) check_walk(ti, tj);
  const uint32_t big_i[] = {112, 120, 16, 15, 9, 8, 31, 32, 33, 7};
  const uint32_t big_j[] = {206, 512, 513, 1, 8, 9, 255};
  for (uint32_t ti : big_i)
    for (uint32_t tj : big_j) check_walk(ti, tj);
  if (failures) return 1;
  std::printf("ok %lld\n", checked);
  return 0;
}
