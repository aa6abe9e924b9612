// Host-side checks of the row-copy launch plan (copy_plan.h): the
// multiply-high division equals n / d for every divisor below 5000 at the
// dividends where rounding could go wrong and at random ones, and for random
// 32-bit divisors; every buffer gets a non-empty, disjoint workgroup range;
// a flat buffer's unit count fits 32 bits and its workgroups (at most the
// cap) cover every unit of max_rows rows in whole steps; and the plans of the
// measured row sizes.  Built with g++ by tests/test_abi.py; prints "ok N"
// after N checks.
#include <cstdint>
#include <cstdio>
#include <random>

#include "../token_level_block_amd/csrc/copy_plan.h"

static int failures = 0;
static long checks = 0;

#define CHECK(cond, ...)                        \
  do {                                          \
    ++checks;                                   \
    if (!(cond)) {                              \
      std::fprintf(stderr, "FAIL %s: ", #cond); \
      std::fprintf(stderr, __VA_ARGS__);        \
      std::fprintf(stderr, "\n");               \
      ++failures;                               \
    }                                           \
  } while (0)

static void check_div(uint32_t d, uint32_t n) {
  const up::FastDiv f = up::make_fastdiv(d);
  CHECK(up::fastdiv(n, f) == n / d, "d=%u n=%u: %u, expected %u", d, n, up::fastdiv(n, f), n / d);
}

int main() {
  std::mt19937_64 rng(12345);
  for (uint32_t d = 1; d < 5000; ++d) {
    const uint32_t edge[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 2 * d, 0x7FFFFFFFu, 0x80000000u,
                             0xFFFFFFFFu - d, 0xFFFFFFFEu, 0xFFFFFFFFu};
    for (uint32_t n : edge) check_div(d, n);
    // multiples of d and their neighbours near the top of the range
    const uint32_t top = 0xFFFFFFFFu / d * d;
    check_div(d, top);
    check_div(d, top - 1);
    for (int k = 0; k < 200; ++k) check_div(d, (uint32_t)rng());
  }
  for (int k = 0; k < 100000; ++k) {
    uint32_t d = (uint32_t)rng();
    if (d == 0) d = 1;
    check_div(d, (uint32_t)rng());
    check_div(d, 0xFFFFFFFFu);
    check_div(d, d);
  }

  // workgroup ranges and flat coverage
  const int64_t rbs[] = {4, 8, 12, 16, 32, 36, 48, 100, 2048, 4096, 7680, 8192, 16384};
  const int64_t rows[] = {1, 7, 4096, 30720, 131072, 2097152, 1 << 24, INT32_MAX};
  for (int64_t mr : rows)
    for (int nb = 1; nb <= up::kMaxCopyBuffers; ++nb) {
      int64_t rb[up::kMaxCopyBuffers];
      int32_t v16[up::kMaxCopyBuffers];
      for (int b = 0; b < nb; ++b) {
        rb[b] = rbs[(b * 5 + nb) % 13];
        v16[b] = (rb[b] % 16 == 0) && ((b + nb) % 3 != 0);
      }
      up::CopyPlan p;
      CHECK(up::make_copy_plan(nb, rb, v16, mr, &p), "plan for %d buffers", nb);
      for (int b = 0; b < nb; ++b) {
        const int64_t g = (int64_t)p.wg_begin[b + 1] - p.wg_begin[b];
        CHECK(g >= 1, "buffer %d of %d: %lld workgroups", b, nb, (long long)g);
        if (p.flat[b]) {
          CHECK(v16[b] && rb[b] > up::kCopyNarrowRow && rb[b] % 16 == 0, "flat buffer %d: row %lld", b,
                (long long)rb[b]);
          CHECK(p.units[b] == (uint32_t)(rb[b] / 16), "units");
          CHECK(mr * (int64_t)p.units[b] < (int64_t(1) << 32), "flat stream of %lld units",
                (long long)(mr * p.units[b]));
          CHECK(g <= up::kCopyFlatMaxGroups, "flat groups %lld", (long long)g);
          // a thread per four units of the longest stream, or the cap
          const int64_t units = mr * p.units[b];
          CHECK(g * 4 * up::kCopyThreads >= units || g == up::kCopyFlatMaxGroups,
                "stream of %lld units: groups %lld", (long long)units, (long long)g);
          CHECK((g - 1) * 4 * up::kCopyThreads < units, "stream of %lld units: %lld groups, one too many",
                (long long)units, (long long)g);
        } else {
          CHECK(g <= 4096, "row-copy groups %lld", (long long)g);
        }
      }
      CHECK(p.wg_begin[0] == 0 && p.wg_begin[up::kMaxCopyBuffers] == p.wg_begin[nb], "range ends");
      // the launch's threads fit the grid's 32-bit work-item count
      CHECK((int64_t)p.wg_begin[nb] * up::kCopyThreads < (int64_t(1) << 32), "%lld workgroups",
            (long long)p.wg_begin[nb]);
    }
  CHECK(!up::make_copy_plan(up::kMaxCopyBuffers + 1, nullptr, nullptr, 1, nullptr), "too many buffers");

  // the measured buffers: 8 KiB hidden rows at 128K (flat, the cap), positions (narrow),
  // Gemma-3-shaped 7680-byte rows at 64K (flat, 480 units: not a power of two)
  {
    const int64_t rb[] = {8192, 4};
    const int32_t v16[] = {1, 0};
    up::CopyPlan p;
    up::make_copy_plan(2, rb, v16, 131072, &p);
    // 131072 rows x 512 units: a thread per four units, 65536 workgroups
    CHECK(p.flat[0] == 1 && p.wg_begin[1] == 65536 && p.flat[1] == 0 &&
              p.wg_begin[2] == 65536 + 512,
          "128K plan: flat %d groups %d, narrow groups %d", p.flat[0], p.wg_begin[1], p.wg_begin[2] - p.wg_begin[1]);
    const int64_t rg[] = {7680};
    const int32_t vg[] = {1};
    up::make_copy_plan(1, rg, vg, 65536, &p);
    CHECK(p.flat[0] == 1 && p.units[0] == 480 && p.wg_begin[1] == 65536 * 480 / 1024, "Gemma plan");
    // 16 x 128K rows of 8 KiB: still a thread per four units (the cap, exactly)
    up::make_copy_plan(2, rb, v16, 2097152, &p);
    CHECK(p.flat[0] == 1 && p.wg_begin[1] == 2097152 * 512 / 1024 && p.wg_begin[1] == up::kCopyFlatMaxGroups,
          "16 x 128K plan: %d groups", p.wg_begin[1]);
  }
  if (failures) return 1;
  std::printf("ok %ld\n", checks);
  return 0;
}
