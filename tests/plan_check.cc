// Host-side checks of the score kernel's launch planner (score_plan.h):
// every window query is covered by exactly the planned slices, shapes stay
// within what the kernel is built for (two waves per SIMD: waves per CU at
// most 8; two query tiles at d = 256 only with eight waves), and chunk lengths
// are multiples of G inside their documented bounds.  Also pins the launch
// shapes of the workloads the benchmark and sweep measure.  Built with g++
// by tests/test_abi.py; prints "ok N" after N checked configurations.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>

#include "../token_level_block_amd/csrc/score_plan.h"

static int failures = 0;

#define CHECK(cond, ...)                                     \
  do {                                                       \
    if (!(cond)) {                                           \
      std::fprintf(stderr, "FAIL %s: ", #cond);              \
      std::fprintf(stderr, __VA_ARGS__);                     \
      std::fprintf(stderr, "\n");                            \
      ++failures;                                            \
    }                                                        \
  } while (0)

static void pin(int d, int hq, int hkv, int n, int G, int64_t T, int R, int nw, int nt, int zs, int per_cu,
                int chunk) {
  const up::ScoreLaunch L = up::score_launch_for(d, hq, hkv, n);
  const int32_t ck = up::chunk_keys_for(G, d, hq, hkv, n, T, R);
  CHECK(L.nw == nw && L.nt == nt && L.zsplit == zs && L.per_cu == per_cu && ck == chunk,
        "d=%d hq=%d hkv=%d n=%d G=%d T=%lld R=%d: plan {%d,%d,%d,%d} chunk %d, expected {%d,%d,%d,%d} chunk %d", d,
        hq, hkv, n, G, (long long)T, R, L.nw, L.nt, L.zsplit, L.per_cu, ck, nw, nt, zs, per_cu, chunk);
}

int main() {
  const int ds[] = {64, 128, 256};
  const int heads[][2] = {{32, 8}, {16, 2}, {16, 8}, {4, 4}, {8, 1}, {64, 8}, {2, 2}, {32, 1}};
  const int ns[] = {1, 8, 16, 32, 100, 128, 256, 512, 4096};
  const int Gs[] = {32, 64, 96, 128, 4096, 32768};
  const int64_t Ts[] = {1, 100, 4096, 30720, 131072, 2097152, INT32_MAX};
  long checked = 0;
  for (int d : ds)
    for (const auto& h : heads)
      for (int n : ns) {
        const int hq = h[0], hkv = h[1];
        const int64_t qn = (int64_t)(hq / hkv) * n;
        const up::ScoreLaunch L = up::score_launch_for(d, hq, hkv, n);
        const int64_t per_slice = (int64_t)L.nw * 32 * L.nt;
        CHECK(L.nw == 4 || L.nw == 8, "nw %d", L.nw);
        CHECK(L.nt == 1 || L.nt == 2, "nt %d", L.nt);
        CHECK(L.per_cu == 1 || L.per_cu == 2, "per_cu %d", L.per_cu);
        CHECK(L.per_cu * L.nw <= 8, "waves per CU %d (two per SIMD at most)", L.per_cu * L.nw);
        CHECK(!(d > 128 && L.nt == 2 && L.nw == 4), "d=%d with two tiles needs eight waves", d);
        CHECK(L.zsplit >= 1 && L.zsplit * per_slice >= qn && (L.zsplit - 1) * per_slice < qn,
              "qn=%lld not covered exactly by %d slices of %lld", (long long)qn, L.zsplit, (long long)per_slice);
        // the kernel derives the slice count from its template shape the same way
        CHECK((qn + per_slice - 1) / per_slice == L.zsplit, "in-kernel slice count differs for qn=%lld",
              (long long)qn);
        for (int G : Gs)
          for (int64_t T : Ts)
            for (int R : {0, 1, 2, 16}) {
              const int32_t ck = up::chunk_keys_for(G, d, hq, hkv, n, T, R);
              const int32_t base = G >= 128 ? G : G * ((128 + G - 1) / G);
              const int32_t limit = R > 1 ? 4096 : 16384;
              const int32_t cap = base > limit ? base : limit;
              CHECK(ck % G == 0, "chunk %d not a multiple of G=%d", ck, G);
              CHECK(ck >= base && ck <= cap, "chunk %d outside [%d, %d] (G=%d T=%lld R=%d)", ck, base, cap, G,
                    (long long)T, R);
              // more requests never lengthen the chunk
              if (R > 1) CHECK(ck <= up::chunk_keys_for(G, d, hq, hkv, n, T, 1), "chunk grows with R=%d", R);
              CHECK(ck % base == 0, "chunk %d not a multiple of the one-stage length %d", ck, base);
              ++checked;
            }
      }
  // the measured workloads (benchmark, sweep, ablations)
  pin(128, 32, 8, 128, 64, 131072, 1, 8, 2, 1, 1, 4096);      // LLaMA-3.1-8B-shaped 128K layer
  pin(128, 32, 8, 128, 64, 4096, 1, 8, 2, 1, 1, 128);         // its 4K request
  pin(128, 32, 8, 128, 64, 30720, 4, 8, 2, 1, 1, 1024);       // four ragged requests, 30K tokens
  pin(128, 32, 8, 32, 64, 131072, 1, 4, 1, 1, 2, 2048);       // n = 32 window
  pin(128, 32, 8, 512, 64, 131072, 1, 8, 2, 4, 1, 16384);     // n = 512 window
  pin(256, 16, 2, 128, 64, 65536, 1, 8, 2, 2, 1, 1024);       // Qwen3-Next-shaped 64K layer
  pin(256, 16, 8, 128, 64, 65536, 1, 8, 1, 1, 1, 2048);       // Gemma-3-shaped 64K layer
  pin(128, 32, 8, 128, 64, 2097152, 16, 8, 2, 1, 1, 4096);    // 16 x 128K serving batch
  pin(128, 32, 8, 128, 64, 1099200, 16, 8, 2, 1, 1, 4096);    // its second drop layer (ragged)
  pin(128, 32, 8, 128, 64, 2097152, 1, 8, 2, 1, 1, 16384);    // one 2M-token request
  if (failures) {
    std::fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  std::printf("ok %ld\n", checked);
  return 0;
}
