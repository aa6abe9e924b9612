// Launch plan of the row copies (compaction gather, Eq. 8 scatter) that the
// host computes: how many workgroups each buffer gets and, for buffers copied
// as a flat stream of 16-byte units, the constants that turn a unit index into
// its row without a hardware divide.  Plain C++: the same code serves the
// launcher and a host-side test.
#pragma once

#include <stdint.h>

namespace up {

// Unsigned 32-bit division by an invariant d >= 1 through a multiply-high
// (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", 1994, the round-up method for full-range dividends):
// with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
//     t = mulhi(m, n),  n / d = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0)
// for every n < 2^32.  m fits 32 bits because 2^l - d < d.
struct FastDiv {
  uint32_t m = 1;
  uint32_t s1 = 0, s2 = 0;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while (l < 32 && (uint64_t(1) << l) < d) ++l;
  const uint64_t num = (uint64_t(1) << 32) * ((uint64_t(1) << l) - d);
  FastDiv f;
  f.m = (uint32_t)(num / d + 1);
  f.s1 = l < 1 ? l : 1;
  f.s2 = l > 1 ? l - 1 : 0;
  return f;
}

// (constexpr: also callable from device code)
constexpr uint32_t fastdiv(uint32_t n, FastDiv f) {
  const uint32_t t = (uint32_t)(((uint64_t)f.m * n) >> 32);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

constexpr int kMaxCopyBuffers = 8;
constexpr int kCopyThreads = 256;
constexpr int64_t kCopyNarrowRow = 32;          // rows up to this many bytes go one per thread
constexpr int64_t kCopyFlatMaxGroups = 1 << 20;   // workgroups of one flat-copied buffer, at most

// Per-buffer workgroup ranges of one copy launch: buffer b owns workgroups
// [wg_begin[b], wg_begin[b+1]).  A buffer whose rows are 16-byte multiples
// wider than kCopyNarrowRow (and 16-byte aligned) is copied flat: its kept
// rows form one stream of 16-byte units, one unit per thread per step, and
// consecutive workgroups take consecutive units, so at any moment the chip
// streams one window of memory.  How many threads: the kept count is only
// known on the device, and threads that find no unit still cost their launch
// (about 10 us per 8 M idle threads measured), while fewer threads per unit
// stream more slowly (8 KiB rows, 40 % of 131072 kept: 136 us at 16.8 M
// threads, 144 us at 4.2 M; four units per thread per step: 164 us).  So a
// buffer gets one thread per four 16-byte units of every row the call may
// copy.  The same rule holds for long streams: a grid held to 65536
// workgroups makes each thread loop over the stream (16 x 131072 rows of
// 8 KiB at 52 % kept: 33 steps, 5.3 TB/s), and a plain copy measured the
// same way drops from 6.45 TB/s in one pass to 5.2 TB/s once it loops over
// more than 4 GiB.  The cap of 2^20 workgroups (2^28 threads) covers every
// stream the flat path takes, which needs max_rows * units below 2^32, and
// keeps the launch of eight such buffers under 2^31 threads.  Other buffers
// copy a row per thread (narrow rows) or per wave.
struct CopyPlan {
  int32_t wg_begin[kMaxCopyBuffers + 1];
  int32_t flat[kMaxCopyBuffers];
  uint32_t units[kMaxCopyBuffers];        // 16-byte units per row (flat buffers)
  FastDiv div[kMaxCopyBuffers];           // division by units[b]
};

inline int64_t copy_groups_for(int64_t max_rows, int64_t row_bytes, bool vec16, bool* flat) {
  const int64_t units = row_bytes / 16;
  *flat = vec16 && row_bytes > kCopyNarrowRow && max_rows * units < (int64_t(1) << 32);
  int64_t g;
  if (*flat) {
    g = (max_rows * units + 4 * kCopyThreads - 1) / (4 * kCopyThreads);
    if (g > kCopyFlatMaxGroups) g = kCopyFlatMaxGroups;
  } else {
    // a row per thread, or per wave for wide rows: up to 4096 workgroups
    const int64_t per = row_bytes <= kCopyNarrowRow ? kCopyThreads : kCopyThreads / 64;
    g = (max_rows + per - 1) / per;
    if (g > 4096) g = 4096;
  }
  return g < 1 ? 1 : g;
}

// Fills the plan for n buffers; returns false if n is out of range.
inline bool make_copy_plan(int n, const int64_t* row_bytes, const int32_t* vec16, int64_t max_rows, CopyPlan* p) {
  if (n < 0 || n > kMaxCopyBuffers) return false;
  int64_t at = 0;
  for (int b = 0; b < n; ++b) {
    bool flat = false;
    const int64_t g = copy_groups_for(max_rows, row_bytes[b], vec16[b] != 0, &flat);
    p->wg_begin[b] = (int32_t)at;
    p->flat[b] = flat ? 1 : 0;
    p->units[b] = flat ? (uint32_t)(row_bytes[b] / 16) : 1u;
    p->div[b] = make_fastdiv(p->units[b]);
    at += g;
  }
  for (int b = n; b <= kMaxCopyBuffers; ++b) p->wg_begin[b] = (int32_t)at;
  for (int b = n; b < kMaxCopyBuffers; ++b) {
    p->flat[b] = 0;
    p->units[b] = 1u;
    p->div[b] = make_fastdiv(1u);
  }
  return true;
}

}  // namespace up
