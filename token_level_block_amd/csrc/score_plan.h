// Launch plan of the score kernel that depends on the problem size: how many
// keys one workgroup scores.
#pragma once

#include <stdint.h>

namespace up {

// Launch shape of the score kernel for one KV head's qn = (Hq/Hkv)*n window
// queries: waves per workgroup, 32-query column tiles per wave, query slices
// (workgroups per key chunk), and how many such workgroups one CU holds at
// the kernel's register use.  Two column tiles per wave halve the LDS reads
// per MFMA; at d = 256 with at most 256 queries that would leave one wave per
// SIMD (query fragments and accumulators of two tiles at d = 256 take 260
// registers), so that case uses one tile per wave and eight waves.  At most
// 128 queries (a short window, or few query heads per KV head) fill four
// waves of one tile exactly, where two tiles would pad half the MFMA work.
struct ScoreLaunch {
  int nw, nt, zsplit, per_cu;
};

inline ScoreLaunch score_launch_for(int32_t d, int32_t hq, int32_t hkv, int32_t n) {
  const int64_t qn = (int64_t)(hq / hkv) * n;
  if (qn <= 128) return {4, 1, 1, 2};
  if (d > 128 && qn <= 256) return {8, 1, 1, 1};
  if (qn <= 256) return {4, 2, 1, 2};
  return {8, 2, (int)((qn + 511) / 512), 1};
}

// Keys per score workgroup.  A workgroup pays a fixed start-up (its query
// fragments and first K stage arrive before any MFMA can issue), so chunks are
// made as long as possible while one launch still offers about one workgroup
// per resident slot (256 CUs times the workgroups a CU holds).  The length is
// a multiple of G (so no G-block straddles two workgroups), between the
// multiple of G nearest 128 from above (one LDS stage: short batches still
// fill the chip) and 16384 keys (long batches then need fewer rounds of
// workgroups).  With more than one request every request ends in a partial
// chunk of unknown length (the lengths live on the device), and long chunks
// leave the last round of workgroups part-filled: there the length is held to
// 4096 keys.  A list-scheduling model of the launch (start-up plus keys at the
// measured rate) puts this within a few percent of the best length on uniform
// multi-request batches (16384 is best when every request is a multiple of it)
// and 13-18 % ahead of longer chunks on ragged ones.
inline int32_t chunk_keys_for(int32_t G, int32_t d, int32_t hq, int32_t hkv, int32_t n, int64_t max_tokens,
                              int32_t num_reqs) {
  const int32_t base = G >= 128 ? G : G * ((128 + G - 1) / G);
  if (hkv < 1 || hq < hkv || n < 1) return base;
  const ScoreLaunch L = score_launch_for(d, hq, hkv, n);
  const int64_t slots = 256 * (int64_t)L.per_cu;
  const int64_t want = (max_tokens * hkv * L.zsplit + slots - 1) / slots;
  const int64_t limit = num_reqs > 1 ? 4096 : 16384;
  const int64_t cap = base > limit ? base : limit;
  int64_t ck = (want + base - 1) / base * base;
  if (ck < base) ck = base;
  if (ck > cap) ck = cap / base * base;
  return (int32_t)ck;
}

}  // namespace up
