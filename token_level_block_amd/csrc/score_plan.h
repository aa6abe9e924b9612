// Launch plan of the score kernel that depends on the problem size: how many
// keys one workgroup scores.
#pragma once

#include <stdint.h>

namespace up {

// Keys per score workgroup.  A workgroup pays a fixed start-up (its query
// fragments and first K stage arrive before any MFMA can issue), so chunks are
// made as long as possible while one launch still offers about one workgroup
// per resident slot: 256 CUs, one 8-wave workgroup per CU at the score
// kernel's register use (two 4-wave ones when a KV head has at most 256
// window queries).  The length is a multiple of G (so no G-block straddles two
// workgroups), between the multiple of G nearest 128 from above (one LDS stage:
// short batches still fill the chip) and 8192 keys.
inline int32_t chunk_keys_for(int32_t G, int32_t hq, int32_t hkv, int32_t n, int64_t max_tokens) {
  const int32_t base = G >= 128 ? G : G * ((128 + G - 1) / G);
  if (hkv < 1 || hq < hkv || n < 1) return base;
  const int64_t qn = (int64_t)(hq / hkv) * n;
  const int64_t zsplit = qn <= 256 ? 1 : (qn + 511) / 512;
  const int64_t slots = qn <= 256 ? 512 : 256;
  const int64_t want = (max_tokens * hkv * zsplit + slots - 1) / slots;
  const int64_t cap = base > 8192 ? base : 8192;
  int64_t ck = (want + base - 1) / base * base;
  if (ck < base) ck = base;
  if (ck > cap) ck = cap / base * base;
  return (int32_t)ck;
}

}  // namespace up
