// Internal declarations shared by the HIP sources of libuniprefill.
// gfx950 (CDNA4) only: 64-lane wavefronts, 32x32x16 bf16 MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace up {

constexpr int kWave = 64;

// Device view of the per-request offsets that every kernel derives from
// cu_seqlens.  Written by the prep kernel into the select workspace.
struct Offsets {
  int32_t* cu;       // [R+1] cu_seqlens clamped to be non-decreasing and <= max_tokens
  int32_t* blk;      // [R+1] prefix sums of ceil(N_r / G)
  int32_t* chunk;    // [R+1] prefix sums of ceil(N_r / chunk_keys)
};

// ---------------------------------------------------------------------------
// Launchers (host functions defined next to their kernels).  Each returns
// hipSuccess or the launch error.
// ---------------------------------------------------------------------------
hipError_t launch_prep(const int32_t* cu_in, int32_t R, int64_t max_tokens, int32_t G,
                       int32_t chunk_keys, Offsets off, int32_t* block_offsets_out,
                       hipStream_t s);

struct ScoreArgs {
  const uint16_t* q;     // bf16 bits
  const uint16_t* k;
  int64_t q_stride;      // elements between tokens
  int64_t k_stride;
  Offsets off;
  int32_t R;
  int32_t hq, hkv, d;
  int32_t G, n;
  int32_t chunk_keys;    // keys per workgroup, a multiple of G
  float c;               // softmax scale * log2(e)
  float* lse;            // [max_blocks][hq*n]  log2-domain block partials
  float* chunk_lse;      // [max_chunks][hq*n]  log2-domain chunk partials
  int64_t max_chunks;
  // Offsets in the kernel itself (R < 64): cu_seqlens as the caller passed it,
  // clamped to [0, cap]; `off` is then written by workgroup (0, 0), and
  // block_offsets_out (optional) receives off.blk.  Null: `off` is ready.
  const int32_t* cu_in;
  int32_t cap;
  int32_t* block_offsets_out;
};
constexpr int kInlineOffsetsMaxReqs = 63;
hipError_t launch_score(const ScoreArgs& a, hipStream_t s);

struct CombineArgs {
  Offsets off;
  int32_t R, hq, n, G;
  const float* lse;
  const float* chunk_lse;
  float* row_lse;        // [R][hq*n]
  float* scores;         // out [sum nb]
  int64_t max_blocks;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

struct ToppArgs {
  Offsets off;
  int32_t R, G, A, n;
  double p;
  const float* scores;   // [sum nb]
  float* scores_copy;    // optional: scores copied here (may be null or == scores)
  uint8_t* keep_block;   // [sum nb]  (internal buffer when the caller passes none)
  uint8_t* mask;         // [max_tokens]
  int32_t* kept;         // [R]
  int64_t max_tokens;
  int64_t max_blocks;
  int32_t chunk_keys;    // tokens per key chunk (off.chunk counts these per request)
  int64_t max_chunks;    // grid: one workgroup per chunk, ids past off.chunk[R] exit
};
hipError_t launch_topp(const ToppArgs& a, hipStream_t s);

constexpr int kMaxCompactBuffers = 8;

struct RowBuffers {
  const uint8_t* src[kMaxCompactBuffers];
  uint8_t* dst[kMaxCompactBuffers];
  int64_t row_bytes[kMaxCompactBuffers];
  int32_t vec16[kMaxCompactBuffers];   // 1: row_bytes and both pointers 16-byte aligned
  int32_t nbuf;
};

struct CompactArgs {
  const uint8_t* mask;
  const int32_t* cu_in;
  int32_t R;
  int64_t max_tokens;
  RowBuffers bufs;
  const int32_t* index_in;
  int32_t* index_out;
  int32_t* cu_out;
  // workspace
  int32_t* tile_count;    // [num_count_tiles]
  int32_t* src_pos;       // [max_tokens] stream position of each kept row
  int64_t num_count_tiles;
};
hipError_t launch_compact(const CompactArgs& a, hipStream_t s);

hipError_t launch_scatter(const void* compacted, int64_t row_bytes, const int32_t* index_map,
                          const int32_t* count_ptr, int64_t max_tokens, void* full,
                          int64_t full_rows, hipStream_t s);

hipError_t launch_metadata(int32_t layer, int32_t L, int32_t R, const int32_t* cu_old,
                           const int32_t* cu_new, int32_t* seq_lens, int32_t* nat,
                           int32_t* drop_count, int32_t* drop_layer, int32_t* drop_len,
                           int32_t max_drops, int32_t* seqused_base, hipStream_t s);

// Tile sizes shared between the host planner and the kernels.
// Eq. 16 slot mapping over the stream rows k < max_tokens
struct SlotArgs {
  const int32_t* table;      // [R][table_stride] physical block ids
  int64_t table_stride;
  int32_t width;             // usable columns per table row
  int32_t B;                 // KV block size (tokens per physical block)
  const int32_t* cu;         // [R+1] stream offsets of the requests
  const int32_t* seq_lens;   // [R] patched lengths
  int32_t R;
  int64_t max_tokens;
  int64_t* slots;            // out [max_tokens]
};
hipError_t launch_slots(const SlotArgs& a, hipStream_t s);

// paged-cache write: cache row slots[k] <- key/value row k, k < min(cu[R], max_tokens)
struct KvWriteArgs {
  const uint8_t* key;
  int64_t key_stride;        // bytes between consecutive key rows
  const uint8_t* value;      // nullptr: keys only
  int64_t value_stride;
  int64_t row_bytes;         // bytes per cache row
  const int64_t* slots;
  const int32_t* cu;
  int32_t R;
  int64_t max_tokens;
  uint8_t* key_cache;        // [cache_slots][row_bytes]
  uint8_t* value_cache;
  int64_t cache_slots;
};
hipError_t launch_kv_write(const KvWriteArgs& a, bool vec, hipStream_t s);

constexpr int kCountTile = 4096;    // tokens per compaction count workgroup
constexpr int64_t kDirectRankMax = 131072;   // up to this many tokens compaction ranks in one launch
constexpr int kGatherTile = 256;    // tokens per compaction gather workgroup

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
// Request owning global index x given prefix offsets off[0..R]: the largest
// r with off[r] <= x (off non-decreasing).  Caller guarantees off[0] <= x < off[R].
__device__ __forceinline__ int find_owner(const int32_t* off, int R, int64_t x) {
  int lo = 0, hi = R;  // invariant: off[lo] <= x < off[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)off[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Inclusive scan over the workgroup (op = max or +); `scratch` holds one slot per wave.
template <bool kMax>
__device__ __forceinline__ int32_t block_inclusive_scan(int32_t v, int32_t* scratch) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    int32_t x = __shfl_up(v, o);
    if (lane >= o) v = kMax ? max(v, x) : v + x;
  }
  if (lane == 63) scratch[wid] = v;
  __syncthreads();
  int32_t pre = kMax ? INT32_MIN : 0;
  for (int w = 0; w < wid; ++w) pre = kMax ? max(pre, scratch[w]) : pre + scratch[w];
  __syncthreads();
  return kMax ? max(v, pre) : v + pre;
}

}  // namespace up
