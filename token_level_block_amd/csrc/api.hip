// C ABI of libuniprefill: argument validation, workspace layout and launch
// order.  Every check runs on the host before anything is enqueued, so a bad
// argument leaves all buffers untouched.
#include <math.h>

#include <mutex>

#include "../../include/uniprefill.h"
#include "../../include/uniprefill_prof.h"
#include "common.h"
#include "score_plan.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct SelectLayout {
  size_t cu, blk, chunk, keep, scores, chunk_lse, lse, row_lse, total;
  int64_t max_blocks, max_chunks;
  int32_t chunk_keys;
  bool scoring;
};

up_status check_select_params(const up_select_params* prm) {
  if (prm == nullptr) return UP_ERR_NULL;
  const bool scoring = (prm->flags & UP_SCORES_IN) == 0u;
  if (prm->flags & ~UP_SCORES_IN) return UP_ERR_PARAM;
  if (prm->num_heads_q < 1 || prm->num_heads_kv < 1) return UP_ERR_SHAPE;
  if (prm->num_heads_q % prm->num_heads_kv != 0) return UP_ERR_SHAPE;
  if (prm->block_size < 1 || prm->num_sink < 0 || prm->window < 1) return UP_ERR_PARAM;
  if (!(prm->top_p > 0.0 && prm->top_p <= 1.0)) return UP_ERR_PARAM;   // also rejects NaN
  if (scoring) {
    if (prm->head_dim != 64 && prm->head_dim != 128 && prm->head_dim != 256) return UP_ERR_PARAM;
    if (prm->block_size % 32 != 0) return UP_ERR_PARAM;
    if (!(isfinite(prm->softmax_scale))) return UP_ERR_PARAM;
    // rows of the block-partial workspace are indexed with 32-bit offsets per block
    if ((int64_t)prm->num_heads_q * prm->window > (1 << 24)) return UP_ERR_PARAM;
  } else {
    if (prm->head_dim < 1) return UP_ERR_PARAM;
  }
  return UP_OK;
}

up_status plan_select(const up_select_params* prm, int32_t R, int64_t max_tokens, SelectLayout* L) {
  up_status st = check_select_params(prm);
  if (st != UP_OK) return st;
  if (R < 0 || max_tokens < 0 || max_tokens > INT32_MAX) return UP_ERR_SHAPE;
  const int32_t G = prm->block_size;
  L->scoring = (prm->flags & UP_SCORES_IN) == 0u;
  L->chunk_keys = up::chunk_keys_for(G, prm->head_dim, prm->num_heads_q, prm->num_heads_kv, prm->window,
                                     max_tokens, R);
  L->max_blocks = max_tokens / G + R;
  L->max_chunks = max_tokens / L->chunk_keys + R;
  if (L->max_chunks > INT32_MAX) return UP_ERR_SHAPE;   // one top-p workgroup per chunk
  if (L->scoring) {
    // the score grid's x dimension enumerates (chunk rounded up to 8, query slice)
    const up::ScoreLaunch SL = up::score_launch_for(prm->head_dim, prm->num_heads_q, prm->num_heads_kv,
                                                    prm->window);
    if ((L->max_chunks + 7) / 8 * 8 * (int64_t)SL.zsplit > INT32_MAX) return UP_ERR_SHAPE;
  }
  const int64_t rows = (int64_t)prm->num_heads_q * prm->window;
  size_t off = 0;
  L->cu = off;      off = align_up(off + sizeof(int32_t) * (size_t)(R + 1));
  L->blk = off;     off = align_up(off + sizeof(int32_t) * (size_t)(R + 1));
  L->chunk = off;   off = align_up(off + sizeof(int32_t) * (size_t)(R + 1));
  L->keep = off;    off = align_up(off + (size_t)L->max_blocks);
  L->scores = off;  off = align_up(off + sizeof(float) * (size_t)L->max_blocks);
  if (L->scoring) {
    L->chunk_lse = off; off = align_up(off + sizeof(float) * (size_t)L->max_chunks * (size_t)rows);
    L->lse = off;       off = align_up(off + sizeof(float) * (size_t)L->max_blocks * (size_t)rows);
    L->row_lse = off;   off = align_up(off + sizeof(float) * (size_t)R * (size_t)rows);
  } else {
    L->chunk_lse = L->lse = L->row_lse = off;
  }
  L->total = off;
  return UP_OK;
}

// Every check of up_compact except the workspace; fills everything in `a`
// but the workspace pointers.  No side effects.
up_status prepare_compact(const uint8_t* keep_mask, const int32_t* cu_seqlens, int32_t num_reqs,
                          int64_t max_tokens, int32_t num_buffers, const void* const* src, void* const* dst,
                          const int64_t* row_bytes, const int32_t* index_in, int32_t* index_out,
                          int32_t* cu_seqlens_out, up::CompactArgs* a) {
  if (num_reqs < 0 || max_tokens < 0 || max_tokens > INT32_MAX) return UP_ERR_SHAPE;
  if (num_buffers < 0 || num_buffers > up::kMaxCompactBuffers) return UP_ERR_PARAM;
  if (keep_mask == nullptr || cu_seqlens == nullptr || index_out == nullptr || cu_seqlens_out == nullptr)
    return UP_ERR_NULL;
  if (num_buffers > 0 && (src == nullptr || dst == nullptr || row_bytes == nullptr)) return UP_ERR_NULL;
  a->bufs.nbuf = num_buffers;
  for (int b = 0; b < num_buffers; ++b) {
    if (src[b] == nullptr || dst[b] == nullptr) return UP_ERR_NULL;
    if (row_bytes[b] <= 0 || row_bytes[b] % 4 != 0) return UP_ERR_PARAM;
    if (!aligned(src[b], 4) || !aligned(dst[b], 4)) return UP_ERR_ALIGN;
    a->bufs.src[b] = static_cast<const uint8_t*>(src[b]);
    a->bufs.dst[b] = static_cast<uint8_t*>(dst[b]);
    a->bufs.row_bytes[b] = row_bytes[b];
    a->bufs.vec16[b] = (row_bytes[b] % 16 == 0 && aligned(src[b], 16) && aligned(dst[b], 16)) ? 1 : 0;
  }
  if (!aligned(keep_mask, 16)) return UP_ERR_ALIGN;
  a->num_count_tiles = (max_tokens + up::kCountTile - 1) / up::kCountTile;
  a->mask = keep_mask;
  a->cu_in = cu_seqlens;
  a->R = num_reqs;
  a->max_tokens = max_tokens;
  a->index_in = index_in;
  a->index_out = index_out;
  a->cu_out = cu_seqlens_out;
  return UP_OK;
}

// compaction workspace layout (up_compact_workspace_bytes): per-4096-token
// counts, then the stream position of each kept row
void place_compact_workspace(up::CompactArgs* a, uint8_t* ws) {
  const int64_t ntiles = a->num_count_tiles;
  a->tile_count = reinterpret_cast<int32_t*>(ws);
  a->src_pos = reinterpret_cast<int32_t*>(ws + align_up(sizeof(int32_t) * (size_t)(ntiles > 0 ? ntiles : 1)));
}

}  // namespace

// Scratch of up_compact_noalloc: one copy per GPU, alive until the process
// ends.  Host code never uses this name as an address (on the host it is a
// stand-in, not device memory): it uses the per-device address that
// hipGetSymbolAddress returns for it.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices];   // address of `scratch` on each device, null until looked up

// The device `stream` runs on, its copy of `scratch` (looked up once per
// device, with that device current).
up_status scratch_of_stream_device(hipStream_t stream, uint8_t** out) {
  int dev = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return UP_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return UP_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return UP_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return UP_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return UP_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return UP_OK;
}

}  // namespace

static_assert(((UP_COMPACT_NOALLOC_MAX_TOKENS + 4095) / 4096 * 4 + 255) / 256 * 256 +
                      (size_t)UP_COMPACT_NOALLOC_MAX_TOKENS * 4 <= kNoAllocScratchBytes,
              "the static scratch holds the compaction workspace of its largest stream");

extern "C" {

const char* up_status_string(up_status s) {
  switch (s) {
    case UP_OK: return "ok";
    case UP_ERR_NULL: return "a required pointer is NULL";
    case UP_ERR_SHAPE: return "inconsistent sizes";
    case UP_ERR_PARAM: return "parameter out of the supported range";
    case UP_ERR_WORKSPACE: return "workspace too small";
    case UP_ERR_ALIGN: return "pointer or stride not aligned as required";
    case UP_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int64_t up_max_blocks(int32_t block_size, int32_t num_reqs, int64_t max_tokens) {
  if (block_size < 1 || num_reqs < 0 || max_tokens < 0) return -1;
  return max_tokens / block_size + num_reqs;
}

size_t up_select_workspace_bytes(const up_select_params* prm, int32_t num_reqs, int64_t max_tokens) {
  SelectLayout L;
  if (plan_select(prm, num_reqs, max_tokens, &L) != UP_OK) return 0;
  return L.total;
}

}  // extern "C"

namespace {

// up_select_blocks, with optional events recorded on `stream` right before
// and after the score kernel (instrumentation: up_select_blocks_profiled)
up_status select_blocks_impl(const up_select_params* prm, const void* q, int64_t q_row_stride,
                             const void* k, int64_t k_row_stride, const int32_t* cu_seqlens,
                             int32_t num_reqs, int64_t max_tokens, const float* scores_in,
                             float* block_scores, int32_t* block_offsets, uint8_t* keep_block,
                             uint8_t* keep_mask, int32_t* kept_per_req, void* workspace,
                             size_t workspace_bytes, hipStream_t stream, hipEvent_t ev_begin,
                             hipEvent_t ev_end) {
  SelectLayout L;
  up_status st = plan_select(prm, num_reqs, max_tokens, &L);
  if (st != UP_OK) return st;
  if (cu_seqlens == nullptr || keep_mask == nullptr || kept_per_req == nullptr || workspace == nullptr)
    return UP_ERR_NULL;
  if (L.scoring) {
    if (q == nullptr || k == nullptr) return UP_ERR_NULL;
    const int64_t d = prm->head_dim;
    if (q_row_stride < prm->num_heads_q * d || k_row_stride < prm->num_heads_kv * d) return UP_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(k, 16) || q_row_stride % 8 != 0 || k_row_stride % 8 != 0)
      return UP_ERR_ALIGN;
  } else {
    if (scores_in == nullptr) return UP_ERR_NULL;
  }
  if (!aligned(workspace, kAlign)) return UP_ERR_ALIGN;
  if (workspace_bytes < L.total) return UP_ERR_WORKSPACE;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  up::Offsets off;
  off.cu = reinterpret_cast<int32_t*>(ws + L.cu);
  off.blk = reinterpret_cast<int32_t*>(ws + L.blk);
  off.chunk = reinterpret_cast<int32_t*>(ws + L.chunk);
  uint8_t* keep = keep_block ? keep_block : (ws + L.keep);
  const int32_t R = num_reqs;

  // a batch of at most 63 requests has its offsets derived inside the score
  // kernel (one request per lane); otherwise, and without scoring, the prep
  // kernel writes them first
  const bool inline_offsets = L.scoring && R >= 1 && R <= up::kInlineOffsetsMaxReqs;
  if (!inline_offsets &&
      up::launch_prep(cu_seqlens, R, max_tokens, prm->block_size, L.chunk_keys, off, block_offsets,
                      stream) != hipSuccess)
    return UP_ERR_HIP;

  const float* scores = scores_in;
  float* scores_copy = nullptr;
  if (L.scoring) {
    float* out = block_scores ? block_scores : reinterpret_cast<float*>(ws + L.scores);
    const double scale = prm->softmax_scale > 0.f ? (double)prm->softmax_scale
                                                  : 1.0 / sqrt((double)prm->head_dim);
    up::ScoreArgs sa;
    sa.q = static_cast<const uint16_t*>(q);
    sa.k = static_cast<const uint16_t*>(k);
    sa.q_stride = q_row_stride;
    sa.k_stride = k_row_stride;
    sa.off = off;
    sa.R = R;
    sa.hq = prm->num_heads_q;
    sa.hkv = prm->num_heads_kv;
    sa.d = prm->head_dim;
    sa.G = prm->block_size;
    sa.n = prm->window;
    sa.chunk_keys = L.chunk_keys;
    sa.c = (float)(scale * 1.4426950408889634074);
    sa.lse = reinterpret_cast<float*>(ws + L.lse);
    sa.chunk_lse = reinterpret_cast<float*>(ws + L.chunk_lse);
    sa.max_chunks = L.max_chunks;
    sa.cu_in = inline_offsets ? cu_seqlens : nullptr;
    sa.cap = (int32_t)max_tokens;
    sa.block_offsets_out = block_offsets;
    if (ev_begin != nullptr && hipEventRecord(ev_begin, stream) != hipSuccess) return UP_ERR_HIP;
    if (up::launch_score(sa, stream) != hipSuccess) return UP_ERR_HIP;
    if (ev_end != nullptr && hipEventRecord(ev_end, stream) != hipSuccess) return UP_ERR_HIP;
    up::CombineArgs ca;
    ca.off = off;
    ca.R = R;
    ca.hq = prm->num_heads_q;
    ca.n = prm->window;
    ca.G = prm->block_size;
    ca.lse = sa.lse;
    ca.chunk_lse = sa.chunk_lse;
    ca.row_lse = reinterpret_cast<float*>(ws + L.row_lse);
    ca.scores = out;
    ca.max_blocks = L.max_blocks;
    if (up::launch_combine(ca, stream) != hipSuccess) return UP_ERR_HIP;
    scores = out;
  } else {
    scores_copy = block_scores;
  }

  up::ToppArgs ta;
  ta.off = off;
  ta.R = R;
  ta.G = prm->block_size;
  ta.A = prm->num_sink;
  ta.n = prm->window;
  ta.p = prm->top_p;
  ta.scores = scores;
  ta.scores_copy = scores_copy;
  ta.keep_block = keep;
  ta.mask = keep_mask;
  ta.kept = kept_per_req;
  ta.max_tokens = max_tokens;
  ta.max_blocks = L.max_blocks;
  ta.chunk_keys = L.chunk_keys;
  ta.max_chunks = L.max_chunks;
  if (up::launch_topp(ta, stream) != hipSuccess) return UP_ERR_HIP;
  return UP_OK;
}

}  // namespace

extern "C" {

up_status up_select_blocks(const up_select_params* prm, const void* q, int64_t q_row_stride,
                           const void* k, int64_t k_row_stride, const int32_t* cu_seqlens,
                           int32_t num_reqs, int64_t max_tokens, const float* scores_in,
                           float* block_scores, int32_t* block_offsets, uint8_t* keep_block,
                           uint8_t* keep_mask, int32_t* kept_per_req, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  return select_blocks_impl(prm, q, q_row_stride, k, k_row_stride, cu_seqlens, num_reqs, max_tokens,
                            scores_in, block_scores, block_offsets, keep_block, keep_mask, kept_per_req,
                            workspace, workspace_bytes, stream, nullptr, nullptr);
}

up_status up_select_blocks_profiled(const up_select_params* prm, const void* q, int64_t q_row_stride,
                                    const void* k, int64_t k_row_stride, const int32_t* cu_seqlens,
                                    int32_t num_reqs, int64_t max_tokens, const float* scores_in,
                                    float* block_scores, int32_t* block_offsets, uint8_t* keep_block,
                                    uint8_t* keep_mask, int32_t* kept_per_req, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream, void* score_begin,
                                    void* score_end) {
  return select_blocks_impl(prm, q, q_row_stride, k, k_row_stride, cu_seqlens, num_reqs, max_tokens,
                            scores_in, block_scores, block_offsets, keep_block, keep_mask, kept_per_req,
                            workspace, workspace_bytes, stream, static_cast<hipEvent_t>(score_begin),
                            static_cast<hipEvent_t>(score_end));
}

size_t up_compact_workspace_bytes(int32_t num_reqs, int64_t max_tokens) {
  if (num_reqs < 0 || max_tokens < 0 || max_tokens > INT32_MAX) return 0;
  // per-4096-token counts, then the stream position of each kept row
  const int64_t ntiles = (max_tokens + up::kCountTile - 1) / up::kCountTile;
  size_t off = align_up(sizeof(int32_t) * (size_t)(ntiles > 0 ? ntiles : 1));
  off = align_up(off + sizeof(int32_t) * (size_t)(max_tokens > 0 ? max_tokens : 1));
  return off;
}

up_status up_compact(const uint8_t* keep_mask, const int32_t* cu_seqlens, int32_t num_reqs,
                     int64_t max_tokens, int32_t num_buffers, const void* const* src,
                     void* const* dst, const int64_t* row_bytes, const int32_t* index_in,
                     int32_t* index_out, int32_t* cu_seqlens_out, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  up::CompactArgs a;
  const up_status st = prepare_compact(keep_mask, cu_seqlens, num_reqs, max_tokens, num_buffers, src, dst,
                                       row_bytes, index_in, index_out, cu_seqlens_out, &a);
  if (st != UP_OK) return st;
  if (workspace == nullptr) return UP_ERR_NULL;
  if (!aligned(workspace, kAlign)) return UP_ERR_ALIGN;
  if (workspace_bytes < up_compact_workspace_bytes(num_reqs, max_tokens)) return UP_ERR_WORKSPACE;
  place_compact_workspace(&a, static_cast<uint8_t*>(workspace));
  if (up::launch_compact(a, stream) != hipSuccess) return UP_ERR_HIP;
  return UP_OK;
}

up_status up_compact_noalloc(const uint8_t* keep_mask, const int32_t* cu_seqlens, int32_t num_reqs,
                             int64_t max_tokens, int32_t num_buffers, const void* const* src,
                             void* const* dst, const int64_t* row_bytes, const int32_t* index_in,
                             int32_t* index_out, int32_t* cu_seqlens_out, hipStream_t stream) {
  up::CompactArgs a;
  const up_status st = prepare_compact(keep_mask, cu_seqlens, num_reqs, max_tokens, num_buffers, src, dst,
                                       row_bytes, index_in, index_out, cu_seqlens_out, &a);
  if (st != UP_OK) return st;
  if (max_tokens > UP_COMPACT_NOALLOC_MAX_TOKENS) return UP_ERR_WORKSPACE;
  uint8_t* ws = nullptr;
  if (scratch_of_stream_device(stream, &ws) != UP_OK) return UP_ERR_HIP;
  place_compact_workspace(&a, ws);
  if (up::launch_compact(a, stream) != hipSuccess) return UP_ERR_HIP;
  return UP_OK;
}

up_status up_scatter_back(const void* compacted, int64_t row_bytes, const int32_t* index_map,
                          const int32_t* cu_seqlens_out, int32_t num_reqs, int64_t max_tokens,
                          void* full, int64_t full_rows, hipStream_t stream) {
  if (num_reqs < 0 || max_tokens < 0 || max_tokens > INT32_MAX || full_rows < 0) return UP_ERR_SHAPE;
  if (compacted == nullptr || index_map == nullptr || cu_seqlens_out == nullptr || full == nullptr)
    return UP_ERR_NULL;
  if (row_bytes <= 0 || row_bytes % 4 != 0) return UP_ERR_PARAM;
  if (!aligned(compacted, 4) || !aligned(full, 4)) return UP_ERR_ALIGN;
  if (up::launch_scatter(compacted, row_bytes, index_map, cu_seqlens_out + num_reqs, max_tokens, full,
                         full_rows, stream) != hipSuccess)
    return UP_ERR_HIP;
  return UP_OK;
}

up_status up_update_metadata(int32_t layer, int32_t num_layers, int32_t num_reqs,
                             const int32_t* cu_seqlens_old, const int32_t* cu_seqlens_new,
                             int32_t* seq_lens, int32_t* num_actual_tokens, int32_t* drop_count,
                             int32_t* drop_layer, int32_t* drop_len, int32_t max_drops,
                             int32_t* seqused_base, hipStream_t stream) {
  if (num_reqs < 0 || layer < 0 || max_drops < 0) return UP_ERR_SHAPE;
  if (seqused_base != nullptr && num_layers < 0) return UP_ERR_SHAPE;
  if (cu_seqlens_old == nullptr || cu_seqlens_new == nullptr || seq_lens == nullptr ||
      num_actual_tokens == nullptr || drop_count == nullptr)
    return UP_ERR_NULL;
  if (max_drops > 0 && (drop_layer == nullptr || drop_len == nullptr)) return UP_ERR_NULL;
  if (up::launch_metadata(layer, seqused_base ? num_layers : 0, num_reqs, cu_seqlens_old,
                          cu_seqlens_new, seq_lens, num_actual_tokens, drop_count, drop_layer,
                          drop_len, max_drops, seqused_base, stream) != hipSuccess)
    return UP_ERR_HIP;
  return UP_OK;
}

up_status up_slot_mapping(const int32_t* block_table, int64_t block_table_stride,
                          int32_t max_blocks_per_req, int32_t kv_block_size,
                          const int32_t* cu_seqlens, const int32_t* seq_lens, int32_t num_reqs,
                          int64_t max_tokens, int64_t* slot_mapping, hipStream_t stream) {
  if (num_reqs < 0 || max_tokens < 0 || max_tokens > INT32_MAX) return UP_ERR_SHAPE;
  if (max_blocks_per_req < 0 || block_table_stride < max_blocks_per_req) return UP_ERR_SHAPE;
  if (kv_block_size < 1) return UP_ERR_PARAM;
  if (cu_seqlens == nullptr || seq_lens == nullptr || slot_mapping == nullptr) return UP_ERR_NULL;
  if (block_table == nullptr && max_blocks_per_req > 0) return UP_ERR_NULL;
  if (!aligned(cu_seqlens, 4) || !aligned(seq_lens, 4) || !aligned(block_table, 4) ||
      !aligned(slot_mapping, 8))
    return UP_ERR_ALIGN;
  up::SlotArgs a{};
  a.table = block_table;
  a.table_stride = block_table_stride;
  a.width = max_blocks_per_req;
  a.B = kv_block_size;
  a.cu = cu_seqlens;
  a.seq_lens = seq_lens;
  a.R = num_reqs;
  a.max_tokens = max_tokens;
  a.slots = slot_mapping;
  return up::launch_slots(a, stream) == hipSuccess ? UP_OK : UP_ERR_HIP;
}

up_status up_write_kv_cache(const void* key, int64_t key_row_stride, const void* value,
                            int64_t value_row_stride, int64_t row_bytes, const int64_t* slot_mapping,
                            const int32_t* cu_seqlens, int32_t num_reqs, int64_t max_tokens,
                            void* key_cache, void* value_cache, int64_t cache_slots,
                            hipStream_t stream) {
  if (num_reqs < 0 || max_tokens < 0 || max_tokens > INT32_MAX || cache_slots < 0) return UP_ERR_SHAPE;
  if (row_bytes < 4 || row_bytes % 4 != 0) return UP_ERR_PARAM;
  if (key == nullptr || key_cache == nullptr || slot_mapping == nullptr || cu_seqlens == nullptr)
    return UP_ERR_NULL;
  if ((value == nullptr) != (value_cache == nullptr)) return UP_ERR_NULL;
  if (key_row_stride < row_bytes || (value != nullptr && value_row_stride < row_bytes)) return UP_ERR_SHAPE;
  if (key_row_stride % 4 != 0 || (value != nullptr && value_row_stride % 4 != 0)) return UP_ERR_ALIGN;
  if (!aligned(key, 4) || !aligned(value, 4) || !aligned(key_cache, 4) || !aligned(value_cache, 4) ||
      !aligned(slot_mapping, 8) || !aligned(cu_seqlens, 4))
    return UP_ERR_ALIGN;
  const bool vec = row_bytes % 16 == 0 && key_row_stride % 16 == 0 && aligned(key, 16) &&
                   aligned(key_cache, 16) &&
                   (value == nullptr || (value_row_stride % 16 == 0 && aligned(value, 16) &&
                                         aligned(value_cache, 16)));
  up::KvWriteArgs a{};
  a.key = static_cast<const uint8_t*>(key);
  a.key_stride = key_row_stride;
  a.value = static_cast<const uint8_t*>(value);
  a.value_stride = value == nullptr ? 0 : value_row_stride;
  a.row_bytes = row_bytes;
  a.slots = slot_mapping;
  a.cu = cu_seqlens;
  a.R = num_reqs;
  a.max_tokens = max_tokens;
  a.key_cache = static_cast<uint8_t*>(key_cache);
  a.value_cache = static_cast<uint8_t*>(value_cache);
  a.cache_slots = cache_slots;
  return up::launch_kv_write(a, vec, stream) == hipSuccess ? UP_OK : UP_ERR_HIP;
}

}  // extern "C"
