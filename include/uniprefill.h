/*
 * uniprefill.h - C ABI of the UniPrefill token-selection hot path on MI355X (gfx950).
 *
 * The operations follow "UniPrefill: Universal Long-Context Prefill
 * Acceleration via Block-wise Dynamic Sparsification" (arXiv 2605.06221),
 * cited below as "UniPrefill" with section and equation numbers.
 *
 * Conventions shared by every call
 *   - All buffers are caller-owned DEVICE memory unless marked (host).
 *   - Every call only enqueues work on `stream` (a hipStream_t; 0 is the null
 *     stream).  No call allocates, frees or synchronises, and the library
 *     keeps no global state (the one exception is the per-GPU scratch of
 *     up_compact_noalloc, below): calls are re-entrant and thread-safe on
 *     disjoint buffers.
 *   - Arguments are validated on the host before anything is enqueued.  A bad
 *     argument returns a negative up_status and changes nothing.  A failed
 *     launch returns UP_ERR_HIP.  Faults inside kernels surface at the
 *     caller's next synchronisation, as for any HIP work.
 *   - The token stream is cu_seqlens-packed (UniPrefill Sec. 3.5, "Kernel
 *     design"): request r owns tokens [cu_seqlens[r], cu_seqlens[r+1]) of every
 *     token-major buffer.  cu_seqlens lives on the device; the host passes only
 *     num_reqs and max_tokens, an upper bound on cu_seqlens[num_reqs] that
 *     sizes grids.  Kernels clamp cu_seqlens to be non-decreasing and within
 *     [0, max_tokens], so inconsistent offsets cannot cause out-of-bounds
 *     accesses (the results for such input are unspecified).
 *   - Data-dependent sizes (kept counts, new offsets) stay on the device.
 */
#ifndef UNIPREFILL_H
#define UNIPREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum up_status {
  UP_OK = 0,
  UP_ERR_NULL = -1,       /* a required pointer is NULL */
  UP_ERR_SHAPE = -2,      /* inconsistent sizes: num_reqs < 0, max_tokens < 0, Hq % Hkv != 0, ... */
  UP_ERR_PARAM = -3,      /* G, A, n, p or head_dim out of the supported range */
  UP_ERR_WORKSPACE = -4,  /* workspace smaller than the matching *_workspace_bytes() */
  UP_ERR_ALIGN = -5,      /* pointer or stride not 16-byte aligned where required */
  UP_ERR_HIP = -6         /* a HIP launch failed */
} up_status;

/* up_select_params.flags */
#define UP_SCORES_IN 1u   /* skip scoring; select from caller-provided block scores */

typedef struct up_select_params {
  int32_t num_heads_q;    /* Hq >= 1 */
  int32_t num_heads_kv;   /* Hkv >= 1, Hq % Hkv == 0; query head h reads KV head floor(h*Hkv/Hq) */
  int32_t head_dim;       /* d in {64, 128, 256} (any value >= 1 with UP_SCORES_IN) */
  int32_t block_size;     /* G >= 1; a multiple of 32 when scoring (UniPrefill Sec. 3.2) */
  int32_t num_sink;       /* A >= 0: the first A tokens of each request are always kept (Sec. 3.3) */
  int32_t window;         /* n >= 1: the last n tokens score the rest and are always kept (Eq. 3) */
  double top_p;           /* 0 < p <= 1 (Eq. 5) */
  float softmax_scale;    /* <= 0 selects 1/sqrt(d) (Eq. 2) */
  uint32_t flags;         /* UP_SCORES_IN or 0 */
} up_select_params;

/* Upper bound on sum_r ceil(N_r / G) for any batch of num_reqs requests and at
 * most max_tokens tokens: floor(max_tokens / G) + num_reqs.  Size block_scores
 * and keep_block with it.  Returns -1 for invalid arguments. */
int64_t up_max_blocks(int32_t block_size, int32_t num_reqs, int64_t max_tokens);

/* Bytes of workspace up_select_blocks needs for these sizes (0 if invalid). */
size_t up_select_workspace_bytes(const up_select_params* prm, int32_t num_reqs, int64_t max_tokens);

/*
 * up_select_blocks - importance estimation and top-p block selection for one
 * full-attention layer (UniPrefill Sec. 3.2-3.3, Eq. 2-5; the pipeline of
 * Sec. 3.5 Eq. 13 with the packed keys of Eq. 14 and the expansion step).
 *
 * For each request r (N_r tokens starting at s_r, n_eff = min(n, N_r)):
 *   1. for every query head h and window row t < n_eff, the scaled logits of
 *      query s_r+N_r-n_eff+t against the request's keys, causally masked;
 *   2. their full-sequence softmax, summed over h and t and reduced to block
 *      scores b_g = sum_{i in block g} o_i / (G * n_eff), blocks anchored at s_r
 *      (the last one may be partial and is still divided by G);
 *   3. top-p over the blocks: blocks ranked by the packed key
 *      (phi(b_g) << 32) | g, descending; the cumulative sum of Eq. 5 is taken on
 *      exact integers floor(b_g * 2^shift), shift = 52 - ceil(log2 nb) - e with
 *      e the binary exponent of the largest positive score; the kept set is the
 *      shortest prefix (at least one block) whose integer mass reaches
 *      p * total (one float64 multiply).  Scores that are not positive and
 *      finite carry no mass;
 *   4. the token mask: M_i = keep[block of i] or i < A or i >= N_r - n.
 *
 * q        bf16 [T, Hq, d] rows, token stride q_row_stride ELEMENTS (>= Hq*d,
 *          multiple of 8); only each request's last n_eff rows are read.
 *          16-byte aligned.  Unused (may be NULL) with UP_SCORES_IN.
 * k        bf16 [T, Hkv, d], token stride k_row_stride elements, same rules.
 * cu_seqlens     int32 [num_reqs + 1].
 * scores_in      with UP_SCORES_IN: fp32 block scores [sum_r nb_r], request-major.
 * block_scores   out fp32 [sum_r nb_r] (may be NULL with UP_SCORES_IN).
 * block_offsets  out int32 [num_reqs + 1]: prefix sums of nb_r = ceil(N_r/G).
 * keep_block     out uint8 [sum_r nb_r], 1 = block kept by top-p (before forcing); may be NULL.
 * keep_mask      out uint8 [max_tokens]: M for tokens < cu_seqlens[num_reqs].
 * kept_per_req   out int32 [num_reqs]: number of set mask entries per request.
 * workspace      device scratch of at least up_select_workspace_bytes(); 256-byte aligned.
 */
up_status up_select_blocks(const up_select_params* prm,
                           const void* q, int64_t q_row_stride,
                           const void* k, int64_t k_row_stride,
                           const int32_t* cu_seqlens, int32_t num_reqs, int64_t max_tokens,
                           const float* scores_in,
                           float* block_scores, int32_t* block_offsets,
                           uint8_t* keep_block, uint8_t* keep_mask, int32_t* kept_per_req,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace up_compact needs (0 if invalid). */
size_t up_compact_workspace_bytes(int32_t num_reqs, int64_t max_tokens);

/*
 * up_compact - keep the rows of set mask entries, in order (the compacted
 * token stream that later sublayers run on: UniPrefill Sec. 3.4 Eq. 7 and
 * Sec. 3.5 "vLLM scheduler integration").
 *
 * For the kept tokens i_0 < i_1 < ... of the packed stream (mask bytes are
 * tested for nonzero):
 *   dst[b] row k          = src[b] row i_k, for every buffer b;
 *   index_out[k]          = index_in ? index_in[i_k] : i_k;
 *   cu_seqlens_out[r]     = number of kept tokens before cu_seqlens[r]
 *                           (the patched query_start_loc; its last entry is
 *                           num_actual_tokens).
 *
 * keep_mask      uint8 [max_tokens].
 * num_buffers    >= 0 row buffers; src, dst and row_bytes are HOST arrays of
 *                num_buffers entries (device pointers / byte counts).  Each
 *                row_bytes[b] is a positive multiple of 4; rows use the
 *                vectorised path when row_bytes and both pointers are 16-byte
 *                aligned.  src[b] holds cu_seqlens[num_reqs] rows; dst[b] room
 *                for as many.  src and dst must not overlap.
 * index_in       optional int32 [max_tokens] (NULL = identity): the original
 *                position of each current row, so that repeated drops compose.
 * index_out      out int32 [max_tokens]; entries past the kept count are untouched.
 * cu_seqlens_out out int32 [num_reqs + 1].
 */
up_status up_compact(const uint8_t* keep_mask, const int32_t* cu_seqlens, int32_t num_reqs,
                     int64_t max_tokens, int32_t num_buffers,
                     const void* const* src, void* const* dst, const int64_t* row_bytes,
                     const int32_t* index_in, int32_t* index_out, int32_t* cu_seqlens_out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * up_compact_noalloc - up_compact for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, work, results and validation as
 * up_compact, without the workspace: the library uses a scratch array of
 * 16 MiB in device memory that exists once per GPU from the first call on that
 * GPU (the GPU of `stream`) until the process ends.  The call allocates
 * nothing; it accepts streams of at most UP_COMPACT_NOALLOC_MAX_TOKENS tokens
 * (max_tokens above it returns UP_ERR_WORKSPACE before any work) and returns
 * UP_ERR_HIP if the scratch cannot be located on that GPU.  Every call on one
 * GPU shares its scratch: calls whose work overlaps on the same GPU (two
 * streams, or two host threads, without ordering between them) race and give
 * undefined results; calls ordered on one stream are safe.  The scratch keeps
 * the last call's contents, and nothing in it needs to start at zero.
 */
#define UP_COMPACT_NOALLOC_MAX_TOKENS 4000000
up_status up_compact_noalloc(const uint8_t* keep_mask, const int32_t* cu_seqlens, int32_t num_reqs,
                             int64_t max_tokens, int32_t num_buffers,
                             const void* const* src, void* const* dst, const int64_t* row_bytes,
                             const int32_t* index_in, int32_t* index_out, int32_t* cu_seqlens_out,
                             hipStream_t stream);

/*
 * up_scatter_back - carry-forward of UniPrefill Sec. 3.4 Eq. 8: for
 * k < cu_seqlens_out[num_reqs], full row index_map[k] = compacted row k;
 * every other row of `full` keeps its value.  Entries of index_map outside
 * [0, full_rows) are skipped.  index_map must not repeat an index (as
 * up_compact's output never does).
 *
 * compacted      [>= count rows] of row_bytes each (row_bytes a positive multiple of 4).
 * index_map      int32 [max_tokens], e.g. up_compact's index_out.
 * cu_seqlens_out int32 [num_reqs + 1]; only its last entry (the count) is read.
 * full           [full_rows rows].
 */
up_status up_scatter_back(const void* compacted, int64_t row_bytes, const int32_t* index_map,
                          const int32_t* cu_seqlens_out, int32_t num_reqs, int64_t max_tokens,
                          void* full, int64_t full_rows, hipStream_t stream);

/*
 * up_update_metadata - metadata patch after a drop at layer `layer`
 * (UniPrefill Sec. 3.5, "vLLM scheduler integration", and Eq. 17).
 *
 * For every request r, with N_r = cu_old[r+1]-cu_old[r] and
 * K_r = cu_new[r+1]-cu_new[r] (both clamped to >= 0):
 *   seq_lens[r]         -= N_r - K_r            (prior context is kept);
 *   num_actual_tokens[0] = cu_new[num_reqs];
 *   drop history: entry drop_count[r] of row r (row stride max_drops) gets
 *     drop_layer = layer, drop_len = the new seq_lens[r], if drop_count[r] <
 *     max_drops; drop_count[r] is incremented in any case, so a count above
 *     max_drops reports lost entries;
 *   seqused_base[l*num_reqs + r] = the new seq_lens[r] for layer < l < num_layers.
 * Decode-time seqused of Eq. 17 is seqused_base[l][r] + (kv_len_r - orig_len_r).
 * Drops must be recorded in increasing layer order; the caller initialises
 * seqused_base[*][r] to the original seq_lens and drop_count to 0.
 * seqused_base may be NULL (then num_layers is ignored).
 */
up_status up_update_metadata(int32_t layer, int32_t num_layers, int32_t num_reqs,
                             const int32_t* cu_seqlens_old, const int32_t* cu_seqlens_new,
                             int32_t* seq_lens, int32_t* num_actual_tokens,
                             int32_t* drop_count, int32_t* drop_layer, int32_t* drop_len,
                             int32_t max_drops, int32_t* seqused_base, hipStream_t stream);

/*
 * up_slot_mapping - per-layer KV cache slots of the (compacted) token stream,
 * UniPrefill Sec. 3.5 ("vLLM scheduler integration"), Eq. 16:
 *   slot_k = block_table[r][p_k / B] * B + p_k % B
 * for stream row k of request r, where p_k is the row's logical position.
 * A layer after a drop caches only the retained tokens, densely after the
 * tokens the request already had cached, so
 *   p_k = seq_lens[r] - kept_r + (k - cu_seqlens[r]),  kept_r = cu_seqlens[r+1] - cu_seqlens[r]
 * with seq_lens the lengths patched by up_update_metadata (p_k = rank among
 * the retained tokens for a fresh prefill).  Each layer passes its own block
 * table (global and sliding-window layers may differ).
 *
 * block_table   int32 [num_reqs][block_table_stride]; columns
 *               [0, max_blocks_per_req) hold physical block ids (negative:
 *               no block).  May be NULL when max_blocks_per_req is 0.
 * kv_block_size B >= 1 tokens per physical block.
 * cu_seqlens    int32 [num_reqs + 1], nondecreasing stream offsets (e.g. up_compact's cu_seqlens_out).
 * seq_lens      int32 [num_reqs].
 * slot_mapping  out int64 [max_tokens]; -1 for rows past cu_seqlens[num_reqs],
 *               for positions p < 0 or p / B >= max_blocks_per_req, and for
 *               negative table entries.
 * Errors: UP_ERR_NULL, UP_ERR_SHAPE (negative sizes, stride < width,
 * max_tokens > INT32_MAX), UP_ERR_PARAM (B < 1), UP_ERR_ALIGN (int32 arrays
 * 4-byte, slot_mapping 8-byte aligned), UP_ERR_HIP.
 */
up_status up_slot_mapping(const int32_t* block_table, int64_t block_table_stride,
                          int32_t max_blocks_per_req, int32_t kv_block_size,
                          const int32_t* cu_seqlens, const int32_t* seq_lens, int32_t num_reqs,
                          int64_t max_tokens, int64_t* slot_mapping, hipStream_t stream);

/*
 * up_write_kv_cache - store the retained rows' keys and values in the paged
 * cache at the slots of Eq. 16 (UniPrefill Sec. 3.5, the physical slot
 * mapping that lets PagedAttention read the compacted cache unchanged).
 *
 * For k < min(cu_seqlens[num_reqs], max_tokens) with 0 <= slot_mapping[k] < cache_slots:
 *   key_cache row slot_mapping[k]   = key row k    (row_bytes bytes)
 *   value_cache row slot_mapping[k] = value row k
 * Rows without a slot are skipped; every other cache row keeps its value.
 * Slots must not repeat (up_slot_mapping's never do for disjoint tables).
 *
 * key, value            rows of row_bytes bytes at strides key_row_stride /
 *                       value_row_stride bytes (>= row_bytes; e.g. a view
 *                       into a fused QKV projection).  value and value_cache
 *                       are both NULL for a key-only cache.
 * key_cache, value_cache slot-major caches [cache_slots][row_bytes], i.e. the
 *                       [num_blocks][B][num_heads_kv][head_dim] layout.
 * row_bytes             positive multiple of 4 (16-byte aligned rows and
 *                       strides take the vector path).
 * Errors: UP_ERR_NULL, UP_ERR_SHAPE, UP_ERR_PARAM, UP_ERR_ALIGN, UP_ERR_HIP.
 */
up_status up_write_kv_cache(const void* key, int64_t key_row_stride, const void* value,
                            int64_t value_row_stride, int64_t row_bytes, const int64_t* slot_mapping,
                            const int32_t* cu_seqlens, int32_t num_reqs, int64_t max_tokens,
                            void* key_cache, void* value_cache, int64_t cache_slots,
                            hipStream_t stream);

/*
 * Downstream sublayer on the retained rows: the gated FFN of the LLaMA family,
 * y = (silu(x Wg^T) * (x Wu^T)) Wd^T row by row.  UniPrefill Sec. 3.4 Eq. 7:
 * after a drop every later sublayer (FFN included) maps only the retained
 * rows, which is the saving Eq. 9-10 counts; calling it on the compacted
 * stream instead of the full one is that saving.
 *
 * up_ffn_workspace_bytes  device workspace up_ffn_forward needs for `rows`
 *                 rows of hidden width D and intermediate width F (both
 *                 positive multiples of 8, at most 2^24): the activation h,
 *                 rows x F bf16, rounded up to 256 bytes.  0 if invalid.
 * up_ffn_forward  x bf16 [rows][D]; w_gate_up bf16 [2F][D] (gate rows, then up
 *                 rows: the [out][in] layout of a linear layer); w_down bf16
 *                 [D][F]; y bf16 out [rows][D].  Products of bf16 inputs
 *                 accumulate in fp32; silu(gate) * up is formed in fp32 from
 *                 the two fp32 accumulators and rounded once to bf16 (h, kept
 *                 in the workspace); y is rounded to bf16.  rows is a host
 *                 value (e.g. the kept count read back once the compaction has
 *                 run); rows == 0 does nothing.  All pointers 16-byte aligned;
 *                 y must not overlap x or the workspace.  Like every other
 *                 call it only enqueues work (no allocation, no handle, no
 *                 state).  Errors: UP_ERR_PARAM (widths), UP_ERR_NULL,
 *                 UP_ERR_SHAPE (rows < 0, or a grid past 32 bits),
 *                 UP_ERR_ALIGN, UP_ERR_WORKSPACE, UP_ERR_HIP.
 */
size_t up_ffn_workspace_bytes(int32_t hidden, int32_t intermediate, int64_t rows);
up_status up_ffn_forward(int32_t hidden, int32_t intermediate, const void* x, int64_t rows,
                         const void* w_gate_up, const void* w_down, void* y, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* Static description of a status code. */
const char* up_status_string(up_status status);

#ifdef __cplusplus
}
#endif

#endif /* UNIPREFILL_H */
