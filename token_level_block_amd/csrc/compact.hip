// Compaction of the packed token stream and the carry-forward scatter
// (UniPrefill Sec. 3.4 Eq. 7-8; Sec. 3.5, the compacted stream that the
// patched query_start_loc describes).
//
//   rank_direct (streams of at most 131072 tokens): one workgroup per
//            4096-token tile counts the kept tokens before its tile from the
//            mask itself, ranks its own, and writes the index map, the stream
//            position of every kept row and the new request offsets (of the
//            clamped, non-decreasing cu_seqlens) that fall in its tile;
//   count + rank (longer streams): the same in two launches, the first
//            counting each 4096-token tile, the second (256-token tiles)
//            adding up the counts before its tile;
//   copy   : every buffer's kept rows in one launch; wide rows as one flat
//            stream of 16-byte units in chip-wide order (the same kernel moves
//            the rows back for the Eq. 8 scatter).
// No atomics and no inter-workgroup waiting: every result is deterministic.
#include "common.h"
#include "copy_plan.h"

static_assert(up::kMaxCompactBuffers == up::kMaxCopyBuffers, "one copy launch plans every compaction buffer");

namespace up {

constexpr int kCountThreads = kCountTile / 16;   // 16 mask bytes per thread
constexpr int kGatherThreads = kGatherTile;      // one token per thread

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// number of nonzero bytes in a 32-bit word
__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
  const uint32_t hi = ((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w;   // 0x80 set in each nonzero byte
  return __popc(hi & 0x80808080u);
}

__device__ __forceinline__ int count_piece(const uint8_t* mask, int64_t pos, int64_t limit) {
  // nonzero bytes among mask[pos .. min(pos+16, limit))
  if (pos + 16 <= limit) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(mask + pos);
    return nonzero_bytes(v[0]) + nonzero_bytes(v[1]) + nonzero_bytes(v[2]) + nonzero_bytes(v[3]);
  }
  int c = 0;
  for (int64_t i = pos; i < limit; ++i) c += mask[i] != 0;
  return c;
}

__global__ __launch_bounds__(kCountThreads) void count_kernel(const uint8_t* __restrict__ mask,
                                                              int64_t max_tokens,
                                                              int32_t* __restrict__ tile_count) {
  __shared__ int32_t red[kCountThreads / kWave];
  const int64_t pos = (int64_t)blockIdx.x * kCountTile + threadIdx.x * 16;
  int c = pos < max_tokens ? count_piece(mask, pos, max_tokens) : 0;
  for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int w = 0; w < kCountThreads / kWave; ++w) t += red[w];
    tile_count[blockIdx.x] = t;
  }
}

// clamp(cu[e]) into [0, cap]; the running maximum of these is the clamped,
// non-decreasing offset array every kernel here works with
__device__ __forceinline__ int32_t clamp_cu(int32_t v, int32_t cap) { return max(0, min(v, cap)); }

__global__ __launch_bounds__(kGatherThreads) void rank_kernel(CompactArgs a) {
  __shared__ int32_t red[kGatherThreads / kWave];
  __shared__ int32_t wsum[kGatherThreads / kWave];
  __shared__ int32_t excl[kGatherThreads + 1];
  __shared__ int32_t s_T, s_prefix, s_carry;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int32_t cap = (int32_t)(a.max_tokens < 0x7fffffff ? a.max_tokens : 0x7fffffff);
  const int R = a.R;

  // stream length T = the last clamped offset = the largest clamped entry
  int32_t m = 0;
  for (int e = tid; e <= R; e += kGatherThreads) m = max(m, clamp_cu(a.cu_in[e], cap));
  for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o));
  if (lane == 0) red[wid] = m;
  __syncthreads();
  if (tid == 0) {
    int32_t t = 0;
    for (int w = 0; w < kGatherThreads / kWave; ++w) t = max(t, red[w]);
    s_T = t;
  }
  __syncthreads();
  const int32_t T = s_T;
  const int64_t start = (int64_t)blockIdx.x * kGatherTile;
  if (T == 0) {
    // an empty stream has no tile to report the request offsets
    if (blockIdx.x == 0)
      for (int e = tid; e <= R; e += kGatherThreads) a.cu_out[e] = 0;
    return;
  }
  if (start >= T) return;
  const int64_t end = min<int64_t>(start + kGatherTile, T);

  // kept tokens before this tile: whole count tiles before it, plus the pieces
  // of its own count tile that precede it
  const int64_t ct = start / kCountTile;
  const int64_t cstart = ct * kCountTile;
  int c = 0;
  for (int64_t t = tid; t < ct; t += kGatherThreads) c += a.tile_count[t];
  {
    const int64_t pos = cstart + (int64_t)tid * 16;
    if (pos < start) c += count_piece(a.mask, pos, start);
  }
  for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o);
  if (lane == 0) red[wid] = c;
  __syncthreads();
  if (tid == 0) {
    int t = 0;
    for (int w = 0; w < kGatherThreads / kWave; ++w) t += red[w];
    s_prefix = t;
    s_carry = 0;
  }

  const int64_t i = start + tid;
  const bool kept = (i < end) && a.mask[i] != 0;
  const unsigned long long bal = __ballot(kept);
  const int below = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wid] = __popcll(bal);
  __syncthreads();
  int wpre = 0;
  for (int w = 0; w < wid; ++w) wpre += wsum[w];
  const int local = wpre + below;
  excl[tid] = local;
  if (tid == kGatherThreads - 1) excl[kGatherThreads] = local + (kept ? 1 : 0);
  __syncthreads();
  const int32_t prefix = s_prefix;

  if (kept) {
    a.index_out[prefix + local] = a.index_in ? a.index_in[i] : (int32_t)i;
    a.src_pos[prefix + local] = (int32_t)i;
  }
  // new request offsets that fall inside this tile (the last tile also owns
  // position T): the clamped running maximum of cu, a chunk at a time
  for (int base = 0; base <= R; base += kGatherThreads) {
    const int e = base + tid;
    const int32_t v = (e <= R) ? clamp_cu(a.cu_in[e], cap) : 0;
    const int32_t p = max(block_inclusive_scan<true>(v, red), s_carry);
    if (e <= R && p >= start && (p < end || (p == T && end == T))) a.cu_out[e] = prefix + excl[p - start];
    __syncthreads();
    if (tid == kGatherThreads - 1) s_carry = p;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Streams of at most kDirectRankMax tokens: one launch instead of count + rank.
// Workgroup x ranks the tokens [4096 x, 4096 x + 4096) and finds the kept
// tokens before its tile by reading the mask bytes before it (at most 128 KB:
// one round of eight 16-byte loads per thread), so it needs no count pass.
// ---------------------------------------------------------------------------
constexpr int kDirectThreads = 1024;
constexpr int kDirectTile = 4 * kDirectThreads;   // four tokens per thread

__global__ __launch_bounds__(kDirectThreads) void rank_direct_kernel(CompactArgs a) {
  __shared__ int32_t red_c[kDirectThreads / kWave], red_k[kDirectThreads / kWave];
  __shared__ int32_t scan[kDirectThreads / kWave];
  __shared__ int32_t excl[kDirectTile + 1];   // kept tokens of the tile before each position
  __shared__ int32_t s_carry;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int32_t cap = (int32_t)(a.max_tokens < 0x7fffffff ? a.max_tokens : 0x7fffffff);
  const int R = a.R;

  // stream length T = the largest clamped offset: every wave finds it itself
  // for fewer than 1024 requests, else the workgroup shares the reads
  int32_t T = 0;
  if (R < kDirectThreads) {
    for (int e = lane; e <= R; e += kWave) T = max(T, clamp_cu(a.cu_in[e], cap));
    for (int o = 32; o >= 1; o >>= 1) T = max(T, __shfl_xor(T, o));
  } else {
    for (int e = tid; e <= R; e += kDirectThreads) T = max(T, clamp_cu(a.cu_in[e], cap));
    for (int o = 32; o >= 1; o >>= 1) T = max(T, __shfl_xor(T, o));
    if (lane == 0) scan[wid] = T;
    __syncthreads();
    for (int w = 0; w < kDirectThreads / kWave; ++w) T = max(T, scan[w]);
    __syncthreads();   // scan is reused below
  }
  const int64_t start = (int64_t)blockIdx.x * kDirectTile;
  if (T == 0) {
    if (blockIdx.x == 0)
      for (int e = tid; e <= R; e += kDirectThreads) a.cu_out[e] = 0;
    return;
  }
  if (start >= T) return;
  const int64_t end = min<int64_t>(start + kDirectTile, T);

  // kept tokens before the tile (start is a multiple of 16: whole pieces)
  int c = 0;
  {
    constexpr int kUnroll = 8;
    for (int64_t base = (int64_t)tid * 16; base < start; base += (int64_t)kDirectThreads * 16 * kUnroll) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t pos = base + (int64_t)u * kDirectThreads * 16;
        v[u] = pos < start ? *reinterpret_cast<const u32x4*>(a.mask + pos) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        c += nonzero_bytes(v[u][0]) + nonzero_bytes(v[u][1]) + nonzero_bytes(v[u][2]) + nonzero_bytes(v[u][3]);
    }
  }

  // this thread's four tokens
  const int64_t i0 = start + 4 * (int64_t)tid;
  uint32_t kb = 0;   // bit j: token i0 + j is kept
  if (i0 + 4 <= end) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(a.mask + i0);
#pragma unroll
    for (int j = 0; j < 4; ++j) kb |= (((w >> (8 * j)) & 0xFFu) != 0u ? 1u : 0u) << j;
  } else {
    for (int j = 0; j < 4; ++j)
      if (i0 + j < end && a.mask[i0 + j] != 0) kb |= 1u << j;
  }
  const int nk = __popc(kb);

  // one exchange between the waves: each wave's count before the tile and its
  // kept tokens in the tile
  int nk_incl = nk;
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(nk_incl, o);
    if (lane >= o) nk_incl += x;
  }
  for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o);
  if (lane == 63) {
    red_c[wid] = c;
    red_k[wid] = nk_incl;
  }
  __syncthreads();
  int32_t prefix = 0, wave_off = 0;
  for (int w = 0; w < kDirectThreads / kWave; ++w) {
    prefix += red_c[w];
    if (w < wid) wave_off += red_k[w];
  }
  int run = wave_off + nk_incl - nk;   // kept tokens of the tile before this thread's first
  {
    int k = prefix + run;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      excl[4 * tid + j] = run;
      if ((kb >> j) & 1u) {
        const int64_t i = i0 + j;
        a.index_out[k] = a.index_in ? a.index_in[i] : (int32_t)i;
        a.src_pos[k] = (int32_t)i;
        ++k;
        ++run;
      }
    }
  }
  if (tid == kDirectThreads - 1) excl[kDirectTile] = run;
  __syncthreads();

  // new request offsets that fall inside this tile (the last tile also owns T):
  // the clamped running maximum of cu, by one wave when it covers every entry
  if (R < kWave) {
    if (wid == 0) {
      int32_t p = lane <= R ? clamp_cu(a.cu_in[lane], cap) : 0;
      for (int o = 1; o < 64; o <<= 1) {
        const int32_t x = __shfl_up(p, o);
        if (lane >= o) p = max(p, x);
      }
      if (lane <= R && p >= start && (p < end || (p == T && end == T))) a.cu_out[lane] = prefix + excl[p - start];
    }
    return;
  }
  if (tid == 0) s_carry = 0;
  for (int base = 0; base <= R; base += kDirectThreads) {
    const int e = base + tid;
    const int32_t v = (e <= R) ? clamp_cu(a.cu_in[e], cap) : 0;
    const int32_t p = max(block_inclusive_scan<true>(v, scan), s_carry);
    if (e <= R && p >= start && (p < end || (p == T && end == T))) a.cu_out[e] = prefix + excl[p - start];
    __syncthreads();
    if (tid == kDirectThreads - 1) s_carry = p;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Row copy over the kept rows k < count:  kGather: dst row k <- src row map[k]
//                                         scatter: dst row map[k] <- src row k
// One launch moves every buffer; buffer b owns the workgroups
// [plan.wg_begin[b], plan.wg_begin[b+1]) (copy_plan.h).
// Flat buffers (16-byte rows wider than 32 bytes): the kept rows form one
// stream of 16-byte units, unit i = (row i / units, piece i % units); a step
// of the buffer's workgroups covers 256 consecutive units per workgroup and
// consecutive workgroups take consecutive units, so the chip streams one
// window of memory at a time (nontemporal: the rows are touched once).  This
// ordering copied 8 KiB rows at ~6.1-6.3 TB/s against ~5.6 TB/s for waves that
// each stream their own run of rows.  Narrow rows (<= 32 bytes): one row per
// thread; other 4-byte-multiple rows: one row per wave.
// ---------------------------------------------------------------------------
constexpr int kCopyWaves = kCopyThreads / kWave;

template <bool kGather>
__device__ __forceinline__ void row_ends(const int32_t* __restrict__ map, int64_t k, int64_t& s, int64_t& d) {
  s = kGather ? (int64_t)map[k] : k;
  d = kGather ? k : (int64_t)map[k];
}

// flat copy of `total` 16-byte units: a step of the nwg workgroups covers
// nwg * 256 consecutive units, one per thread
template <bool kGather>
__device__ __forceinline__ void copy_flat(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                          const int32_t* __restrict__ map, uint32_t total, uint32_t units,
                                          FastDiv div, int wg, int nwg, int64_t dst_rows) {
  const u32x4* __restrict__ s16 = reinterpret_cast<const u32x4*>(src);
  u32x4* __restrict__ d16 = reinterpret_cast<u32x4*>(dst);
  // 64-bit position: a 32-bit one could wrap past total near 2^32 and never end
  const uint64_t step = (uint64_t)nwg * kCopyThreads;
  for (uint64_t i = (uint64_t)wg * kCopyThreads + threadIdx.x; i < total; i += step) {
    const uint32_t k = fastdiv((uint32_t)i, div);
    const uint32_t j = (uint32_t)i - k * units;
    int64_t sr, dr;
    row_ends<kGather>(map, k, sr, dr);
    if (dr < 0 || dr >= dst_rows) continue;
    const u32x4 v = __builtin_nontemporal_load(s16 + sr * units + j);
    __builtin_nontemporal_store(v, d16 + dr * units + j);
  }
}

template <bool kGather>
__global__ __launch_bounds__(kCopyThreads) void copy_rows_kernel(RowBuffers bufs, CopyPlan plan,
                                                                 const int32_t* __restrict__ map,
                                                                 const int32_t* __restrict__ count_ptr,
                                                                 int64_t max_rows, int64_t dst_rows) {
  int b = 0;
  while (b + 1 < bufs.nbuf && (int)blockIdx.x >= plan.wg_begin[b + 1]) ++b;
  const int wg = (int)blockIdx.x - plan.wg_begin[b];
  const int nwg = plan.wg_begin[b + 1] - plan.wg_begin[b];
  const uint8_t* __restrict__ src = bufs.src[b];
  uint8_t* __restrict__ dst = bufs.dst[b];
  const int64_t rb = bufs.row_bytes[b];
  const int64_t count = min<int64_t>(*count_ptr, max_rows);
  if (plan.flat[b]) {
    const uint32_t total = (uint32_t)count * plan.units[b];   // < 2^32: checked when planned
    copy_flat<kGather>(src, dst, map, total, plan.units[b], plan.div[b], wg, nwg, dst_rows);
  } else if (rb <= kCopyNarrowRow) {
    // narrow rows (positions, indices): one thread per row
    const int units = (int)(rb >> 2);
    for (int64_t k = (int64_t)wg * kCopyThreads + threadIdx.x; k < count; k += (int64_t)nwg * kCopyThreads) {
      int64_t sr, dr;
      row_ends<kGather>(map, k, sr, dr);
      if (dr < 0 || dr >= dst_rows) continue;
      const uint32_t* sp = reinterpret_cast<const uint32_t*>(src + sr * rb);
      uint32_t* dp = reinterpret_cast<uint32_t*>(dst + dr * rb);
      for (int u = 0; u < units; ++u) dp[u] = sp[u];
    }
  } else {
    // other rows of 4-byte multiples: one row per wave
    const int lane = threadIdx.x & 63;
    const int units = (int)(rb >> 2);
    for (int64_t k = (int64_t)wg * kCopyWaves + (threadIdx.x >> 6); k < count; k += (int64_t)nwg * kCopyWaves) {
      int64_t sr, dr;
      row_ends<kGather>(map, k, sr, dr);
      if (dr < 0 || dr >= dst_rows) continue;
      const uint32_t* sp = reinterpret_cast<const uint32_t*>(src + sr * rb);
      uint32_t* dp = reinterpret_cast<uint32_t*>(dst + dr * rb);
      for (int u = lane; u < units; u += kWave) dp[u] = sp[u];
    }
  }
}

static hipError_t launch_copy(bool gather, const RowBuffers& bufs, const int32_t* map, const int32_t* count_ptr,
                              int64_t max_rows, int64_t dst_rows, hipStream_t s) {
  if (bufs.nbuf <= 0 || max_rows <= 0) return hipSuccess;
  CopyPlan plan;
  if (!make_copy_plan(bufs.nbuf, bufs.row_bytes, bufs.vec16, max_rows, &plan)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)plan.wg_begin[bufs.nbuf]), block(kCopyThreads);
  if (gather)
    hipLaunchKernelGGL((copy_rows_kernel<true>), grid, block, 0, s, bufs, plan, map, count_ptr, max_rows, dst_rows);
  else
    hipLaunchKernelGGL((copy_rows_kernel<false>), grid, block, 0, s, bufs, plan, map, count_ptr, max_rows,
                       dst_rows);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  if (a.max_tokens <= kDirectRankMax) {
    const int64_t ntiles = (a.max_tokens + kDirectTile - 1) / kDirectTile;
    hipLaunchKernelGGL(rank_direct_kernel, dim3((unsigned)(ntiles > 0 ? ntiles : 1)), dim3(kDirectThreads), 0, s,
                       a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_copy(true, a.bufs, a.src_pos, a.cu_out + a.R, a.max_tokens, a.max_tokens, s);
  }
  if (a.num_count_tiles > 0) {
    hipLaunchKernelGGL(count_kernel, dim3((unsigned)a.num_count_tiles), dim3(kCountThreads), 0, s,
                       a.mask, a.max_tokens, a.tile_count);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t ntiles = (a.max_tokens + kGatherTile - 1) / kGatherTile;
  hipLaunchKernelGGL(rank_kernel, dim3((unsigned)(ntiles > 0 ? ntiles : 1)), dim3(kGatherThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_copy(true, a.bufs, a.src_pos, a.cu_out + a.R, a.max_tokens, a.max_tokens, s);
}

// ---------------------------------------------------------------------------
// Eq. 8 carry-forward: full[index_map[k]] = compacted[k], k < count
// ---------------------------------------------------------------------------
hipError_t launch_scatter(const void* compacted, int64_t row_bytes, const int32_t* index_map,
                          const int32_t* count_ptr, int64_t max_tokens, void* full,
                          int64_t full_rows, hipStream_t s) {
  if (max_tokens <= 0) return hipSuccess;
  RowBuffers one{};
  one.nbuf = 1;
  one.src[0] = static_cast<const uint8_t*>(compacted);
  one.dst[0] = static_cast<uint8_t*>(full);
  one.row_bytes[0] = row_bytes;
  one.vec16[0] = (row_bytes % 16 == 0) && ((uintptr_t)compacted % 16 == 0) && ((uintptr_t)full % 16 == 0);
  return launch_copy(false, one, index_map, count_ptr, max_tokens, full_rows, s);
}

}  // namespace up
