// Per-layer KV cache slots of the compacted token stream and the paged-cache
// write (UniPrefill Sec. 3.5, "vLLM scheduler integration", Eq. 16).
//
//   slot  : one thread per stream row.  Row k of request r is the request's
//           (k - cu[r])-th retained token; its logical position is
//           p = seq_lens[r] - kept_r + (k - cu[r]) (the layer caches retained
//           tokens densely after what the request already had cached), and
//           slot = block_table[r][p / B] * B + p % B.  A position outside
//           the table or a negative table entry gives -1, as do the padding
//           rows past cu[R].
//   write : waves dealt round-robin over the rows; a wave copies its row's
//           key (and value) to cache row `slot` with 16-byte accesses, the
//           loads in flight before the stores (two rows per trip for rows of
//           at most 4 KiB).
#include "common.h"

namespace up {

constexpr int kSlotThreads = 256;
constexpr int kKvThreads = 256;
constexpr int kKvWaves = kKvThreads / kWave;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kSlotThreads) void slot_kernel(SlotArgs a) {
  const int64_t k = (int64_t)blockIdx.x * kSlotThreads + threadIdx.x;
  if (k >= a.max_tokens) return;
  int64_t slot = -1;
  const int64_t T = a.R > 0 ? (int64_t)a.cu[a.R] : 0;
  if (k < T) {
    const int r = find_owner(a.cu, a.R, k);
    const int64_t first = a.cu[r];
    const int64_t kept = (int64_t)a.cu[r + 1] - first;
    const int64_t p = (int64_t)a.seq_lens[r] - kept + (k - first);
    if (p >= 0 && k >= first) {
      const int64_t col = p / a.B;
      if (col < a.width) {
        const int32_t phys = a.table[(int64_t)r * a.table_stride + col];
        if (phys >= 0) slot = (int64_t)phys * a.B + (p - col * a.B);
      }
    }
  }
  a.slots[k] = slot;
}

template <bool kVec>
__global__ __launch_bounds__(kKvThreads) void kv_write_kernel(KvWriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * kKvWaves + (threadIdx.x >> 6);
  const int64_t W = (int64_t)gridDim.x * kKvWaves;
  const int64_t T = a.R > 0 ? (int64_t)a.cu[a.R] : 0;
  const int64_t count = T < 0 ? 0 : (T < a.max_tokens ? T : a.max_tokens);
  const bool has_v = a.value != nullptr;
  for (int64_t k = gw; k < count; k += W) {
    const int64_t s = a.slots[k];
    if (s < 0 || s >= a.cache_slots) continue;
    const uint8_t* ksrc = a.key + k * a.key_stride;
    const uint8_t* vsrc = has_v ? a.value + k * a.value_stride : nullptr;
    uint8_t* kdst = a.key_cache + s * a.row_bytes;
    uint8_t* vdst = has_v ? a.value_cache + s * a.row_bytes : nullptr;
    if (kVec) {
      const u32x4* ks = reinterpret_cast<const u32x4*>(ksrc);
      const u32x4* vs = reinterpret_cast<const u32x4*>(vsrc);
      u32x4* kd = reinterpret_cast<u32x4*>(kdst);
      u32x4* vd = reinterpret_cast<u32x4*>(vdst);
      const int units = (int)(a.row_bytes >> 4);
      int u = lane;
      for (; u + 3 * kWave < units; u += 4 * kWave) {
        u32x4 kv[4], vv[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) kv[x] = __builtin_nontemporal_load(ks + u + x * kWave);
        if (has_v) {
#pragma unroll
          for (int x = 0; x < 4; ++x) vv[x] = __builtin_nontemporal_load(vs + u + x * kWave);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) kd[u + x * kWave] = kv[x];
        if (has_v) {
#pragma unroll
          for (int x = 0; x < 4; ++x) vd[u + x * kWave] = vv[x];
        }
      }
      for (; u < units; u += kWave) {
        const u32x4 kv = __builtin_nontemporal_load(ks + u);
        if (has_v) {
          const u32x4 vv = __builtin_nontemporal_load(vs + u);
          vd[u] = vv;
        }
        kd[u] = kv;
      }
    } else {
      const uint32_t* ks = reinterpret_cast<const uint32_t*>(ksrc);
      const uint32_t* vs = reinterpret_cast<const uint32_t*>(vsrc);
      uint32_t* kd = reinterpret_cast<uint32_t*>(kdst);
      uint32_t* vd = reinterpret_cast<uint32_t*>(vdst);
      const int units = (int)(a.row_bytes >> 2);
      for (int u = lane; u < units; u += kWave) {
        kd[u] = ks[u];
        if (has_v) vd[u] = vs[u];
      }
    }
  }
}

// Rows of at most UPL KiB (UPL 16-byte units per lane): a wave moves two rows
// per trip, so up to 4 * UPL loads per lane are in flight before the stores
// (a 2 KiB K/V row pair alone would leave only two).
template <int UPL>
__global__ __launch_bounds__(kKvThreads) void kv_write_small_kernel(KvWriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * kKvWaves + (threadIdx.x >> 6);
  const int64_t W = (int64_t)gridDim.x * kKvWaves;
  const int64_t T = a.R > 0 ? (int64_t)a.cu[a.R] : 0;
  const int64_t count = T < 0 ? 0 : (T < a.max_tokens ? T : a.max_tokens);
  const bool has_v = a.value != nullptr;
  const int units = (int)(a.row_bytes >> 4);
  for (int64_t k0 = gw; k0 < count; k0 += 2 * W) {
    int64_t row[2] = {k0, k0 + W};
    int64_t slot[2];
    bool ok[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      slot[j] = row[j] < count ? a.slots[row[j]] : -1;
      ok[j] = slot[j] >= 0 && slot[j] < a.cache_slots;
    }
    u32x4 kv[2][UPL], vv[2][UPL];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u32x4* ks = reinterpret_cast<const u32x4*>(a.key + row[j] * a.key_stride);
#pragma unroll
      for (int x = 0; x < UPL; ++x)
        if (ok[j] && lane + x * kWave < units) kv[j][x] = __builtin_nontemporal_load(ks + lane + x * kWave);
      if (has_v) {
        const u32x4* vs = reinterpret_cast<const u32x4*>(a.value + row[j] * a.value_stride);
#pragma unroll
        for (int x = 0; x < UPL; ++x)
          if (ok[j] && lane + x * kWave < units) vv[j][x] = __builtin_nontemporal_load(vs + lane + x * kWave);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (!ok[j]) continue;
      u32x4* kd = reinterpret_cast<u32x4*>(a.key_cache + slot[j] * a.row_bytes);
#pragma unroll
      for (int x = 0; x < UPL; ++x)
        if (lane + x * kWave < units) kd[lane + x * kWave] = kv[j][x];
      if (has_v) {
        u32x4* vd = reinterpret_cast<u32x4*>(a.value_cache + slot[j] * a.row_bytes);
#pragma unroll
        for (int x = 0; x < UPL; ++x)
          if (lane + x * kWave < units) vd[lane + x * kWave] = vv[j][x];
      }
    }
  }
}

hipError_t launch_slots(const SlotArgs& a, hipStream_t s) {
  if (a.max_tokens <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((a.max_tokens + kSlotThreads - 1) / kSlotThreads);
  hipLaunchKernelGGL(slot_kernel, dim3(grid), dim3(kSlotThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_kv_write(const KvWriteArgs& a, bool vec, hipStream_t s) {
  if (a.max_tokens <= 0 || a.R <= 0) return hipSuccess;
  // enough waves to fill the chip (256 CUs x 32 waves), fewer for small batches
  int64_t want = (a.max_tokens + kKvWaves - 1) / kKvWaves;
  want = want < 1 ? 1 : (want > 2048 ? 2048 : want);
  if (vec && a.row_bytes <= 1024)
    hipLaunchKernelGGL(kv_write_small_kernel<1>, dim3((unsigned)want), dim3(kKvThreads), 0, s, a);
  else if (vec && a.row_bytes <= 2048)
    hipLaunchKernelGGL(kv_write_small_kernel<2>, dim3((unsigned)want), dim3(kKvThreads), 0, s, a);
  else if (vec && a.row_bytes <= 4096)
    hipLaunchKernelGGL(kv_write_small_kernel<4>, dim3((unsigned)want), dim3(kKvThreads), 0, s, a);
  else if (vec)
    hipLaunchKernelGGL(kv_write_kernel<true>, dim3((unsigned)want), dim3(kKvThreads), 0, s, a);
  else
    hipLaunchKernelGGL(kv_write_kernel<false>, dim3((unsigned)want), dim3(kKvThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace up
