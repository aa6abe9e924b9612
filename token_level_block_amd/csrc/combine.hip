// Offset preparation and the second pass of the block-score softmax.
//
// The score kernel leaves, for every (window row, block) pair, the log2-domain
// partial  lse[g][row] = log2 sum_{i in block g} 2^(c z_i)  and for every
// (window row, key chunk) pair the same quantity over the chunk.  This pass
// forms each row's full-sequence normaliser and then the block scores of
// UniPrefill Sec. 3.2 Eq. 4:
//     b_g = 1/(G n_eff) * sum_{h,t} 2^(lse[g][h,t] - LSE[h,t]).
// All reductions run in a fixed order, so results are bit-reproducible.
#include "common.h"

namespace up {

// ---------------------------------------------------------------------------
// prep: clamp cu_seqlens and build block / chunk prefix offsets (one workgroup;
// used for more than 63 requests and for selection from given scores, since
// the score kernel derives them itself for smaller batches)
// ---------------------------------------------------------------------------
constexpr int kPrepThreads = 1024;
constexpr int kPrepWaves = kPrepThreads / kWave;

__global__ __launch_bounds__(kPrepThreads) void prep_kernel(const int32_t* __restrict__ cu_in, int R,
                                                            int64_t max_tokens, int G, int CK,
                                                            Offsets off, int32_t* block_offsets_out) {
  __shared__ int32_t scratch[kPrepWaves];
  __shared__ int32_t s_cu[kPrepThreads];
  __shared__ int32_t carry[3];  // last clamped cu, running block total, running chunk total
  const int tid = threadIdx.x;
  if (tid == 0) { carry[0] = 0; carry[1] = 0; carry[2] = 0; }
  __syncthreads();
  const int32_t cap = (int32_t)(max_tokens < 0x7fffffff ? max_tokens : 0x7fffffff);
  for (int base = 0; base <= R; base += kPrepThreads) {
    const int e = base + tid;
    // clamped cu: running maximum of max(cu_in, 0), capped at max_tokens
    const int32_t v = (e <= R) ? max(0, min(cu_in[e], cap)) : 0;
    const int32_t cu_e = max(block_inclusive_scan<true>(v, scratch), carry[0]);
    s_cu[tid] = cu_e;
    __syncthreads();
    const int32_t prev = (tid == 0) ? carry[0] : s_cu[tid - 1];
    const int32_t len = (e >= 1 && e <= R) ? (cu_e - prev) : 0;
    const int32_t nb = (len + G - 1) / G;
    const int32_t nc = (len + CK - 1) / CK;
    const int32_t sb = block_inclusive_scan<false>(nb, scratch) + carry[1];
    const int32_t sc = block_inclusive_scan<false>(nc, scratch) + carry[2];
    if (e <= R) {
      off.cu[e] = cu_e;
      off.blk[e] = sb;       // total over requests < e
      off.chunk[e] = sc;
      if (block_offsets_out) block_offsets_out[e] = sb;
    }
    __syncthreads();
    if (tid == kPrepThreads - 1) { carry[0] = cu_e; carry[1] = sb; carry[2] = sc; }
    __syncthreads();
  }
}

hipError_t launch_prep(const int32_t* cu_in, int32_t R, int64_t max_tokens, int32_t G,
                       int32_t chunk_keys, Offsets off, int32_t* block_offsets_out,
                       hipStream_t s) {
  hipLaunchKernelGGL(prep_kernel, dim3(1), dim3(kPrepThreads), 0, s, cu_in, (int)R, max_tokens,
                     (int)G, (int)chunk_keys, off, block_offsets_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// row normalisers: LSE[r][row] = log2 sum over the request's chunks
// one workgroup = 64 rows (one per lane) x 4 waves striding over the chunks
// ---------------------------------------------------------------------------
// online merge of a log2-domain term v into (m, s) = (running max, sum 2^(x-m))
__device__ __forceinline__ void lse_merge(float& m, float& s, float v) {
  const float mn = fmaxf(m, v);
  if (mn == -INFINITY) return;
  s = s * __builtin_amdgcn_exp2f(m - mn) + __builtin_amdgcn_exp2f(v - mn);
  m = mn;
}

__device__ __forceinline__ void lse_merge_pair(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * __builtin_amdgcn_exp2f(m - mn) + s2 * __builtin_amdgcn_exp2f(m2 - mn);
  m = mn;
}

constexpr int kRowWaves = 4;

__global__ __launch_bounds__(kRowWaves * kWave) void row_lse_kernel(Offsets off, int R, int rows, int n,
                                                                    const float* __restrict__ chunk_lse,
                                                                    float* __restrict__ row_lse) {
  __shared__ float pm[kRowWaves][kWave], ps[kRowWaves][kWave];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = blockIdx.y;
  const int row = blockIdx.x * kWave + lane;
  const int N = off.cu[r + 1] - off.cu[r];
  const int ne = min(n, N);
  const bool valid = row < rows && (row % n) < ne;
  float m = -INFINITY, sum = 0.f;
  if (valid) {
    const int c0 = off.chunk[r], c1 = off.chunk[r + 1];
    int c = c0 + w;
    for (; c + 3 * kRowWaves < c1; c += 4 * kRowWaves) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = chunk_lse[(int64_t)(c + u * kRowWaves) * rows + row];
#pragma unroll
      for (int u = 0; u < 4; ++u) lse_merge(m, sum, v[u]);
    }
    for (; c < c1; c += kRowWaves) lse_merge(m, sum, chunk_lse[(int64_t)c * rows + row]);
  }
  pm[w][lane] = m;
  ps[w][lane] = sum;
  __syncthreads();
  if (w == 0 && row < rows) {
    for (int u = 1; u < kRowWaves; ++u) lse_merge_pair(m, sum, pm[u][lane], ps[u][lane]);
    row_lse[(int64_t)r * rows + row] = valid ? m + __log2f(sum) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// block scores: one wave per block, 16-byte loads along the rows
// ---------------------------------------------------------------------------
constexpr int kSumWaves = 4;
typedef float floatx4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kSumWaves * kWave) void block_sum_kernel(
    Offsets off, int R, int rows, int n, int G, const float* __restrict__ lse,
    const float* __restrict__ row_lse, float* __restrict__ scores, int64_t max_blocks) {
  const int lane = threadIdx.x & 63;
  const int64_t gb = (int64_t)blockIdx.x * kSumWaves + (threadIdx.x >> 6);
  if (gb >= max_blocks) return;
  const int total = off.blk[R];
  if (gb >= total) return;
  const int r = find_owner(off.blk, R, gb);
  const int N = off.cu[r + 1] - off.cu[r];
  const int ne = min(n, N);
  const float* src = lse + gb * rows;
  const float* rl = row_lse + (int64_t)r * rows;
  float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
  if (ne == n && (rows & 3) == 0) {
    // every window row is valid: 4 rows per lane per step, eight steps' loads
    // in flight before their exponentials
    constexpr int kSteps = 8;
    for (int base = 4 * lane; base < rows; base += 4 * kWave * kSteps) {
      floatx4 v[kSteps], l[kSteps];
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
        const int row = base + u * 4 * kWave;
        if (row < rows) {
          v[u] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(src + row));
          l[u] = *reinterpret_cast<const floatx4*>(rl + row);
        }
      }
#pragma unroll
      for (int u = 0; u < kSteps; ++u) {
        if (base + u * 4 * kWave < rows) {
          acc0 += __builtin_amdgcn_exp2f(v[u][0] - l[u][0]);
          acc1 += __builtin_amdgcn_exp2f(v[u][1] - l[u][1]);
          acc2 += __builtin_amdgcn_exp2f(v[u][2] - l[u][2]);
          acc3 += __builtin_amdgcn_exp2f(v[u][3] - l[u][3]);
        }
      }
    }
  } else {
    for (int row = lane; row < rows; row += kWave)
      if (row % n < ne) acc0 += __builtin_amdgcn_exp2f(src[row] - rl[row]);
  }
  float acc = (acc0 + acc1) + (acc2 + acc3);
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) scores[gb] = acc / ((float)G * (float)ne);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const int rows = a.hq * a.n;
  if (a.R > 0) {
    hipLaunchKernelGGL(row_lse_kernel, dim3((unsigned)((rows + kWave - 1) / kWave), (unsigned)a.R),
                       dim3(kRowWaves * kWave), 0, s, a.off, (int)a.R, rows, (int)a.n, a.chunk_lse,
                       a.row_lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.max_blocks > 0) {
    hipLaunchKernelGGL(block_sum_kernel, dim3((unsigned)((a.max_blocks + kSumWaves - 1) / kSumWaves)),
                       dim3(kSumWaves * kWave), 0, s, a.off, (int)a.R, rows, (int)a.n, (int)a.G,
                       a.lse, a.row_lse, a.scores, a.max_blocks);
  }
  return hipGetLastError();
}

}  // namespace up
