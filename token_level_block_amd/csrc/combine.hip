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
// prep: clamp cu_seqlens and build block / chunk prefix offsets (one workgroup)
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
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void row_lse_kernel(Offsets off, int R, int rows, int n,
                                                      const float* __restrict__ chunk_lse,
                                                      float* __restrict__ row_lse) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)R * rows) return;
  const int r = (int)(idx / rows);
  const int row = (int)(idx - (int64_t)r * rows);
  const int t = row % n;
  const int N = off.cu[r + 1] - off.cu[r];
  const int ne = min(n, N);
  float res = -INFINITY;
  if (t < ne) {
    const int c0 = off.chunk[r], c1 = off.chunk[r + 1];
    float m = -INFINITY;
    for (int c = c0; c < c1; ++c) m = fmaxf(m, chunk_lse[(int64_t)c * rows + row]);
    float sum = 0.f;
    for (int c = c0; c < c1; ++c) sum += __builtin_amdgcn_exp2f(chunk_lse[(int64_t)c * rows + row] - m);
    res = m + __log2f(sum);
  }
  row_lse[idx] = res;
}

// ---------------------------------------------------------------------------
// block scores: one wave per block
// ---------------------------------------------------------------------------
constexpr int kSumWaves = 4;

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
  float acc = 0.f;
  for (int row = lane; row < rows; row += kWave) {
    if (row % n < ne) acc += __builtin_amdgcn_exp2f(src[row] - rl[row]);
  }
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) scores[gb] = acc / ((float)G * (float)ne);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const int rows = a.hq * a.n;
  const int64_t nthreads = (int64_t)a.R * rows;
  if (nthreads > 0) {
    hipLaunchKernelGGL(row_lse_kernel, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, s,
                       a.off, (int)a.R, rows, (int)a.n, a.chunk_lse, a.row_lse);
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
