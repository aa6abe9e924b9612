// Metadata patch after a drop (UniPrefill Sec. 3.5, "vLLM scheduler
// integration", and Eq. 17): seq_lens lose the dropped tokens,
// num_actual_tokens becomes the compacted total, each request's drop history
// gains (layer, retained length), and the per-layer decode table
// seqused_base[l][r] takes the retained length for every later layer.
// Runs on the device so the host never waits for the kept counts.
#include "common.h"

namespace up {

__global__ __launch_bounds__(256) void metadata_kernel(int layer, int L, int R,
                                                       const int32_t* __restrict__ cu_old,
                                                       const int32_t* __restrict__ cu_new,
                                                       int32_t* __restrict__ seq_lens,
                                                       int32_t* __restrict__ nat,
                                                       int32_t* __restrict__ drop_count,
                                                       int32_t* __restrict__ drop_layer,
                                                       int32_t* __restrict__ drop_len, int max_drops,
                                                       int32_t* __restrict__ seqused_base) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r == 0) nat[0] = cu_new[R];
  if (r >= R) return;
  const int32_t N = max(0, cu_old[r + 1] - cu_old[r]);
  const int32_t K = max(0, cu_new[r + 1] - cu_new[r]);
  const int32_t s = seq_lens[r] - (N - K);
  seq_lens[r] = s;
  const int32_t c = drop_count[r];
  if (c >= 0 && c < max_drops) {
    drop_layer[(int64_t)r * max_drops + c] = layer;
    drop_len[(int64_t)r * max_drops + c] = s;
  }
  drop_count[r] = c + 1;
  if (seqused_base != nullptr)
    for (int l = layer + 1; l < L; ++l) seqused_base[(int64_t)l * R + r] = s;
}

hipError_t launch_metadata(int32_t layer, int32_t L, int32_t R, const int32_t* cu_old,
                           const int32_t* cu_new, int32_t* seq_lens, int32_t* nat,
                           int32_t* drop_count, int32_t* drop_layer, int32_t* drop_len,
                           int32_t max_drops, int32_t* seqused_base, hipStream_t s) {
  const int blocks = (R + 255) / 256 > 0 ? (R + 255) / 256 : 1;
  hipLaunchKernelGGL(metadata_kernel, dim3(blocks), dim3(256), 0, s, (int)layer, (int)L, (int)R,
                     cu_old, cu_new, seq_lens, nat, drop_count, drop_layer, drop_len, (int)max_drops,
                     seqused_base);
  return hipGetLastError();
}

}  // namespace up
