// Reference rates of the GPU the path runs on, measured the way its kernels
// use the hardware, so that roofline fractions can be quoted against what the
// part sustains as well as against its published peaks.
//
//   upk_mfma_launch  dense v_mfma_f32_32x32x16_bf16 on random operands.  The
//                    matrix pipe's power draw, and with it the clock the part
//                    holds, depends on the operand bits: constant operands
//                    run markedly faster than random ones, so random bf16
//                    values in [0.5, 2) with random signs are used.  Two
//                    independent accumulator chains per wave, two waves per
//                    SIMD (the score kernel's occupancy).
//   upk_mfma16_launch  the same with v_mfma_f32_16x16x32_bf16 (the FFN
//                    GEMM's instruction), eight accumulator chains per wave.
//                    It moves half the accumulator bytes per flop and holds a
//                    higher clock under the same power limit.
//   upk_copy_launch  a streaming device copy: one 16-byte nontemporal unit
//                    per thread, consecutive workgroups on consecutive units
//                    (the row copies' access pattern without the gather), by
//                    default one unit per thread in a single pass, the fastest
//                    plain copy shape measured on the part.
//
// Built into libuppeaks.so, separate from libuniprefill.so; only the
// benchmark loads it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaThreads = 512;   // 8 waves: two per SIMD
constexpr int kMfmaSteps = 256;     // loop trips; 16 MFMAs per trip per wave
constexpr int kCopyThreads = 256;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// two bf16 values per word: random sign and mantissa, exponent 126 or 127
__device__ __forceinline__ uint32_t random_bf16_pair(uint32_t seed) {
  return (mix32(seed) & 0x807f807fu) | 0x3f003f00u;
}

__global__ __launch_bounds__(kMfmaThreads) void mfma_peak_kernel(float* out) {
  const uint32_t t = blockIdx.x * kMfmaThreads + threadIdx.x;
  bf16x8 a[8], b0[8], b1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u32x4 va, vb0, vb1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      va[e] = random_bf16_pair(t * 97u + i * 13u + e);
      vb0[e] = random_bf16_pair(t * 31u + i * 7u + e + 1000u);
      vb1[e] = random_bf16_pair(t * 11u + i * 5u + e + 5000u);
    }
    a[i] = __builtin_bit_cast(bf16x8, va);
    b0[i] = __builtin_bit_cast(bf16x8, vb0);
    b1[i] = __builtin_bit_cast(bf16x8, vb1);
  }
  floatx16 c0 = {}, c1 = {};
  for (int it = 0; it < kMfmaSteps; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b0[i], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b1[i], c1, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e];
  out[t] = s;
}

__global__ __launch_bounds__(kMfmaThreads) void mfma16_peak_kernel(float* out) {
  const uint32_t t = blockIdx.x * kMfmaThreads + threadIdx.x;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u32x4 va, vb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      va[e] = random_bf16_pair(t * 97u + i * 13u + e);
      vb[e] = random_bf16_pair(t * 31u + i * 7u + e + 1000u);
    }
    a[i] = __builtin_bit_cast(bf16x8, va);
    b[i] = __builtin_bit_cast(bf16x8, vb);
  }
  floatx4 c[8] = {};
  for (int it = 0; it < kMfmaSteps; ++it) {
    // 32 MFMAs of 16x16x32 per trip: the flops of the 32x32x16 loop's 16
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[(i * 2 + j) & 7], b[(i + j) & 7], c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (c[j][0] + c[j][1]) + (c[j][2] + c[j][3]);
  out[t] = s;
}

// thread t of workgroup w copies units w*256 + t + k*(grid*256), k = 0, 1, ...
__global__ __launch_bounds__(kCopyThreads) void copy_peak_kernel(const u32x4* __restrict__ src,
                                                                 u32x4* __restrict__ dst, int64_t n) {
  const int64_t step = (int64_t)gridDim.x * kCopyThreads;
  for (int64_t i = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x; i < n; i += step)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

extern "C" {

// Floats upk_mfma_launch writes to `out` (one per thread).
int64_t upk_mfma_out_floats(int32_t blocks) { return (int64_t)blocks * kMfmaThreads; }

// Dense flops one upk_mfma_launch performs.
double upk_mfma_flops(int32_t blocks) {
  const double per_wave = (double)kMfmaSteps * 16.0 * 2.0 * 32.0 * 32.0 * 16.0;
  return per_wave * (kMfmaThreads / 64) * (double)blocks;
}

// Enqueue the MFMA loop on `stream`; `out` holds upk_mfma_out_floats(blocks)
// floats of device memory.  Returns 0, or -1 on bad arguments, or the HIP error.
int32_t upk_mfma_launch(float* out, int32_t blocks, hipStream_t stream) {
  if (out == nullptr || blocks < 1) return -1;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(kMfmaThreads), 0, stream, out);
  return (int32_t)hipGetLastError();
}

// The 16x16x32 loop: the same flops per launch (upk_mfma_flops), the same
// output size, the same return values.
int32_t upk_mfma16_launch(float* out, int32_t blocks, hipStream_t stream) {
  if (out == nullptr || blocks < 1) return -1;
  hipLaunchKernelGGL(mfma16_peak_kernel, dim3((unsigned)blocks), dim3(kMfmaThreads), 0, stream, out);
  return (int32_t)hipGetLastError();
}

// Enqueue a copy of `bytes` (a multiple of 16; both pointers 16-byte aligned)
// from src to dst on `stream` with `blocks` workgroups of 256 threads, or with
// one thread per 16-byte unit when blocks < 1 (at most 2^31 - 1 workgroups).
// Returns 0, -1 on bad arguments, or the HIP error.
int32_t upk_copy_launch(const void* src, void* dst, int64_t bytes, int32_t blocks, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || bytes <= 0 || bytes % 16 != 0) return -1;
  if (((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return -1;
  const int64_t n = bytes / 16;
  const int64_t g = blocks >= 1 ? blocks : (n + kCopyThreads - 1) / kCopyThreads;
  if (g > 0x7fffffff) return -1;
  hipLaunchKernelGGL(copy_peak_kernel, dim3((unsigned)g), dim3(kCopyThreads), 0, stream,
                     (const u32x4*)src, (u32x4*)dst, n);
  return (int32_t)hipGetLastError();
}

}  // extern "C"
