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
//   upk_copy_launch  a streaming device copy, one 8 KiB piece per wave at a
//                    time with eight 16-byte nontemporal loads in flight per
//                    lane (the row copies' access pattern without the gather).
//
// Built into libuppeaks.so, separate from libuniprefill.so; only the
// benchmark loads it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
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

// each wave copies whole 8 KiB pieces: lane l moves 16-byte units l + 64 x,
// x = 0..7, all eight loads in flight before the stores
__global__ __launch_bounds__(kCopyThreads) void copy_peak_kernel(const u32x4* __restrict__ src,
                                                                 u32x4* __restrict__ dst, int64_t n) {
  constexpr int kUnits = 8 * 64;   // 16-byte units per 8 KiB piece
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (kCopyThreads / 64);
  const int64_t pieces = (n + kUnits - 1) / kUnits;
  for (int64_t c = (int64_t)blockIdx.x * (kCopyThreads / 64) + (threadIdx.x >> 6); c < pieces; c += waves) {
    const int64_t base = c * kUnits + lane;
    u32x4 v[8];
#pragma unroll
    for (int x = 0; x < 8; ++x)
      if (base + 64 * x < n) v[x] = __builtin_nontemporal_load(src + base + 64 * x);
#pragma unroll
    for (int x = 0; x < 8; ++x)
      if (base + 64 * x < n) __builtin_nontemporal_store(v[x], dst + base + 64 * x);
  }
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

// Enqueue a copy of `bytes` (a multiple of 16; both pointers 16-byte aligned)
// from src to dst on `stream`.  Returns 0, -1 on bad arguments, or the HIP error.
int32_t upk_copy_launch(const void* src, void* dst, int64_t bytes, int32_t blocks, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || bytes <= 0 || bytes % 16 != 0 || blocks < 1) return -1;
  if (((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return -1;
  hipLaunchKernelGGL(copy_peak_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream,
                     (const u32x4*)src, (u32x4*)dst, bytes / 16);
  return (int32_t)hipGetLastError();
}

}  // extern "C"
