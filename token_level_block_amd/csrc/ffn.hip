// A downstream sublayer on the retained rows: the gated FFN of the LLaMA
// family, y = (silu(x Wg^T) * (x Wu^T)) Wd^T, token by token (UniPrefill
// Sec. 3.4 Eq. 7: after a drop every later sublayer maps only the retained
// rows; Eq. 9-10: that is where the saving comes from).
//
// Two launches of one bf16 MFMA GEMM kernel, C[i][j] = sum_k W[i][k] X[j][k]
// (weights in the [out_features][in_features] layout of a linear layer, so
// both operands are K-contiguous rows):
//   1. gate/up: i runs over the 2F gate and up rows, j over the tokens; the
//      epilogue forms h = silu(gate) * up in fp32 from the two accumulators
//      and stores h as bf16 [rows][F] (the [rows][2F] product never leaves
//      the registers);
//   2. down: i over the D rows of Wd, j over the tokens, K = F; y as bf16.
// A workgroup computes a 256 (weight rows) x 256 (tokens) tile with
// v_mfma_f32_32x32x16_bf16: four waves of 128 x 128, each holding 4 x 4
// accumulator tiles.  Operands stream through a two-stage LDS ring with
// gfx950's direct global-to-LDS 16-byte loads, 64 K-elements per stage, in
// 128-byte rows whose 16-byte pieces are XOR-swizzled by (row / 2) & 7, so
// the 16 lanes of each pass of a fragment read hit 16 different bank groups.
// In the gate/up launch the workgroup's 256 weight rows are 64 gate rows, the
// 64 up rows of the same channels, then the next 64 of each: a wave's first
// two accumulator rows of tiles are gate and its last two the matching up
// channels, so gate and up of one (token, channel) sit in the same lane and
// register.  Rows past the end are clamped (their results are not stored) and
// K past the end reads a zero piece.  Workgroups are dealt to the XCDs so that
// each XCD walks its own run of tiles, 8 token panels at a time, and the
// workgroups running together share weight and token panels in their L2.
#include "../../include/uniprefill.h"
#include "common.h"

namespace up {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFfnThreads = 256;          // four waves
constexpr int kTileI = 256;               // weight rows per workgroup
constexpr int kTileJ = 256;               // tokens per workgroup
constexpr int kBK = 64;                   // K elements per stage (128-byte rows)
constexpr int kStageBytes = (kTileI + kTileJ) * kBK * 2;   // 64 KB
constexpr int kGroupJ = 8;                // token panels walked together

__device__ __attribute__((aligned(16))) const uint32_t kZeroPiece[4] = {0u, 0u, 0u, 0u};

struct FfnGemmArgs {
  const uint16_t* w;     // bf16 [n_rows][K] weight rows (gate/up: [2F][K])
  const uint16_t* x;     // bf16 [rows][K] token rows
  int64_t K;             // multiple of 8
  int64_t rows;          // tokens
  int64_t F;             // gate/up launch: channels (w holds gate rows then up rows)
  int64_t n_out;         // output columns: F (gate/up) or D (down)
  uint16_t* out;         // bf16 [rows][n_out]
  int32_t tiles_i, tiles_j;
};

__device__ __forceinline__ float silu_f32(float g) {
  // g * sigmoid(g) = g / (1 + 2^(-g log2 e)); large negative g gives -0
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

template <bool kGateUp>
__global__ __launch_bounds__(kFfnThreads, 1) void ffn_gemm_kernel(FfnGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wi = wid >> 1, wj = wid & 1;
  const int half = lane >> 5;

  // tile of this workgroup: XCD x (= id mod 8) walks tiles [x T/8, (x+1) T/8)
  // in order; a run of tiles covers kGroupJ token panels for each weight panel
  const int64_t ntiles = (int64_t)a.tiles_i * a.tiles_j;
  const int64_t per_xcd = (ntiles + 7) / 8;
  const int64_t t = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (t >= ntiles) return;
  const int64_t grp = t / ((int64_t)kGroupJ * a.tiles_i), wgi = t % ((int64_t)kGroupJ * a.tiles_i);
  const int64_t gj = min((int64_t)kGroupJ, (int64_t)a.tiles_j - grp * kGroupJ);
  const int ti = (int)(wgi / gj);
  const int tj = (int)(grp * kGroupJ + wgi % gj);

  const int64_t K = a.K;
  const int64_t n_w = kGateUp ? 2 * a.F : a.n_out;   // weight rows
  // weight row of tile row r
  auto wrow = [&](int r) -> int64_t {
    int64_t i;
    if (kGateUp) {
      // [gate 64 | up 64 | gate 64 | up 64] of channels f0 .. f0 + 127
      const int64_t f = (int64_t)ti * 128 + (r >> 7) * 64 + (r & 63);
      i = ((r >> 6) & 1) ? a.F + min(f, a.F - 1) : min(f, a.F - 1);
    } else {
      i = min((int64_t)ti * kTileI + r, n_w - 1);
    }
    return i;
  };

  // this lane's loads: wave chunk c (0..7) of the weight tile and of the
  // token tile covers 8 rows; lane L writes LDS row 8c' + L/8, slot L % 8 and
  // reads global piece slot ^ ((row / 2) & 7)
  const uint16_t* wptr[8];
  const uint16_t* xptr[8];
  const int slot = lane & 7;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int r = (wid * 8 + c) * 8 + (lane >> 3);
    const int p = slot ^ ((r >> 1) & 7);
    wptr[c] = a.w + wrow(r) * K + p * 8;
    const int64_t j = min((int64_t)tj * kTileJ + r, a.rows - 1);
    xptr[c] = a.x + j * K + p * 8;
  }
  auto load_stage = [&](int64_t kb, int buf) {
    uint8_t* sbase = smem + buf * kStageBytes;
    const bool full = kb + kBK <= K;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int r = (wid * 8 + c) * 8 + (lane >> 3);
      const int64_t kp = kb + (int64_t)((slot ^ ((r >> 1) & 7)) * 8);   // first K of the piece
      const void* gw = (full || kp < K) ? (const void*)(wptr[c] + kb) : (const void*)kZeroPiece;
      const void* gx = (full || kp < K) ? (const void*)(xptr[c] + kb) : (const void*)kZeroPiece;
      __builtin_amdgcn_global_load_lds(gw, (__attribute__((address_space(3))) void*)(sbase + (wid * 8 + c) * 1024),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          gx, (__attribute__((address_space(3))) void*)(sbase + kTileI * kBK * 2 + (wid * 8 + c) * 1024), 16, 0, 0);
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = floatx16{};

  // fragment rows of this lane: weight rows wi*128 + m*32 + lane%32, token
  // rows wj*128 + n*32 + lane%32 (both with (row / 2) & 7 == (lane % 32 / 2) & 7)
  const int frow = lane & 31;
  const int fswz = (frow >> 1) & 7;
  const int nst = (int)((K + kBK - 1) / kBK);
  load_stage(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) load_stage((int64_t)(st + 1) * kBK, buf ^ 1);
    const uint8_t* wt = smem + buf * kStageBytes + (wi * 128 + frow) * 128;
    const uint8_t* xt = smem + buf * kStageBytes + kTileI * kBK * 2 + (wj * 128 + frow) * 128;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int off = ((kk * 2 + half) ^ fswz) * 16;
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        af[m] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(wt + m * 32 * 128 + off));
#pragma unroll
      for (int n = 0; n < 4; ++n)
        bfr[n] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xt + n * 32 * 128 + off));
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[m], bfr[n], acc[m][n], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // this wave's loads of the next stage have landed
    __syncthreads();
  }

  // epilogue: element e of tile (m, n) is weight row i0 + 8 (e / 4) + 4 half +
  // e % 4, token j = tj*256 + wj*128 + n*32 + lane % 32; four consecutive
  // output columns go out as one 8-byte store
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int64_t j = (int64_t)tj * kTileJ + wj * 128 + n * 32 + frow;
    if (j >= a.rows) continue;
    uint16_t* orow = a.out + j * a.n_out;
    if constexpr (kGateUp) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t f = (int64_t)ti * 128 + wi * 64 + m * 32 + 8 * g + 4 * half;
          bf16x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = (__bf16)(silu_f32(acc[m][n][4 * g + q]) * acc[m + 2][n][4 * g + q]);
          if (f + 4 <= a.F) {
            *reinterpret_cast<bf16x4*>(orow + f) = o;
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (f + q < a.F) reinterpret_cast<__bf16*>(orow)[f + q] = o[q];
          }
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t i = (int64_t)ti * kTileI + wi * 128 + m * 32 + 8 * g + 4 * half;
          bf16x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = (__bf16)acc[m][n][4 * g + q];
          if (i + 4 <= a.n_out) {
            *reinterpret_cast<bf16x4*>(orow + i) = o;
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (i + q < a.n_out) reinterpret_cast<__bf16*>(orow)[i + q] = o[q];
          }
        }
      }
    }
  }
}

static hipError_t launch_ffn_gemm(bool gate_up, const FfnGemmArgs& a, hipStream_t s) {
  const int64_t ntiles = (int64_t)a.tiles_i * a.tiles_j;
  const unsigned grid = (unsigned)((ntiles + 7) / 8 * 8);
  if (gate_up)
    hipLaunchKernelGGL(ffn_gemm_kernel<true>, dim3(grid), dim3(kFfnThreads), 0, s, a);
  else
    hipLaunchKernelGGL(ffn_gemm_kernel<false>, dim3(grid), dim3(kFfnThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace up

namespace {

size_t align_up256(size_t x) { return (x + 255) / 256 * 256; }

// widths the kernels take: positive multiples of 8 (16-byte rows), at most 2^24
bool ffn_widths_ok(int32_t D, int32_t F) {
  return D >= 8 && F >= 8 && D % 8 == 0 && F % 8 == 0 && D <= (1 << 24) && F <= (1 << 24);
}

}  // namespace

extern "C" {

size_t up_ffn_workspace_bytes(int32_t hidden, int32_t intermediate, int64_t rows) {
  if (!ffn_widths_ok(hidden, intermediate) || rows < 0) return 0;
  return align_up256((size_t)(rows > 0 ? rows : 1) * (size_t)intermediate * 2);
}

up_status up_ffn_forward(int32_t hidden, int32_t intermediate, const void* x, int64_t rows,
                         const void* w_gate_up, const void* w_down, void* y, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (!ffn_widths_ok(hidden, intermediate)) return UP_ERR_PARAM;
  if (rows < 0) return UP_ERR_SHAPE;
  if (rows == 0) return UP_OK;
  if (x == nullptr || w_gate_up == nullptr || w_down == nullptr || y == nullptr || workspace == nullptr)
    return UP_ERR_NULL;
  if (((uintptr_t)x | (uintptr_t)w_gate_up | (uintptr_t)w_down | (uintptr_t)y | (uintptr_t)workspace) % 16 != 0)
    return UP_ERR_ALIGN;
  const int64_t D = hidden, F = intermediate;
  const int64_t tj = (rows + up::kTileJ - 1) / up::kTileJ;
  const int64_t ti1 = (F + 127) / 128, ti2 = (D + up::kTileI - 1) / up::kTileI;
  // token-panel and tile counts must fit the 32-bit grid
  if (tj > INT32_MAX || ti1 * tj > (int64_t)UINT32_MAX - 8 || ti2 * tj > (int64_t)UINT32_MAX - 8)
    return UP_ERR_SHAPE;
  if (workspace_bytes < up_ffn_workspace_bytes(hidden, intermediate, rows)) return UP_ERR_WORKSPACE;
  uint16_t* h = static_cast<uint16_t*>(workspace);
  up::FfnGemmArgs g1{};
  g1.w = static_cast<const uint16_t*>(w_gate_up);
  g1.x = static_cast<const uint16_t*>(x);
  g1.K = D;
  g1.rows = rows;
  g1.F = F;
  g1.n_out = F;
  g1.out = h;
  g1.tiles_i = (int32_t)ti1;
  g1.tiles_j = (int32_t)tj;
  if (up::launch_ffn_gemm(true, g1, stream) != hipSuccess) return UP_ERR_HIP;
  up::FfnGemmArgs g2{};
  g2.w = static_cast<const uint16_t*>(w_down);
  g2.x = h;
  g2.K = F;
  g2.rows = rows;
  g2.F = F;
  g2.n_out = D;
  g2.out = static_cast<uint16_t*>(y);
  g2.tiles_i = (int32_t)ti2;
  g2.tiles_j = (int32_t)tj;
  if (up::launch_ffn_gemm(false, g2, stream) != hipSuccess) return UP_ERR_HIP;
  return UP_OK;
}

}  // extern "C"
