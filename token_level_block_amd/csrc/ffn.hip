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
// accumulator tiles.  Operands stream through a four-stage LDS ring with
// gfx950's direct global-to-LDS 16-byte loads, 32 K-elements per stage, each
// stage's loads issued three stages before it is consumed (the loads come from
// L2 or further: one stage of lead left the waves waiting on them).  Rows are
// 64 bytes; their 16-byte pieces are XOR-swizzled by (row / 4) & 3, so the 16
// lanes of each pass of a fragment read hit 16 different bank groups.
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
constexpr int kBK = 32;                   // K elements per stage (64-byte rows)
constexpr int kStages = 4;                // LDS ring depth; loads run kStages - 1 stages ahead
constexpr int kRowBytes = kBK * 2;
constexpr int kStageBytes = (kTileI + kTileJ) * kRowBytes;   // 32 KB
constexpr int kLoadsPerStage = kStageBytes / 4 / 1024;       // 1 KB wave loads per wave per stage (8)
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

// s_waitcnt vmcnt(n) with the other counters left free (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// a pointer in the LDS address space, as the direct-to-LDS loads take it (cast
// at the call: a helper, or a lambda, that returns one loses the kernel's
// host-side launch stub)
typedef __attribute__((address_space(3))) void* lds_void_ptr;

template <bool kGateUp>
__global__ __launch_bounds__(kFfnThreads, 1) void ffn_gemm_kernel(FfnGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStageBytes];
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

  // this wave's loads: chunk c (0..3) of its 64 weight rows and of its 64
  // token rows covers 16 rows, tile row r = 16 (4 wid + c) + L / 4 for lane L,
  // which fills LDS slot L % 4 of row r with global piece (L % 4) ^ ((r / 4) & 3)
  // = (L % 4) ^ ((L / 16) & 3).  Rows past the end are clamped.  Each wave
  // addresses its rows from a uniform first-row pointer plus a fixed 32-bit
  // lane offset (< 64 K 2 + 64 bytes), so a stage's loads need no vector
  // arithmetic.
  // In the gate/up launch tile rows [gate 64 | up 64 | gate 64 | up 64] are the
  // channels ti*128 + 0..127: wave wid holds gate (wid even) or up (wid odd)
  // rows of channels ti*128 + (wid / 2)*64 + 0..63.
  constexpr int kChunks = kLoadsPerStage / 2;
  const int piece = (lane & 3) ^ ((lane >> 4) & 3);
  int64_t w_first, w0, w_last;   // first weight row of the wave, unclamped first, last valid
  if (kGateUp) {
    const int64_t f0 = (int64_t)ti * 128 + (wid >> 1) * 64;
    w0 = f0;
    w_last = a.F - 1;
    w_first = (wid & 1) ? a.F : 0;   // gate or up half
  } else {
    w0 = (int64_t)ti * kTileI + wid * 64;
    w_last = n_w - 1;
    w_first = 0;
  }
  const int64_t wb = min(w0, w_last);
  const int64_t j0 = (int64_t)tj * kTileJ + wid * 64;
  const int64_t jb = min(j0, a.rows - 1);
  const uint8_t* wave_w = reinterpret_cast<const uint8_t*>(a.w + (w_first + wb) * K);
  const uint8_t* wave_x = reinterpret_cast<const uint8_t*>(a.x + jb * K);
  uint32_t w_off[kChunks], x_off[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int64_t rw = min(w0 + c * 16 + (lane >> 2), w_last) - wb;
    const int64_t rx = min(j0 + c * 16 + (lane >> 2), a.rows - 1) - jb;
    w_off[c] = (uint32_t)(rw * K * 2 + piece * 16);
    x_off[c] = (uint32_t)(rx * K * 2 + piece * 16);
  }
  auto lds_at = [&](int buf, bool tokens, int c) {
    return smem + buf * kStageBytes + (tokens ? kTileI * kRowBytes : 0) + (wid * kChunks + c) * 1024;
  };
  // load i (0..7) of a full stage: weight chunk i / 2 (i even) or token chunk i / 2
  auto load_full = [&](int64_t kb, int buf, int i) {
    const int c = i >> 1;
    if (i & 1)
      __builtin_amdgcn_global_load_lds(wave_x + kb * 2 + x_off[c], (lds_void_ptr)lds_at(buf, true, c), 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(wave_w + kb * 2 + w_off[c], (lds_void_ptr)lds_at(buf, false, c), 16, 0, 0);
  };
  // any stage, the last one possibly past K: pieces past K read a zero piece
  auto load_stage = [&](int64_t kb, int buf) {
    const bool full = kb + kBK <= K;
    const bool in_k = full || kb + piece * 8 < K;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const void* gw = in_k ? (const void*)(wave_w + kb * 2 + w_off[c]) : (const void*)kZeroPiece;
      const void* gx = in_k ? (const void*)(wave_x + kb * 2 + x_off[c]) : (const void*)kZeroPiece;
      __builtin_amdgcn_global_load_lds(gw, (lds_void_ptr)lds_at(buf, false, c), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(gx, (lds_void_ptr)lds_at(buf, true, c), 16, 0, 0);
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = floatx16{};

  // fragment rows of this lane: weight rows wi*128 + m*32 + lane%32, token
  // rows wj*128 + n*32 + lane%32 (both with (row / 4) & 3 == (lane % 32 / 4) & 3)
  const int frow = lane & 31;
  const int fswz = (frow >> 2) & 3;
  const int nst = (int)((K + kBK - 1) / kBK);
  auto read_frags = [&](int buf, int kk, bf16x8 (&af)[4], bf16x8 (&bfr)[4]) {
    const uint8_t* wt = smem + buf * kStageBytes + (wi * 128 + frow) * kRowBytes;
    const uint8_t* xt = smem + buf * kStageBytes + kTileI * kRowBytes + (wj * 128 + frow) * kRowBytes;
    const int off = ((kk * 2 + half) ^ fswz) * 16;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      af[m] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(wt + m * 32 * kRowBytes + off));
#pragma unroll
    for (int n = 0; n < 4; ++n)
      bfr[n] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xt + n * 32 * kRowBytes + off));
  };
  // the 16 MFMAs of one K-step: the first, then the other 15
  auto first_mfma = [&](const bf16x8 (&af)[4], const bf16x8 (&bfr)[4]) {
    acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0], bfr[0], acc[0][0], 0, 0, 0);
  };
  auto other_mfmas = [&](const bf16x8 (&af)[4], const bf16x8 (&bfr)[4]) {
#pragma unroll
    for (int t = 1; t < 16; ++t)
      acc[t >> 2][t & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t >> 2], bfr[t & 3], acc[t >> 2][t & 3], 0, 0, 0);
  };
  // the same 15 with loads i0 .. i0 + 3 of a full stage issued after MFMAs 2,
  // 5, 8 and 11: a stage's eight loads are spread over both K-steps, so that
  // the four waves' loads come no faster than the texture path takes them
  // (a load it cannot take yet stalls the wave, and the MFMAs behind it)
  auto other_mfmas_loading = [&](const bf16x8 (&af)[4], const bf16x8 (&bfr)[4], int64_t kb, int lbuf, int i0) {
#pragma unroll
    for (int t = 1; t < 16; ++t) {
      acc[t >> 2][t & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t >> 2], bfr[t & 3], acc[t >> 2][t & 3], 0, 0, 0);
      if (t % 3 == 2 && t <= 11) load_full(kb, lbuf, i0 + t / 3);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // wait until a stage has landed, given the number of loads issued after its
  // last one (loads complete in issue order), then make every wave's loads
  // visible and every wave's earlier LDS reads complete
  auto stage_landed = [&](int later) {
    if (later >= 24)
      wait_vmcnt<24>();
    else if (later >= 20)
      wait_vmcnt<20>();
    else if (later >= 16)
      wait_vmcnt<16>();
    else if (later >= 12)
      wait_vmcnt<12>();
    else if (later >= 8)
      wait_vmcnt<8>();
    else if (later >= 4)
      wait_vmcnt<4>();
    else
      wait_vmcnt<0>();
    // lgkmcnt(0) + barrier, without the vmcnt(0) that a workgroup fence adds
    // (it would also wait for the loads of the stages still ahead)
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("s_barrier" ::: "memory");
  };

  // Per stage st (its K-step 0 fragments already in registers): load stage
  // ls = st + kStages - 1 into the buffer stage st - 1 used, read K-step 1
  // while the MFMAs of K-step 0 run (after the first, so that the wait before
  // it covers only the older reads), then (stage st + 1 landed) read its
  // K-step 0 while the MFMAs of K-step 1 run.  A full stage's loads go half
  // into each K-step's MFMAs; the last, partial one is loaded at once.  Every
  // read of a stage's buffer is issued before the barrier of the iteration
  // that computes it and has completed at that barrier (lgkmcnt(0)), so loads
  // issued after it overwrite a buffer no wave still reads.
  static_assert(kBK == 32 && kStages >= 3 && kStages <= 5 && kLoadsPerStage == 8,
                "two K-steps per stage, eight loads per stage, at most three later stages in flight");
  bf16x8 a0[4], b0[4], a1[4], b1[4];
  const int nst_full = (int)(K / kBK);   // stages entirely inside K
  auto step = [&](int st, bool interleaved) __attribute__((always_inline)) {
    const int buf = st % kStages;
    const int ls = st + kStages - 1;
    const int64_t lkb = (int64_t)ls * kBK;
    if (!interleaved && ls < nst) load_stage(lkb, ls % kStages);
    first_mfma(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(buf, 1, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    if (interleaved)
      other_mfmas_loading(a0, b0, lkb, ls % kStages, 0);
    else
      other_mfmas(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    // stage st + 1; issued after it: the stages up to ls - 1 and half of ls
    // (interleaved), else the stages up to min(ls, nst - 1).  In the last
    // stage this waits for nothing and reads a buffer it never uses.
    stage_landed(interleaved ? kLoadsPerStage * (kStages - 3) + kLoadsPerStage / 2
                             : kLoadsPerStage * max(0, min(ls, nst - 1) - st - 1));
    first_mfma(a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    read_frags((st + 1) % kStages, 0, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    if (interleaved)
      other_mfmas_loading(a1, b1, lkb, ls % kStages, kLoadsPerStage / 2);
    else
      other_mfmas(a1, b1);
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int q = 0; q < kStages - 1; ++q)
    if (q < nst) load_stage((int64_t)q * kBK, q);
  stage_landed(kLoadsPerStage * min(kStages - 2, nst - 1));
  read_frags(0, 0, a0, b0);
  int st = 0;
  // while the stage loaded is a full one, its loads go between MFMAs
  for (; st + kStages - 1 < nst_full; ++st) step(st, true);
  for (; st < nst; ++st) step(st, false);

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
