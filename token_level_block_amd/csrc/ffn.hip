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
// v_mfma_f32_16x16x32_bf16: eight waves (two per SIMD, so that one wave's
// stall on a load it cannot issue yet leaves the other issuing MFMAs) of
// 128 x 64, each holding 8 x 4 accumulator tiles.  The part runs this kernel
// at its power limit, and the 16 x 16 x 32 form moves half the accumulator
// bytes per flop of the 32 x 32 x 16 one: the same loop with it holds a
// clock about 12 % higher.  Operands stream through LDS with gfx950's direct
// global-to-LDS 16-byte loads in stages of 64 K-elements: a row's 128 bytes
// per stage make whole 128-byte L2 requests (64-byte rows took twice the
// requests, and were slower).  The 160 KB of
// LDS hold a ring of five operand units (one operand's 256 rows of a stage,
// 32 KB each), so the loads of a unit are issued one to two stages before it
// is read, spread between the MFMAs (a burst stalls the waves at the texture
// unit); they are buffer loads whose only per-stage change is a scalar
// offset.  The next K-step's fragments are read one at a time between the
// current one's MFMAs, and the one barrier per stage waits only for the stage
// it needs.
// Pieces are XOR-swizzled by (row / 2) & 7, so the 16 rows of a fragment read
// hit 16 different bank groups.
// In the gate/up launch the workgroup's 256 weight rows are 64 gate rows, the
// 64 up rows of the same channels, then the next 64 of each: a wave's first
// four accumulator rows of tiles are gate and its last four the matching up
// channels, so gate and up of one (token, channel) sit in the same lane and
// register.  Rows past the end are clamped (their results are not stored) and
// K past the end reads a zero piece.  The tile walk shares token panels
// across the XCDs (through the MALL) and weight and token panels among the
// workgroups of an XCD (through its L2): ffn_walk.h.
#include "../../include/uniprefill.h"
#include "common.h"
#include "ffn_walk.h"

namespace up {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;                 // two per SIMD
constexpr int kFfnThreads = 64 * kWaves;
constexpr int kTileI = 256;               // weight rows per workgroup
constexpr int kTileJ = 256;               // tokens per workgroup
constexpr int kBK = 64;                   // K elements per stage
constexpr int kRowBytes = kBK * 2;        // one row's bytes in a stage (128)
constexpr int kPieces = kRowBytes / 16;   // 16-byte pieces per row (8)
constexpr int kNK = kBK / 32;             // MFMA K-steps per stage (2)
constexpr int kUnitBytes = 256 * kRowBytes;   // one operand's 256 rows of a stage (32 KB)
constexpr int kUnits = 5;                 // LDS ring of operand units (160 KB)
constexpr int kRowsPerLoad = 1024 / kRowBytes;   // rows one 1 KB wave load covers (8)
constexpr int kWaveRows = 256 / kWaves;         // rows of each unit one wave loads
constexpr int kChunks = kWaveRows / kRowsPerLoad;  // loads per operand per wave per stage
// wave tile: 128 weight rows (kMT MFMA tiles of 16) x kWaveTok tokens (kNT tiles of 16)
constexpr int kWaveTok = kTileJ / (kWaves / 2);
constexpr int kMT = 128 / 16;
constexpr int kNT = kWaveTok / 16;
constexpr int kTiles = kMT * kNT;                  // MFMAs per K-step per wave (32)
static_assert(kWaves == 8 && kNK == 2, "wave layout and K-step schedule");
// LDS pieces are XOR-swizzled by (row / 2) & 7: the 16 rows that share a
// 256-byte window of banks get distinct pieces
constexpr int kSwzShift = 1;
static_assert(kTileI == 256 && kTileJ == 256 && kUnits * kUnitBytes <= 160 * 1024, "LDS");

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

// buffer descriptor word 3 for raw 32-bit-element loads on gfx9-family parts
// (data format 32, no swizzle, no thread-id addressing)
constexpr int kRawBufferFlags = 0x00020000;

// a pointer in the LDS address space, as the direct-to-LDS loads take it (cast
// at the call: a helper, or a lambda, that returns one loses the kernel's
// host-side launch stub)
typedef __attribute__((address_space(3))) void* lds_void_ptr;

template <bool kGateUp>
__global__ __launch_bounds__(kFfnThreads, 1) void ffn_gemm_kernel(FfnGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kUnits * kUnitBytes];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wi = wid / (kWaves / 2), wj = wid % (kWaves / 2);
  const int quad = lane >> 4;

  // tile of this workgroup (ffn_walk.h)
  int ti = 0, tj = 0;
  if (!ffn_tile_of(blockIdx.x & 7, blockIdx.x >> 3, (uint32_t)a.tiles_i, (uint32_t)a.tiles_j, &ti, &tj)) return;

  const int64_t K = a.K;
  const int64_t n_w = kGateUp ? 2 * a.F : a.n_out;   // weight rows

  // this wave's loads: chunk c of its kWaveRows weight rows and of its
  // kWaveRows token rows covers kRowsPerLoad rows, tile row r = kWaveRows wid
  // + c kRowsPerLoad + L / kPieces for lane L, which fills LDS slot L % kPieces
  // of row r with global piece (L % kPieces) ^ swizzle(r).  Rows past the end
  // are clamped.  Each wave addresses its rows from a uniform first-row
  // pointer plus a fixed 32-bit lane offset (< 64 K 2 + 128 bytes), so a
  // stage's loads need no vector arithmetic.
  // In the gate/up launch tile rows [gate 64 | up 64 | gate 64 | up 64] are the
  // channels ti*128 + 0..127: the wave's rows rb .. rb + kWaveRows - 1 (rb =
  // kWaveRows wid) are up rows when (rb / 64) is odd, of channels ti*128 +
  // (rb / 128)*64 + rb % 64 + 0, 1, ...
  const int rb = wid * kWaveRows;
  int64_t w_first, w0, w_last;   // first weight row of the wave, unclamped first, last valid
  if (kGateUp) {
    w0 = (int64_t)ti * 128 + (rb >> 7) * 64 + (rb & 63);
    w_last = a.F - 1;
    w_first = ((rb >> 6) & 1) ? a.F : 0;   // gate or up half
  } else {
    w0 = (int64_t)ti * kTileI + rb;
    w_last = n_w - 1;
    w_first = 0;
  }
  const int64_t wb = min(w0, w_last);
  const int64_t j0 = (int64_t)tj * kTileJ + rb;
  const int64_t jb = min(j0, a.rows - 1);
  const uint8_t* wave_w = reinterpret_cast<const uint8_t*>(a.w + (w_first + wb) * K);
  const uint8_t* wave_x = reinterpret_cast<const uint8_t*>(a.x + jb * K);
  uint32_t w_off[kChunks], x_off[kChunks];
  int piece_of[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int rr = c * kRowsPerLoad + lane / kPieces;   // row within the wave's
    const int r = rb + rr;
    piece_of[c] = (lane % kPieces) ^ ((r >> kSwzShift) & (kPieces - 1));
    const int64_t rw = min(w0 + rr, w_last) - wb;
    const int64_t rx = min(j0 + rr, a.rows - 1) - jb;
    w_off[c] = (uint32_t)(rw * K * 2 + piece_of[c] * 16);
    x_off[c] = (uint32_t)(rx * K * 2 + piece_of[c] * 16);
  }
  // Operand units: unit u holds one operand of stage u / 2, 256 rows of 128
  // bytes in LDS buffer u % kUnits; the weights are the units of parity kWUnit.
  // The load schedule below gives even units the longer lead, so it goes to
  // the operand whose L2 misses go further: in the gate/up launch the weights
  // (every XCD walks its own weight panels, 235 MB between them for LLaMA-8B
  // widths), in the down launch the tokens (the activation h streams from
  // HBM, while the 117 MB of Wd stay in the MALL).
  constexpr int kWUnit = kGateUp ? 0 : 1;
  auto unit_lds = [&](int u) { return smem + (u % kUnits) * kUnitBytes; };
  // load c (0 .. kChunks - 1) of unit u, a full stage: a buffer load from the wave's
  // first row (raw, unswizzled descriptor) with the lane offset in the VGPR and
  // the stage's K position in the scalar offset, so it takes no vector
  // arithmetic at all; lane offset plus K position stay below 128 K 2 <= 2^31,
  // the descriptor's range
  const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc((void*)wave_w, (short)0, 0x7FFFFFFF, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t rs_x = __builtin_amdgcn_make_buffer_rsrc((void*)wave_x, (short)0, 0x7FFFFFFF, kRawBufferFlags);
  auto load_full = [&](int u, int c) {
    const int kb2 = (u >> 1) * (2 * kBK);
    uint8_t* dst = unit_lds(u) + (wid * kChunks + c) * 1024;
    if ((u & 1) != kWUnit)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_x, (lds_void_ptr)dst, 16, x_off[c], kb2, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_w, (lds_void_ptr)dst, 16, w_off[c], kb2, 0, 0);
  };
  // loads c0 .. kChunks - 1 of unit u of any stage, the last one possibly past K:
  // pieces past K read a zero piece
  auto load_unit = [&](int u, int c0) {
    const int64_t kb = (int64_t)(u >> 1) * kBK;
    const bool full = kb + kBK <= K;
    const bool tok = (u & 1) != kWUnit;
    const uint8_t* base = tok ? wave_x : wave_w;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      if (c < c0) continue;
      const bool in_k = full || kb + piece_of[c] * 8 < K;
      const uint8_t* g = base + (tok ? x_off[c] : w_off[c]) + kb * 2;
      __builtin_amdgcn_global_load_lds(in_k ? (const void*)g : (const void*)kZeroPiece,
                                       (lds_void_ptr)(unit_lds(u) + (wid * kChunks + c) * 1024), 16, 0, 0);
    }
  };

  floatx4 acc[kMT][kNT];
#pragma unroll
  for (int m = 0; m < kMT; ++m)
#pragma unroll
    for (int n = 0; n < kNT; ++n) acc[m][n] = floatx4{};

  // fragment f of a K-step (A tiles 0 .. kMT - 1, then B tiles): lane rows
  // weight wi*128 + 16 f + lane%16 or token wj*kWaveTok + 16 (f - kMT) + lane%16,
  // 16-byte piece 4 kk + lane/16 of the stage's 128-byte row; the swizzle is
  // that of lane%16 (the tile offsets are multiples of the swizzle period)
  const int frow = lane & 15;
  const int fswz = (frow >> kSwzShift) & (kPieces - 1);
  const int nst = (int)((K + kBK - 1) / kBK);
  const int nst_full = (int)(K / kBK);   // stages entirely inside K
  constexpr int kFrags = kMT + kNT;
  static_assert(kMT == 8 && kNT == 4 && (kFrags - 1) * 8 / 3 < kTiles, "read schedule");
  auto read_frag = [&](int st, int kk, int f, bf16x8 (&af)[kMT], bf16x8 (&bfr)[kNT]) {
    const int off = ((kk * 4 + quad) ^ fswz) * 16;
    if (f < kMT) {
      const uint8_t* wt = unit_lds(2 * st + kWUnit) + (wi * 128 + f * 16 + frow) * kRowBytes;
      af[f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(wt + off));
    } else {
      const uint8_t* xt = unit_lds(2 * st + 1 - kWUnit) + (wj * kWaveTok + (f - kMT) * 16 + frow) * kRowBytes;
      bfr[f - kMT] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xt + off));
    }
  };

  // Load sequence j: the 2 kChunks loads of units 2j + 5 (the odd unit of
  // stage j + 2) and 2j + 6 (the even unit of stage j + 3), in that order.
  // Their buffers are those of stage j's two units, free once every wave is
  // past the barrier of iteration j.  The first go out in the K-step after that
  // barrier (one stage ahead of their use), the second in the first K-step of
  // iteration j + 1 (one and a half stages ahead).
  constexpr int kN1 = kChunks, kN0 = kChunks;   // loads in K-step 1, K-step 0
  static_assert(kN1 + kN0 == 2 * kChunks && kN0 <= 8 && kN1 <= 8, "load spread");
  auto load_seq = [&](int j, int p) { load_full(2 * j + 5 + p / kChunks, p % kChunks); };
  // wait until a stage has landed, given the number of loads issued after its
  // last one (loads complete in issue order), then make every wave's loads
  // visible and every wave's earlier LDS reads complete
  auto stage_landed = [&](int later) {
    if (later >= 16)
      wait_vmcnt<16>();
    else if (later >= 8)
      wait_vmcnt<8>();
    else if (later >= 4)
      wait_vmcnt<4>();
    else
      wait_vmcnt<0>();
    // lgkmcnt(0) + barrier, without the vmcnt(0) that a workgroup fence adds
    // (it would also wait for the loads still ahead)
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("s_barrier" ::: "memory");
  };

  // Iteration st computes stage st, K-step by K-step: 32 MFMAs with the reads
  // of the next K-step's fragments spread between them; before the last
  // K-step (whose reads are those of stage st + 1's first K-step) the wave
  // waits for stage st + 1 at a barrier.  Every read of a stage's units is
  // issued before that barrier and has completed at it (lgkmcnt(0)).
  // Steady state (all units involved full): iteration st issues positions
  // kN1 .. 2 kChunks - 1 of sequence st - 1 in K-step 0 and positions
  // 0 .. kN1 - 1 of sequence st after its barrier, in K-step 1.  At the
  // barrier, stage st + 1's odd unit is positions 0 .. kChunks - 1 of
  // sequence st - 1, and the kChunks loads issued after them may still be in
  // flight.
  // Past the steady state, units are issued whole at the top of the iteration
  // (the last stage possibly partial), up to unit 2 st + 4, whose buffer was
  // freed at the barrier before.
  int next_unit = 0, partial = 0;   // first unit not fully issued; loads of it issued
  auto top_up = [&](int st) -> int {   // returns the loads issued after unit 2 st + 3
    int later = 0;
    while (next_unit <= 2 * st + 4 && (next_unit >> 1) < nst) {
      load_unit(next_unit, partial);
      if (next_unit > 2 * st + 3) later += kChunks - partial;
      ++next_unit;
      partial = 0;
    }
    return later;
  };
  bf16x8 a0[kMT], b0[kNT], a1[kMT], b1[kNT];
  auto kstep = [&](int st, int kk, bool steady, int later) __attribute__((always_inline)) {
    bf16x8(&ca)[kMT] = (kk & 1) ? a1 : a0;
    bf16x8(&cb)[kNT] = (kk & 1) ? b1 : b0;
    bf16x8(&na)[kMT] = (kk & 1) ? a0 : a1;
    bf16x8(&nb)[kNT] = (kk & 1) ? b0 : b1;
    int j = 0, p0 = 0, n = 0;
    if (steady) {
      if (kk == kNK - 1) { j = st; p0 = 0; n = kN1; }
      else { j = st - 1; p0 = kN1; n = kN0; }
    }
    // the next K-step: this stage's second, or stage st + 1's first (in the
    // last stage the wave waits for everything and reads units it never uses)
    const int rst = (kk < kNK - 1) ? st : st + 1;
    const int rkk = (kk < kNK - 1) ? kk + 1 : 0;
    if (kk == kNK - 1) stage_landed(later);
    // MFMA t, then the reads and loads of its slot: the next K-step's
    // fragments one every 8/3 slots, in the order the next K-step first uses
    // them (B0, A0, B1, B2, B3, A1 .. A7: each at least 23 slots ahead of its
    // use), and positions p0 .. p0 + n - 1 of load sequence j spread over the
    // K-step (a load the texture path cannot take yet stalls the wave, and
    // the MFMAs behind it).  The MFMA stays ahead of its slot's read: a read
    // issued first would make the wait for the previous K-step's fragments,
    // at the top of the stage loop, wait for it too.
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      acc[t / kNT][t % kNT] =
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca[t / kNT], cb[t % kNT], acc[t / kNT][t % kNT], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kFrags; ++i)
        if (t == (i * 8) / 3) read_frag(rst, rkk, i == 0 ? kMT : (i == 1 ? 0 : (i <= kNT ? kMT + i - 1 : i - kNT)), na, nb);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q < n && t == 1 + q * (kTiles - 1) / n) load_seq(j, p0 + q);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto iteration = [&](int st, bool steady) __attribute__((always_inline)) {
    const int later = steady ? kChunks : top_up(st);
#pragma unroll
    for (int kk = 0; kk < kNK; ++kk) kstep(st, kk, steady, later);
  };

  // iterations 0 .. steady_end - 1 are steady: sequences -1 .. steady_end - 1
  // are of full units
  const int steady_end = max(0, nst_full - 3);
  // prologue: stage 0 and the even unit of stage 1, then (when iteration 0 is
  // steady) the first positions of sequence -1, as iteration -1 would have
  int pro_later = top_up(-1);
  if (steady_end > 0) {
#pragma unroll
    for (int p = 0; p < kN1; ++p) load_seq(-1, p);
    pro_later += kN1;
  }
  stage_landed(pro_later);
#pragma unroll
  for (int f = 0; f < kFrags; ++f) read_frag(0, 0, f, a0, b0);
  int st = 0;
  for (; st < steady_end; ++st) iteration(st, true);
  if (steady_end > 0) {   // sequence steady_end - 1 was begun
    next_unit = 2 * steady_end + 3;
    partial = kN1;
  }
  for (; st < nst; ++st) iteration(st, false);

  // Epilogue.  Element e of accumulator tile (m, n) is weight row (output
  // column) wi*128 + m*16 + 4 (lane / 16) + e of the tile and token
  // wj*kWaveTok + n*16 + lane % 16: a lane holds runs of four columns of one
  // token.  Stored as they are, every 8-byte piece of a store instruction
  // lands in a different token row (64 cache lines per instruction), so the
  // wave first writes its output block to LDS (token-major rows, free after
  // the loop's last barrier: no wave reads the ring any more) and reads it
  // back as 16-byte pieces of 8 columns, 8 (or 4) whole row segments per
  // instruction.  16-byte pieces in an LDS row are XOR-swizzled by the token
  // so that both the 8-byte writes and the 16-byte reads spread over the banks.
  // Output widths are multiples of 8, so a 16-byte piece is wholly inside or
  // wholly past the last column.
  constexpr int kOutCols = kGateUp ? 64 : 128;        // output columns of a wave
  constexpr int kOutPieces = kOutCols / 8;            // 16-byte pieces per token row
  constexpr int kOutRowBytes = kOutCols * 2;
  static_assert(kWaves * kWaveTok * kOutRowBytes <= kUnits * kUnitBytes, "epilogue blocks fit the LDS");
  uint8_t* ob = smem + wid * (kWaveTok * kOutRowBytes);
  auto out_at = [&](int t, int c) {   // byte offset of column c (a multiple of 4) of token t
    return t * kOutRowBytes + (((c >> 3) ^ (t % kOutPieces)) << 4) + (c & 7) * 2;
  };
#pragma unroll
  for (int n = 0; n < kNT; ++n) {
    const int t = n * 16 + frow;
#pragma unroll
    for (int m = 0; m < (kGateUp ? kMT / 2 : kMT); ++m) {
      const int c = m * 16 + 4 * quad;
      bf16x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (kGateUp)
          o[q] = (__bf16)(silu_f32(acc[m][n][q]) * acc[m + kMT / 2][n][q]);
        else
          o[q] = (__bf16)acc[m][n][q];
      }
      *reinterpret_cast<bf16x4*>(ob + out_at(t, c)) = o;
    }
  }
  // first output column of the wave, and the row stride, in elements
  const int64_t col0 = kGateUp ? (int64_t)ti * 128 + wi * 64 : (int64_t)ti * kTileI + wi * 128;
  const int64_t ncols = kGateUp ? a.F : a.n_out;
  constexpr int kTokPerRound = 64 / kOutPieces;   // token rows one 64-lane pass covers
#pragma unroll
  for (int r = 0; r < kWaveTok / kTokPerRound; ++r) {
    const int t = r * kTokPerRound + lane / kOutPieces;
    const int p = lane % kOutPieces;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ob + out_at(t, p * 8));
    const int64_t j = (int64_t)tj * kTileJ + wj * kWaveTok + t;
    const int64_t col = col0 + p * 8;
    if (j < a.rows && col < ncols) *reinterpret_cast<u32x4*>(a.out + j * a.n_out + col) = v;
  }
}

static hipError_t launch_ffn_gemm(bool gate_up, const FfnGemmArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)ffn_gemm_grid(a.tiles_i, a.tiles_j);
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
  // panel counts and the grids must fit 32 bits
  if (tj > INT32_MAX || ti1 > INT32_MAX || up::ffn_gemm_grid(ti1, tj) > (int64_t)UINT32_MAX ||
      up::ffn_gemm_grid(ti2, tj) > (int64_t)UINT32_MAX)
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
