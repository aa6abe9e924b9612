// Score pass of the token-selection path: the partial GEMM of UniPrefill
// Sec. 3.2 / Sec. 3.5 Eq. 13, S = Q[N-n:N] K^T, fused with the first half of
// the online softmax and the block reduction.
//
// One workgroup owns (request, chunk of keys, KV head, slice of queries).  The
// window queries of every query head that shares the KV head (GQA) are held in
// registers as the B operand of v_mfma_f32_32x32x16_bf16 (at d = 128 they
// arrive through LDS in the K rows' layout, so their loads are coalesced).  K streams through
// a double-buffered LDS ring with gfx950's direct global-to-LDS 16-byte loads
// (no staging registers, XOR-swizzled rows so the A-operand reads are free of
// bank conflicts) and feeds the A operand, so each 32x32 accumulator tile has
// keys on rows and queries on columns and each lane owns one query column.
// Each lane keeps, per query column, a reference logit (the running maximum
// so far, raised only when needed) and sums 2^(c(z-ref))
// over the keys of the current G-block (c = softmax scale * log2 e).  A tile
// whose per-lane partial sum exceeds 2^20 (or is not finite) is redone with
// its exact maximum as the new reference, so every term stays within fp32
// range; the common case needs no per-logit max.  At each block end a lane
// emits the log2-domain partial
//     lse[g][row] = log2 sum_{i in block g} 2^(c z_i)
// and adds the block's linear sum (relative to the same reference, rescaled
// with it) to a per-chunk sum.  Blocks are written in pairs: the first of two
// is held in registers, and when the second closes one lane swap gives both
// column sums (one block per half-wave), so a pair costs one logarithm and
// one store.  The logits never reach memory.
// Keys after a window row's own position are masked (causal masking), as
// are keys past the end of the request.
#include "common.h"
#include "score_plan.h"

namespace up {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int D, int NW, int NT_>
struct ScoreCfg {
  static constexpr int KSTEPS = D / 16;              // MFMA k-steps per 32-key tile
  static constexpr int NT = NT_;                     // 32-query column tiles per wave
  static constexpr int QW = 32 * NT;                 // queries per wave
  static constexpr int KT = (D <= 128) ? 128 : 64;   // keys per LDS stage
  static constexpr int SUB = KT / 32;                // 32-key tiles per stage
  static constexpr int ROWB = D * 2;                 // bytes per key row in LDS (no padding)
  static constexpr int PPR = D / 8;                  // 16-byte pieces per key row
  static constexpr int SWZ = PPR < 16 ? PPR - 1 : 15;   // piece p of key r sits in slot p ^ (r & SWZ)
  static constexpr int STAGE = KT * ROWB;            // bytes per LDS stage
  static constexpr int KPI = 1024 / ROWB;            // keys per 1 KB wave load
  static constexpr int NPW = STAGE / 1024 / NW;      // 1 KB wave loads per wave per stage
  static_assert(STAGE % (1024 * NW) == 0, "a stage must split evenly into 1 KB wave loads");
  // Window queries staged through LDS at start-up: each wave's 32-query tiles
  // land in the second K buffer (idle until the first stage prefetches into
  // it) and a region after the ring, wherever the workgroups a CU holds still
  // fit in its 160 KB.  Row loads then fill whole cache lines, where loads in
  // the MFMA operand layout touch 32 lines each (128K layer: 1.5 us faster).
  static constexpr int TILEB = 32 * ROWB;            // bytes of one 32-query tile
  static constexpr int QBYTES = NW * NT * TILEB;
  static constexpr int QR = QBYTES > STAGE ? QBYTES - STAGE : 0;
  static constexpr int WGCU = NW == 4 ? 2 : 1;        // workgroups per CU (launch bounds)
  static constexpr bool QLDS = (2 * STAGE + QR) * WGCU <= 160 * 1024;
};

template <int V> struct IntC { static constexpr int value = V; };

// s_waitcnt vmcnt(0) with the other counters left free (gfx9 encoding)
constexpr int kWaitVmcnt0 = 0x0F70;

// value of the lane 32 positions away (the other half of the same query column)
__device__ __forceinline__ float other_half(float v) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  // each lane now holds {v[l], v[l ^ 32]} in some order
  const float a = __uint_as_float(pr[0]), b = __uint_as_float(pr[1]);
  return (__lane_id() < 32) ? b : a;
}

__device__ __forceinline__ float half_max(float v) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}

__device__ __forceinline__ float half_sum(float v) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// half sums of two values at once: lanes 0-31 get a[l] + a[l + 32], lanes
// 32-63 get b[l - 32] + b[l] (the swap trades a's upper half for b's lower)
__device__ __forceinline__ float pair_sum(float a, float b) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// sum over this lane's 16 logits of 2^(c z + nrc), nrc = -c * ref
__device__ __forceinline__ float tile_sum(const floatx16& acc, float cl2, float nrc) {
  float s0 = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[0], cl2, nrc));
  float s1 = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[1], cl2, nrc));
  float s2 = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[2], cl2, nrc));
  float s3 = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[3], cl2, nrc));
#pragma unroll
  for (int e = 4; e < 16; e += 4) {
    s0 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[e + 0], cl2, nrc));
    s1 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[e + 1], cl2, nrc));
    s2 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[e + 2], cl2, nrc));
    s3 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[e + 3], cl2, nrc));
  }
  return (s0 + s1) + (s2 + s3);
}

// Largest tile partial accepted without rescaling; keeps the block and chunk
// sums far from fp32 overflow (a lane adds at most 2^20 per 32-key tile, so
// even a chunk of 2^20 keys stays below 2^35).
constexpr float kRescaleAbove = 1048576.0f;   // 2^20

// GT = G/32 tiles per block when G is 32, 64 or 128 (block ends known at
// compile time in the plain stages), 0 for any other multiple of 32.
// Launch bounds: eight-wave workgroups run one per CU, four-wave ones two per
// CU (the residency the chunk planner counts on); either way two waves per
// SIMD, so each wave may use 256 registers.
template <int D, int NW, int GT, int NT>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void score_kernel(ScoreArgs a) {
  using C = ScoreCfg<D, NW, NT>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE + (C::QLDS ? C::QR : 0)];

  // Grid x enumerates (key chunk, query slice).  Workgroups are dealt to the
  // 8 XCDs round-robin by id, so ids 8 apart share an XCD and its L2: the
  // slices of one chunk take ids 8 apart and run together, reading the
  // chunk's K from HBM once.
  const int qslices = ((a.hq / a.hkv) * a.n + NW * C::QW - 1) / (NW * C::QW);
  const int lx = (int)blockIdx.x & 7, rest = (int)blockIdx.x >> 3;
  const int zs = rest % qslices;
  const int gc = (rest / qslices) * 8 + lx;
  const int R = a.R;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int r, s, N, c, gblk0;
  if (a.cu_in != nullptr) {
    // Offsets straight from cu_seqlens (R < 64): lane e loads entry e; two
    // uniform loops over the entries (lane reads into scalar registers) form
    // the clamped running maximum and the prefix sums of the block and chunk
    // counts, lane e keeping entry e of each.  Every wave derives them itself;
    // workgroup (0, 0) publishes them for the kernels that follow.
    const int32_t cuv = lane <= R ? max(0, min(a.cu_in[lane], a.cap)) : 0;
    int32_t cu_l = 0, len_l = 0, run = 0;
    for (int e = 0; e <= R; ++e) {
      const int32_t v = max(run, __builtin_amdgcn_readlane(cuv, e));
      if (lane == e) {
        cu_l = v;
        len_l = v - run;   // request e - 1 (lane 0: nothing before it)
      }
      run = v;
    }
    if (lane == 0) len_l = 0;
    const int32_t nb_l = (int32_t)((uint32_t)(len_l + a.G - 1) / (uint32_t)a.G);
    const int32_t nc_l = (int32_t)((uint32_t)(len_l + a.chunk_keys - 1) / (uint32_t)a.chunk_keys);
    int32_t blk_l = 0, chunk_l = 0, sb = 0, sc = 0;
    for (int e = 0; e <= R; ++e) {
      sb += __builtin_amdgcn_readlane(nb_l, e);
      sc += __builtin_amdgcn_readlane(nc_l, e);
      if (lane == e) {
        blk_l = sb;
        chunk_l = sc;
      }
    }
    if (blockIdx.x == 0 && blockIdx.y == 0 && wid == 0 && lane <= R) {
      a.off.cu[lane] = cu_l;
      a.off.blk[lane] = blk_l;
      a.off.chunk[lane] = chunk_l;
      if (a.block_offsets_out) a.block_offsets_out[lane] = blk_l;
    }
    if (gc >= sc) return;
    // owner: the last request whose first chunk is at or before gc
    r = (int)__popcll(__ballot(lane < R && chunk_l <= gc)) - 1;
    s = __builtin_amdgcn_readlane(cu_l, r);
    N = __builtin_amdgcn_readlane(cu_l, r + 1) - s;
    c = gc - __builtin_amdgcn_readlane(chunk_l, r);
    gblk0 = __builtin_amdgcn_readlane(blk_l, r);
  } else {
    if (gc >= a.off.chunk[R]) return;
    r = find_owner(a.off.chunk, R, gc);
    s = a.off.cu[r];
    N = a.off.cu[r + 1] - s;
    c = gc - a.off.chunk[r];
    gblk0 = a.off.blk[r];
  }
  const int k0 = c * a.chunk_keys;
  const int k1 = min(N, k0 + a.chunk_keys);
  const int n = a.n;
  const int ne = min(n, N);
  const int G = a.G;
  const int j = blockIdx.y;                 // KV head
  const int gq = a.hq / a.hkv;
  const int rows = a.hq * n;
  const int qn = gq * n;                    // queries that read KV head j
  constexpr int nwaves = NW;
  const int half = lane >> 5;

  // ---- this lane's queries (one per 32-column tile) and their B fragments ----
  const int qbase = (zs * nwaves + wid) * C::QW;
  int qrow[C::NT];      // output row h*n + t, or -1 if the lane's query is padding
  int qlim[C::NT];      // last visible key (request-relative), -1 if none
  bf16x8 qf[C::NT][C::KSTEPS];
  const int lkey = lane / C::PPR, lslot = lane % C::PPR;
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) {
    const int qi = qbase + nt * 32 + (lane & 31);
    const int hh = qi / n, t = qi - (qi / n) * n;
    const bool valid = (qi < qn) && (t < ne);
    const int h = j * gq + hh;
    qrow[nt] = valid ? h * n + t : -1;
    qlim[nt] = valid ? (N - ne + t) : -1;
    if constexpr (!C::QLDS) {
      const uint16_t* qp = a.q + (int64_t)(s + N - ne + t) * a.q_stride + (int64_t)h * D + half * 8;
#pragma unroll
      for (int kk = 0; kk < C::KSTEPS; ++kk) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (valid) v = *reinterpret_cast<const u32x4*>(qp + kk * 16);
        qf[nt][kk] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }
  // tile nt of this wave: LDS address of its 32 query rows (the region after
  // the ring, then the ring's second buffer)
  auto qtile = [&](int nt) -> uint8_t* {
    const int q = nt * nwaves + wid;
    return q * C::TILEB < C::QR ? smem + 2 * C::STAGE + q * C::TILEB : smem + C::STAGE + (q * C::TILEB - C::QR);
  };
  // a tile whose 32 queries are all valid and rows of one query head
  // (wave-uniform)
  auto tile_full = [&](int nt) -> bool {
    const int f = qbase + nt * 32;
    return f + 32 <= qn && f - (f / n) * n + 32 <= ne;
  };
  if constexpr (C::QLDS) {
    // rows of each tile as K rows are staged: wave load i holds rows KPI*i ..
    // KPI*i + KPI-1, lane slot lslot holds piece lslot ^ (row & SWZ).  A full
    // tile is 32 consecutive window rows of one head; otherwise each row is
    // placed on its own, and a row past the window or the last query re-reads
    // the first window query (zeroed after the read)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      if (tile_full(nt)) {
        const int f = qbase + nt * 32, hf = f / n, tf = f - hf * n;
        const uint16_t* tb = a.q + (int64_t)(s + N - ne + tf) * a.q_stride + (int64_t)(j * gq + hf) * D;
#pragma unroll
        for (int i = 0; i < 32 / C::KPI; ++i) {
          const int rr = C::KPI * i + lkey;
          const int p = lslot ^ (rr & C::SWZ);
          __builtin_amdgcn_global_load_lds((const void*)(tb + (int64_t)rr * a.q_stride + p * 8),
              (__attribute__((address_space(3))) void*)(qtile(nt) + i * 1024), 16, 0, 0);
        }
        continue;
      }
      const int qi0 = qbase + nt * 32 + lkey;
      int hh = qi0 / n, t = qi0 - (qi0 / n) * n;
#pragma unroll
      for (int i = 0; i < 32 / C::KPI; ++i) {
        if (i > 0) {
          t += C::KPI;
          while (t >= n) { t -= n; ++hh; }
        }
        const int rr = C::KPI * i + lkey;
        const bool valid = (qi0 + C::KPI * i < qn) && (t < ne);
        const int tt = valid ? t : 0, h = j * gq + (valid ? hh : 0);
        const int p = lslot ^ (rr & C::SWZ);
        const uint16_t* g = a.q + (int64_t)(s + N - ne + tt) * a.q_stride + (int64_t)h * D + p * 8;
        __builtin_amdgcn_global_load_lds((const void*)g,
            (__attribute__((address_space(3))) void*)(qtile(nt) + i * 1024), 16, 0, 0);
      }
    }
  }

  // ---- K staging: direct global -> LDS loads (16 bytes per lane) ----
  // wave load c of a stage fills LDS bytes [c KB, c KB + 1 KB): keys KPI*c + lane/PPR,
  // slot lane%PPR, which holds piece slot ^ (key & SWZ) of that key (XOR swizzle)
  const uint16_t* kbase = a.k + (int64_t)s * a.k_stride + (int64_t)j * D;
  auto load_stage = [&](int kb, int buf) {
#pragma unroll
    for (int i = 0; i < C::NPW; ++i) {
      const int cidx = wid * C::NPW + i;
      const int key = C::KPI * cidx + lkey;
      const int p = lslot ^ (key & C::SWZ);
      const int gk = min(kb + key, k1 - 1);   // rows past the chunk end re-read a valid row; they are masked
      const uint16_t* g = kbase + (int64_t)gk * a.k_stride + p * 8;
      __builtin_amdgcn_global_load_lds((const void*)g,
          (__attribute__((address_space(3))) void*)(smem + buf * C::STAGE + cidx * 1024), 16, 0, 0);
    }
  };

  // A-fragment reads: key row ks*32 + (lane&31), pieces kk*2 + half (swizzled)
  const int arow = lane & 31;
  const int aswz = arow & C::SWZ;   // (ks*32 + arow) & SWZ == arow & SWZ since SWZ < 32
  auto mfma_tile = [&](const uint8_t* sbuf, int ks, floatx16 (&acc)[C::NT]) {
    const uint8_t* rowp = sbuf + (ks * 32 + arow) * C::ROWB;
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      const int slot = (kk * 2 + half) ^ aswz;
      const bf16x8 av = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(rowp + (slot << 4)));
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt)
        acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[nt][kk], kk == 0 ? floatx16{} : acc[nt], 0, 0, 0);
    }
  };

  // ---- softmax state per query column ----
  const float cl2 = a.c;
  // ref: reference logit; eb: this lane's sum over the open block, ebh over
  // the held block (number hold_gi, -1 if none) and cs over the chunk's
  // closed blocks, all of 2^(c (z - ref))
  float ref[C::NT], nrc[C::NT], eb[C::NT], ebh[C::NT], cs[C::NT];
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) {
    ref[nt] = -INFINITY; nrc[nt] = INFINITY; eb[nt] = 0.f; ebh[nt] = 0.f; cs[nt] = 0.f;
  }
  int hold_gi = -1;
  // byte offset of a lane's entry in a block pair's partials: half 0 writes the
  // held block, half 1 the next one (row qrow of each)
  uint32_t pair_off[C::NT];
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) pair_off[nt] = (uint32_t)(qrow[nt] + half * rows) * 4u;

  // rare: raise the reference to the exact running maximum and redo the tile
  auto rescale = [&](floatx16 (&acc)[C::NT], float (&ts)[C::NT]) {
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      float mx = fmaxf(fmaxf(acc[nt][0], acc[nt][1]), acc[nt][2]);
#pragma unroll
      for (int e = 3; e < 15; e += 2) mx = fmaxf(fmaxf(mx, acc[nt][e]), acc[nt][e + 1]);
      mx = fmaxf(mx, acc[nt][15]);
      const float mnew = fmaxf(ref[nt], half_max(mx));
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      const float f = __builtin_amdgcn_exp2f((ref[nt] - muse) * cl2);
      eb[nt] *= f;
      ebh[nt] *= f;
      cs[nt] *= f;
      ref[nt] = mnew;
      nrc[nt] = -muse * cl2;
      ts[nt] = tile_sum(acc[nt], cl2, nrc[nt]);
    }
  };
  // block gi is complete: hold it, or emit it with the held one; either way
  // add it to the chunk sum
  auto flush = [&](int gi) {
    if (hold_gi < 0) {
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt) {
        ebh[nt] = eb[nt];
        cs[nt] += eb[nt];
        eb[nt] = 0.f;
      }
      hold_gi = gi;
      return;
    }
    // blocks close in order, so the pair is (gi - 1, gi): the held block's row
    // base is uniform and each lane adds its own fixed byte offset
    char* pb = reinterpret_cast<char*>(a.lse + (int64_t)(gblk0 + hold_gi) * rows);
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      const float E = pair_sum(ebh[nt], eb[nt]);
      const float l = (ref[nt] == -INFINITY) ? -INFINITY : ref[nt] * cl2 + __log2f(E);
      if (qrow[nt] >= 0) *reinterpret_cast<float*>(pb + pair_off[nt]) = l;
      cs[nt] += eb[nt];
      eb[nt] = 0.f;
    }
    hold_gi = -1;
  };
  // general tile: causal / tail masking, any block size
  auto process = [&](floatx16 (&acc)[C::NT], int kt) {
    // accumulator element e of this lane holds key kt + 8*(e/4) + 4*half + (e%4)
    if (kt + 32 > N - ne) {
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kt + 8 * (e >> 2) + 4 * half + (e & 3);
          if (key > qlim[nt]) acc[nt][e] = -INFINITY;
        }
    }
    float ts[C::NT];
    bool bad = false;
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      ts[nt] = tile_sum(acc[nt], cl2, nrc[nt]);
      bad |= !(ts[nt] <= kRescaleAbove);
    }
    if (__any(bad)) rescale(acc, ts);
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) eb[nt] += ts[nt];
    // block end: the next tile starts a new G-block, or the chunk ends here
    if (((kt + 32) % G == 0) || (kt + 32 >= k1)) flush(kt / G);
  };

  const int nstages = (k1 - k0 + C::KT - 1) / C::KT;
  load_stage(k0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  if constexpr (C::QLDS) {
    // this wave's query tiles have landed (its own loads): B fragments in the
    // MFMA operand layout, read like the A fragments (row lane&31, piece
    // kk*2 + half, swizzled); padding and out-of-window lanes get zeros
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      const uint8_t* rowp = qtile(nt) + arow * C::ROWB;
#pragma unroll
      for (int kk = 0; kk < C::KSTEPS; ++kk) {
        const int slot = (kk * 2 + half) ^ aswz;
        qf[nt][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(rowp + (slot << 4)));
      }
      if (!tile_full(nt)) {
        // padding and out-of-window lanes get zeros
#pragma unroll
        for (int kk = 0; kk < C::KSTEPS; ++kk)
          if (qrow[nt] < 0) qf[nt][kk] = bf16x8{};
      }
    }
  }
  // every wave's fragment reads are done before the first stage prefetches
  // into the second buffer
  __syncthreads();

  floatx16 acc[C::NT];
  // one stage; the LDS buffer it reads is a compile-time constant, so the
  // fragment addresses are loop-invariant registers plus immediate offsets
  auto stage = [&](int st, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const int kb = k0 + st * C::KT;
    // the next stage lands in the other buffer while this one is consumed
    if (st + 1 < nstages) load_stage(kb + C::KT, BUF ^ 1);
    const uint8_t* sbuf = smem + BUF * C::STAGE;
    const bool plain = (kb + C::KT <= k1) && (kb + C::KT <= N - ne);
    if (GT > 0 && plain) {
      // every tile full and unmasked; block ends at fixed tiles
#pragma unroll
      for (int ks = 0; ks < C::SUB; ++ks) {
        // MFMA bursts at raised wave priority: the SIMD's other wave fills the
        // VALU while this one streams the matrix core
        __builtin_amdgcn_s_setprio(1);
        mfma_tile(sbuf, ks, acc);
        __builtin_amdgcn_s_setprio(0);
        float ts[C::NT];
        bool bad = false;
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) {
          ts[nt] = tile_sum(acc[nt], cl2, nrc[nt]);
          bad |= !(ts[nt] <= kRescaleAbove);
        }
        if (__any(bad)) rescale(acc, ts);
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) eb[nt] += ts[nt];
        if constexpr (GT > 0 && GT <= C::SUB) {
          if ((ks + 1) % GT == 0) flush((int)((unsigned)(kb + ks * 32) / (32u * GT)));
        } else if constexpr (GT > 0) {
          if (ks + 1 == C::SUB && ((unsigned)(kb + C::KT) % (32u * GT)) == 0)
            flush((int)((unsigned)(kb + ks * 32) / (32u * GT)));
        }
      }
    } else {
      const int nsub = min(C::SUB, (k1 - kb + 31) / 32);   // 32-key tiles holding keys < k1
#pragma unroll
      for (int ks = 0; ks < C::SUB; ++ks) {
        if (ks < nsub) {
          mfma_tile(sbuf, ks, acc);
          process(acc, kb + ks * 32);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // this wave's loads of the next stage have landed
    __syncthreads();
  };
  int st = 0;
  for (; st + 1 < nstages; st += 2) {
    stage(st, IntC<0>{});
    stage(st + 1, IntC<1>{});
  }
  if (st < nstages) stage(st, IntC<0>{});

  if (hold_gi >= 0) {
    // the chunk ended on the first of a pair
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) {
      const float E = half_sum(ebh[nt]);
      const float l = (ref[nt] == -INFINITY) ? -INFINITY : ref[nt] * cl2 + __log2f(E);
      if (half == 0 && qrow[nt] >= 0) a.lse[(int64_t)(gblk0 + hold_gi) * rows + qrow[nt]] = l;
    }
  }
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) {
    const float S = half_sum(cs[nt]);
    if (half == 0 && qrow[nt] >= 0) {
      const float l = (ref[nt] == -INFINITY) ? -INFINITY : ref[nt] * cl2 + __log2f(S);
      a.chunk_lse[(int64_t)gc * rows + qrow[nt]] = l;
    }
  }
}

template <int D, int GT>
static hipError_t launch_score_dg(const ScoreArgs& a, hipStream_t s) {
  const ScoreLaunch L = score_launch_for(a.d, a.hq, a.hkv, a.n);
  // x: (key chunk, query slice) with the chunk count rounded up to 8 (ids
  // past the last chunk exit at once), y: KV head
  const dim3 grid((unsigned)((a.max_chunks + 7) / 8 * 8 * L.zsplit), (unsigned)a.hkv);
  if (L.nt == 1) {
    if (L.nw == 4)
      hipLaunchKernelGGL((score_kernel<D, 4, GT, 1>), grid, dim3(4 * kWave), 0, s, a);
    else
      hipLaunchKernelGGL((score_kernel<D, 8, GT, 1>), grid, dim3(8 * kWave), 0, s, a);
    return hipGetLastError();
  }
  if (L.nw == 4) {
    // four waves of two tiles only at d <= 128 (score_launch_for): at d = 256 the
    // fragments would not fit the two workgroups per CU its launch bounds promise
    if constexpr (D <= 128)
      hipLaunchKernelGGL((score_kernel<D, 4, GT, 2>), grid, dim3(4 * kWave), 0, s, a);
    else
      return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((score_kernel<D, 8, GT, 2>), grid, dim3(8 * kWave), 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_score_d(const ScoreArgs& a, hipStream_t s) {
  switch (a.G) {
    case 32: return launch_score_dg<D, 1>(a, s);
    case 64: return launch_score_dg<D, 2>(a, s);
    case 128: return launch_score_dg<D, 4>(a, s);
    default: return launch_score_dg<D, 0>(a, s);
  }
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t s) {
  if (a.max_chunks <= 0) return hipSuccess;
  switch (a.d) {
    case 64: return launch_score_d<64>(a, s);
    case 128: return launch_score_d<128>(a, s);
    case 256: return launch_score_d<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace up
