// Score pass of the token-selection path: the partial GEMM of UniPrefill
// Sec. 3.2 / Sec. 3.5 Eq. 13, S = Q[N-n:N] K^T, fused with the first half of
// the online softmax and the block reduction.
//
// One workgroup owns (request, chunk of keys, KV head, slice of queries).  The
// window queries of every query head that shares the KV head (GQA) are held in
// registers as the B operand of v_mfma_f32_32x32x16_bf16; 32-key tiles of K
// are staged through LDS (double buffered) as the A operand, so each 32x32
// accumulator tile has keys on rows and queries on columns and each lane owns
// one query column.  Per 32-key tile a lane keeps a running maximum and a
// rescaled sum of 2^(c z) over the keys of the current G-block (c = softmax
// scale * log2 e); at each block end it emits the log2-domain partial
//     lse[g][row] = log2 sum_{i in block g} 2^(c z_i)
// and folds it into a per-chunk partial.  The logits never reach memory.
// Keys after a window row's own position are masked (causal masking), as
// are keys past the end of the request.
#include "common.h"

namespace up {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int D>
struct ScoreCfg {
  static constexpr int KSTEPS = D / 16;        // MFMA k-steps per 32-key tile
  static constexpr int NT = 2;                 // 32-query column tiles per wave
  static constexpr int QW = 32 * NT;           // queries per wave
  static constexpr int KT = (D <= 128) ? 64 : 32;   // keys per LDS stage
  static constexpr int ROWB = D * 2 + 16;      // padded LDS bytes per key row
  static constexpr int STAGE = KT * ROWB;      // bytes per LDS stage
  static constexpr int CHUNKS = KT * D / 8;    // 16-byte pieces per stage
  static constexpr int MIN_THREADS = 256;
  static constexpr int MAXC = (CHUNKS + MIN_THREADS - 1) / MIN_THREADS;  // pieces per thread
};

__device__ __forceinline__ float wave_swap_half(float v) { return __shfl_xor(v, 32); }

template <int D>
__global__ __launch_bounds__(512) void score_kernel(ScoreArgs a) {
  using C = ScoreCfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

  const int gc = blockIdx.x;
  const int R = a.R;
  if (gc >= a.off.chunk[R]) return;
  const int r = find_owner(a.off.chunk, R, gc);
  const int s = a.off.cu[r];
  const int N = a.off.cu[r + 1] - s;
  const int c = gc - a.off.chunk[r];
  const int k0 = c * a.chunk_keys;
  const int k1 = min(N, k0 + a.chunk_keys);
  const int n = a.n;
  const int ne = min(n, N);
  const int G = a.G;
  const int j = blockIdx.y;                 // KV head
  const int gq = a.hq / a.hkv;
  const int rows = a.hq * n;
  const int qn = gq * n;                    // queries that read KV head j
  const int nthreads = blockDim.x;
  const int nwaves = nthreads >> 6;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int half = lane >> 5;
  const int gblk0 = a.off.blk[r];

  // ---- this lane's queries (one per 32-column tile) and their B fragments ----
  const int qbase = (blockIdx.z * nwaves + wid) * C::QW;
  int qrow[C::NT];      // output row h*n + t, or -1 if the lane's query is padding
  int qlim[C::NT];      // last visible key (request-relative), -1 if none
  bf16x8 qf[C::NT][C::KSTEPS];
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) {
    const int qi = qbase + nt * 32 + (lane & 31);
    const int hh = qi / n, t = qi - (qi / n) * n;
    const bool valid = (qi < qn) && (t < ne);
    const int h = j * gq + hh;
    qrow[nt] = valid ? h * n + t : -1;
    qlim[nt] = valid ? (N - ne + t) : -1;
    const uint16_t* qp = a.q + (int64_t)(s + N - ne + t) * a.q_stride + (int64_t)h * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (valid) v = *reinterpret_cast<const u32x4*>(qp + kk * 16);
      qf[nt][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- K staging: global -> registers -> LDS ----
  const uint16_t* kbase = a.k + (int64_t)s * a.k_stride + (int64_t)j * D;
  u32x4 pre[C::MAXC];
  auto load_stage = [&](int kb) {
#pragma unroll
    for (int i = 0; i < C::MAXC; ++i) {
      const int ch = tid + i * nthreads;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ch < C::CHUNKS) {
        const int key = ch / (D / 8), part = ch - (ch / (D / 8)) * (D / 8);
        if (kb + key < k1)
          v = *reinterpret_cast<const u32x4*>(kbase + (int64_t)(kb + key) * a.k_stride + part * 8);
      }
      pre[i] = v;
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::MAXC; ++i) {
      const int ch = tid + i * nthreads;
      if (ch < C::CHUNKS) {
        const int key = ch / (D / 8), part = ch - (ch / (D / 8)) * (D / 8);
        *reinterpret_cast<u32x4*>(smem + buf * C::STAGE + key * C::ROWB + part * 16) = pre[i];
      }
    }
  };

  // ---- running softmax state per query column ----
  const float cl2 = a.c;
  float mb[C::NT], eb[C::NT], cm[C::NT], ce[C::NT];
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) { mb[nt] = -INFINITY; eb[nt] = 0.f; cm[nt] = -INFINITY; ce[nt] = 0.f; }

  const int nstages = (k1 - k0 + C::KT - 1) / C::KT;
  load_stage(k0);
  store_stage(0);
  __syncthreads();

  for (int st = 0; st < nstages; ++st) {
    const int kb = k0 + st * C::KT;
    if (st + 1 < nstages) load_stage(kb + C::KT);
    const uint8_t* sbuf = smem + (st & 1) * C::STAGE;

#pragma unroll
    for (int ks = 0; ks < C::KT / 32; ++ks) {
      const int kt = kb + ks * 32;          // first key of this tile (request-relative)
      if (kt < k1) {
        floatx16 acc[C::NT];
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) acc[nt] = floatx16{};
        const uint8_t* arow = sbuf + (ks * 32 + (lane & 31)) * C::ROWB + half * 16;
#pragma unroll
        for (int kk = 0; kk < C::KSTEPS; ++kk) {
          const bf16x8 av = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(arow + kk * 32));
#pragma unroll
          for (int nt = 0; nt < C::NT; ++nt)
            acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[nt][kk], acc[nt], 0, 0, 0);
        }
        // accumulator element e of this lane holds key kt + 8*(e/4) + 4*half + (e%4)
        const bool edge = (kt + 32 > N - ne);
#pragma unroll
        for (int nt = 0; nt < C::NT; ++nt) {
          if (edge) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int key = kt + 8 * (e >> 2) + 4 * half + (e & 3);
              if (key > qlim[nt]) acc[nt][e] = -INFINITY;
            }
          }
          float mx = acc[nt][0];
#pragma unroll
          for (int e = 1; e < 16; ++e) mx = fmaxf(mx, acc[nt][e]);
          mx = fmaxf(mx, wave_swap_half(mx));
          const float mnew = fmaxf(mb[nt], mx);
          const float muse = (mnew == -INFINITY) ? 0.f : mnew;
          const float alpha = __builtin_amdgcn_exp2f((mb[nt] - muse) * cl2);
          const float nmc = -muse * cl2;
          float sum = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[nt][e], cl2, nmc));
          eb[nt] = eb[nt] * alpha + sum;
          mb[nt] = mnew;
        }
        // block end: the next tile starts a new G-block, or the chunk ends here
        const bool bend = ((kt + 32) % G == 0) || (kt + 32 >= k1);
        if (bend) {
          const int gi = kt / G;
#pragma unroll
          for (int nt = 0; nt < C::NT; ++nt) {
            const float E = eb[nt] + wave_swap_half(eb[nt]);
            const float l = (mb[nt] == -INFINITY) ? -INFINITY : mb[nt] * cl2 + __log2f(E);
            if (half == 0 && qrow[nt] >= 0) a.lse[(int64_t)(gblk0 + gi) * rows + qrow[nt]] = l;
            const float cnew = fmaxf(cm[nt], l);
            const float cuse = (cnew == -INFINITY) ? 0.f : cnew;
            ce[nt] = ce[nt] * __builtin_amdgcn_exp2f(cm[nt] - cuse) + __builtin_amdgcn_exp2f(l - cuse);
            cm[nt] = cnew;
            mb[nt] = -INFINITY;
            eb[nt] = 0.f;
          }
        }
      }
    }
    if (st + 1 < nstages) store_stage((st + 1) & 1);
    __syncthreads();
  }

#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) {
    if (half == 0 && qrow[nt] >= 0) {
      const float l = (cm[nt] == -INFINITY) ? -INFINITY : cm[nt] + __log2f(ce[nt]);
      a.chunk_lse[(int64_t)gc * rows + qrow[nt]] = l;
    }
  }
}

template <int D>
static hipError_t launch_score_d(const ScoreArgs& a, hipStream_t s) {
  using C = ScoreCfg<D>;
  const int qn = (a.hq / a.hkv) * a.n;
  int nwaves = (qn + C::QW - 1) / C::QW;
  if (nwaves < C::MIN_THREADS / kWave) nwaves = C::MIN_THREADS / kWave;
  if (nwaves > 8) nwaves = 8;
  const int zsplit = (qn + nwaves * C::QW - 1) / (nwaves * C::QW);
  dim3 grid((unsigned)a.max_chunks, (unsigned)a.hkv, (unsigned)zsplit);
  hipLaunchKernelGGL(score_kernel<D>, grid, dim3(nwaves * kWave), 0, s, a);
  return hipGetLastError();
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
