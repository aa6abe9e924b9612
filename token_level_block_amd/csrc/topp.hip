// Top-p block selection and block-to-token expansion (UniPrefill Sec. 3.3
// Eq. 5 and Sec. 3.5 Eq. 14 with the expansion step that follows it).
//
// Blocks are ranked by the packed key  (phi(b_g) << 32) | g  in descending
// order, phi being the sign-bit-decided monotone map of Eq. 14.  Instead of
// sorting, the kernel finds the pivot block pi(k*) directly: a weighted
// most-significant-digit radix select over the 64-bit keys, whose weights
// are the exact integer masses q_g = floor(b_g * 2^shift) (shift chosen so
// that the total fits 52 bits).  The pivot is the largest key whose suffix
// mass (over keys >= it) reaches thr = p * total; the kept blocks are exactly
// the keys >= pivot.  Integer sums make the result independent of the order
// of any reduction, so it matches a sequential sort-and-scan bit for bit.
//
// The digits start at the highest bit in which the request's keys differ
// (the bits above it are common to all keys): block scores share their sign
// and the top exponent bits, so a plain top-byte digit would put most keys
// into a handful of bins, serialise their LDS atomics, and need one pass more.
//
// The same kernel expands the kept blocks into the token mask.  One workgroup
// runs per key chunk of a request (the chunks the score pass uses): every
// workgroup of a request finds the same pivot (the selection is a pure
// function of the request's scores), then writes the mask bytes of its own
// chunk; the request's first chunk also writes the keep flags and the kept
// count.  So the mask of a long request is written by many workgroups at once
// without a second launch.
#include "common.h"

namespace up {

constexpr int kToppThreads = 1024;
constexpr int kToppWaves = kToppThreads / kWave;
constexpr int kToppCache = 4096;   // requests with at most this many blocks keep their keys in LDS

__device__ __forceinline__ uint32_t phi_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b >> 31) ? ~b : (b ^ 0x80000000u);
}

// Positive and finite (excludes +0, negatives, inf, nan).
__device__ __forceinline__ bool usable(uint32_t b) { return b != 0u && b < 0x7F800000u; }

template <typename T>
__device__ __forceinline__ T block_reduce(T v, T* red, bool is_max) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  for (int o = 32; o >= 1; o >>= 1) {
    T x = __shfl_xor(v, o);
    v = is_max ? (x > v ? x : v) : v + x;
  }
  if (lane == 0) red[wid] = v;
  __syncthreads();
  T t = red[0];
  for (int w = 1; w < kToppWaves; ++w) t = is_max ? (red[w] > t ? red[w] : t) : t + red[w];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kToppThreads) void topp_kernel(ToppArgs a) {
  __shared__ unsigned long long s_keys[kToppCache];
  // two histograms: one is filled while the other, used by the previous pass,
  // is cleared, so a pass needs no barrier of its own for the clearing
  __shared__ unsigned long long h_mass[2][256];
  __shared__ uint32_t h_cnt[2][256];
  __shared__ unsigned long long h_key[256];   // a key of each bin (the key, when the bin holds one)
  __shared__ uint32_t red32[kToppWaves], red_or[kToppWaves], red_and[kToppWaves];
  __shared__ unsigned long long s_above;
  __shared__ int s_dsel;
  __shared__ uint32_t s_cnt;

  const int gc = blockIdx.x;
  const int R = a.R;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  // empty requests own no chunk: the first workgroup reports them
  if (gc == 0)
    for (int e = tid; e < R; e += kToppThreads)
      if (a.off.cu[e + 1] == a.off.cu[e]) a.kept[e] = 0;
  if (gc >= a.off.chunk[R]) return;
  const int r = find_owner(a.off.chunk, R, gc);
  const int c = gc - a.off.chunk[r];   // chunk within the request
  const bool first = c == 0;           // writes the request's flags, count and score copy
  const int N = a.off.cu[r + 1] - a.off.cu[r];
  const int b0 = a.off.blk[r];
  const int nb = a.off.blk[r + 1] - b0;   // >= 1: a request with a chunk has tokens
  const float* sc = a.scores + b0;
  const bool copy = first && a.scores_copy != nullptr && a.scores_copy != a.scores;
  const bool cached = nb <= kToppCache;
  auto key = [&](float x, int g) -> unsigned long long {
    return ((unsigned long long)phi_bits(x) << 32) | (unsigned long long)(uint32_t)g;
  };
  for (int d = tid; d < 256; d += kToppThreads) { h_mass[0][d] = 0ull; h_cnt[0][d] = 0u; }

  // one read of the scores: the largest usable one (for the mass scale), the
  // keys (into LDS), and the OR / AND of the keys' score halves (for the
  // first digit)
  uint32_t mxb = 0, por = 0u, pand = ~0u;
  for (int g = tid; g < nb; g += kToppThreads) {
    const float x = sc[g];
    if (copy) a.scores_copy[b0 + g] = x;
    const uint32_t b = __float_as_uint(x);
    if (usable(b) && b > mxb) mxb = b;
    const uint32_t ph = phi_bits(x);
    if (cached) s_keys[g] = ((unsigned long long)ph << 32) | (unsigned long long)(uint32_t)g;
    por |= ph;
    pand &= ph;
  }
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t xm = __shfl_xor(mxb, o);
    mxb = xm > mxb ? xm : mxb;
    por |= __shfl_xor(por, o);
    pand &= __shfl_xor(pand, o);
  }
  if (lane == 0) {
    red32[wid] = mxb;
    red_or[wid] = por;
    red_and[wid] = pand;
  }
  __syncthreads();   // (also publishes s_keys and the cleared first histogram)
  mxb = red32[0];
  por = red_or[0];
  pand = red_and[0];
  for (int w = 1; w < kToppWaves; ++w) {
    mxb = red32[w] > mxb ? red32[w] : mxb;
    por |= red_or[w];
    pand &= red_and[w];
  }
  // largest usable score -> binary exponent e, shift = 52 - ceil(log2 nb) - e
  int e = 0;
  if (mxb != 0u) (void)frexp((double)__uint_as_float(mxb), &e);
  const int nbits = (nb <= 1) ? 0 : 32 - __clz(nb - 1);
  const int shift = 52 - nbits - e;

  auto mass = [&](float x) -> unsigned long long {
    return usable(__float_as_uint(x)) ? (unsigned long long)ldexp((double)x, shift) : 0ull;
  };
  // the score back from the high half of a packed key (phi is invertible)
  auto score_of = [](unsigned long long k) -> float {
    const uint32_t ph = (uint32_t)(k >> 32);
    return __uint_as_float((ph & 0x80000000u) ? (ph ^ 0x80000000u) : ~ph);
  };
  auto key_at = [&](int g) -> unsigned long long { return cached ? s_keys[g] : key(sc[g], g); };

  // thr = p * (total integer mass); only wave 0 uses it, and it takes the total
  // from the first pass's histogram, which every key enters
  double thr = 0.0;

  // Weighted radix select, at most 8 bits per pass, from the highest bit in
  // which keys differ down; `prefix` holds the pivot's bits above `rem`.  The
  // block indices 0 .. nb-1 fill the low half, so when all score halves agree
  // the keys first differ in the top bit of nb - 1.
  const uint32_t pdiff = por ^ pand;
  int rem;
  unsigned long long prefix;
  if (pdiff != 0u) {
    rem = 64 - __clz(pdiff);
    prefix = rem >= 64 ? 0ull : (unsigned long long)(pand >> (rem - 32));
  } else {
    rem = nbits;
    prefix = ((unsigned long long)pand << 32) >> rem;
  }
  unsigned long long above = 0, pivot = (unsigned long long)pand << 32;   // (the key, when nb == 1)
  int buf = 0;
  bool first_pass = true;
  while (rem > 0) {
    const int sh = rem > 8 ? rem - 8 : 0, w = rem - sh;
    for (int g = tid; g < nb; g += kToppThreads) {
      const unsigned long long k = key_at(g);
      if (rem >= 64 || (k >> rem) == prefix) {
        const int d = (int)((k >> sh) & ((1ull << w) - 1ull));
        atomicAdd(&h_mass[buf][d], mass(score_of(k)));
        atomicAdd(&h_cnt[buf][d], 1u);
        h_key[d] = k;
      }
    }
    __syncthreads();
    if (wid == 0) {
      // lane L covers digits 255-4L .. 252-4L, i.e. descending key order
      unsigned long long m[4];
      uint32_t cn[4];
      unsigned long long loc = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 255 - 4 * lane - i;
        m[i] = h_mass[buf][d];
        cn[i] = h_cnt[buf][d];
        loc += m[i];
      }
      unsigned long long incl = loc;
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long x = __shfl_up(incl, o);
        if (lane >= o) incl += x;
      }
      if (first_pass) thr = a.p * (double)__shfl(incl, 63);   // all 256 bins: the total mass
      unsigned long long run = above + (incl - loc);
      int first = -1;
      unsigned long long abv = 0;
      uint32_t cfirst = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned long long before = run;
        run += m[i];
        if (first < 0 && cn[i] > 0u && (double)run >= thr) { first = i; abv = before; cfirst = cn[i]; }
      }
      const unsigned long long bal = __ballot(first >= 0);
      const int sel = bal ? (__ffsll((long long)bal) - 1) : 63;
      if (lane == sel) {
        if (first < 0) { first = 3; abv = run - m[3]; cfirst = cn[3]; }  // unreachable: total >= thr
        s_dsel = 255 - 4 * lane - first;
        s_above = abv;
        s_cnt = cfirst;
      }
    } else {
      // the other waves clear the histogram the next pass fills
      for (int d = tid - kWave; d < 256; d += kToppThreads - kWave) {
        h_mass[buf ^ 1][d] = 0ull;
        h_cnt[buf ^ 1][d] = 0u;
      }
    }
    __syncthreads();
    const int dsel = s_dsel;
    prefix = (prefix << w) | (unsigned long long)dsel;
    above = s_above;
    rem = sh;
    if (rem == 0) {
      pivot = prefix;   // all 64 bits fixed
    } else if (s_cnt == 1u) {
      pivot = h_key[dsel];   // the group holds a single key
      break;
    }
    buf ^= 1;
    first_pass = false;
  }

  const int A = a.A, n = a.n, G = a.G;
  if (first) {
    // keep flags and the closed-form token count of the expanded mask
    const int w0 = max(max(N - n, 0), A);
    uint32_t cnt = 0;
    for (int g = tid; g < nb; g += kToppThreads) {
      const bool kp = key_at(g) >= pivot;
      a.keep_block[b0 + g] = kp ? 1 : 0;
      const int lo = g * G, hi = min(N, lo + G);
      int t;
      if (kp) {
        t = hi - lo;
      } else {
        t = max(0, min(hi, A) - lo) + max(0, hi - max(lo, w0));
      }
      cnt += (uint32_t)t;
    }
    cnt = block_reduce<uint32_t>(cnt, red32, false);
    if (tid == 0) a.kept[r] = (int32_t)cnt;
  }

  // this chunk's token mask: M_i = keep[block(i)] or i < A or i >= N - n
  // (request-relative i)
  const int lo = c * a.chunk_keys, hi = min(N, lo + a.chunk_keys);
  uint8_t* __restrict__ mrow = a.mask + a.off.cu[r];
  for (int i = lo + tid; i < hi; i += kToppThreads) {
    const bool m = i < A || i >= N - n || key_at(i / G) >= pivot;
    mrow[i] = m ? 1 : 0;
  }
}

hipError_t launch_topp(const ToppArgs& a, hipStream_t s) {
  if (a.max_chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(topp_kernel, dim3((unsigned)a.max_chunks), dim3(kToppThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace up
