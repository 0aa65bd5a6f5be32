// (d) Rank and select: keep the protected window plus the top N - |protected|
// tokens by (composite score desc, position desc).
//
// CONF-KV explainer, Methodology, token ranking and eviction: tokens are ranked
// by a score combining EMA attention mass and recency within the chosen budget,
// and a hard protected window P is never evicted.  Significance and claims: the
// method is a no-op while the cache stays within its budget.
//
// The score s = s_ema*(e/e_max) + s_rec*(pos/t) is evaluated in fp32 with one
// rounding per operation (contraction off).  s >= 0, so its IEEE bits order like
// the value; the 64-bit key (bits(s) << 32 | pos) is unique per token and orders
// exactly as (s desc, pos desc).  The K-th largest candidate key is found by an
// MSB-first radix select over 8-bit digits: a 256-bin histogram in LDS per pass,
// the bin holding the K-th key found by one wavefront's suffix scan, and an early
// stop as soon as that bin's keys are all kept.  When only a few candidates go
// (the steady state evicts one token per step), the threshold is found instead by
// that many rounds of a block-wide minimum over the candidate keys.  Keys live in
// LDS when the cache fits (the steady state); otherwise each pass recomputes them
// from the cache.
#include "common.hpp"

namespace confkv {

constexpr int kSelThreads = 1024;
constexpr int kSelLdsKeys = 6144;  // keys cached in LDS (48 KB)
constexpr int kFewEvict = 8;       // evictions up to which minimum rounds replace the radix select

__device__ inline uint64_t wave_min_u64(uint64_t x) {
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)x, off), hi = __shfl_xor((uint32_t)(x >> 32), off);
    const uint64_t y = ((uint64_t)hi << 32) | lo;
    x = y < x ? y : x;
  }
  return x;
}

__device__ inline uint64_t sel_key(float e, float emax, int pos, int t, float s_ema, float s_rec) {
#pragma clang fp contract(off)
  const float ehat = emax > 0.f ? e / emax : 0.f;
  const float r = t > 0 ? (float)pos / (float)t : 1.0f;
  const float a = s_ema * ehat;
  const float b = s_rec * r;
  const float s = a + b;
  return ((uint64_t)__float_as_uint(s) << 32) | (uint32_t)pos;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(conf_cache c, Dims dm, int layer0,
                                                             const int32_t* __restrict__ budget,
                                                             uint8_t* __restrict__ keep_all) {
  const int lb = layer0 * dm.B + blockIdx.x;
  const int l = lb / dm.B, b = lb % dm.B;
  const int n8 = c.n8[lb], n16 = c.n16[lb], t = c.t[lb];
  const int n = n8 + n16;
  const int N = budget[(size_t)b * dm.L + l];
  uint8_t* keep8 = keep_all + (size_t)lb * dm.capt;
  uint8_t* keep16 = keep8 + dm.cap8;
  const int32_t* pos8 = c.pos8 + (size_t)lb * dm.cap8;
  const float* ema8 = c.ema8 + (size_t)lb * dm.cap8;
  const int32_t* pos16 = c.pos16 + (size_t)lb * dm.cap16;
  const float* ema16 = c.ema16 + (size_t)lb * dm.cap16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (n <= N) {
    for (int j = tid; j < n8; j += kSelThreads) keep8[j] = 1;
    for (int j = tid; j < n16; j += kSelThreads) keep16[j] = 1;
    return;
  }
  __shared__ uint64_t s_key[kSelLdsKeys];
  __shared__ unsigned hist[256];
  __shared__ float s_wmax[kSelThreads / 64];
  __shared__ int s_wprot[kSelThreads / 64];
  __shared__ unsigned long long s_prefix, s_mask;
  __shared__ unsigned long long s_wmin[kSelThreads / 64];
  __shared__ int s_rem, s_done;
  const int prot_lo = t - dm.P;  // protected: pos > prot_lo
  const bool cached = n <= kSelLdsKeys;
  auto tok = [&](int j, float& e, int& p) {
    if (j < n8) {
      e = ema8[j];
      p = pos8[j];
    } else {
      e = ema16[j - n8];
      p = pos16[j - n8];
    }
  };
  // e_max over every cached token and the protected count
  float emax = 0.f;
  int nprot = 0;
  for (int j = tid; j < n; j += kSelThreads) {
    float e;
    int p;
    tok(j, e, p);
    emax = fmaxf(emax, e);
    nprot += p > prot_lo;
  }
  for (int off = 32; off > 0; off >>= 1) {
    emax = fmaxf(emax, __shfl_xor(emax, off));
    nprot += __shfl_xor(nprot, off);
  }
  if (lane == 0) {
    s_wmax[wave] = emax;
    s_wprot[wave] = nprot;
  }
  __syncthreads();
  float em = 0.f;
  int np = 0;
  for (int w = 0; w < kSelThreads / 64; ++w) {
    em = fmaxf(em, s_wmax[w]);
    np += s_wprot[w];
  }
  int K = N - np;
  if (K < 0) K = 0;
  // candidate keys; protected tokens get key 0, which no candidate can have
  // (pos + 1 > 0 is folded in below so that 0 stays reserved)
  auto key_of = [&](int j) -> uint64_t {
    float e;
    int p;
    tok(j, e, p);
    if (p > prot_lo) return 0ull;
    return sel_key(e, em, p, t, dm.s_ema, dm.s_rec) + 1ull;
  };
  if (cached)
    for (int j = tid; j < n; j += kSelThreads) s_key[j] = key_of(j);
  const int evict = (n - np) - K;  // candidates that go
  if (K > 0 && evict <= kFewEvict) {
    // the evict smallest candidate keys (keys are unique): after round e, thr is
    // the (e+1)-th smallest; the candidates above the last thr stay
    if (cached) __syncthreads();
    uint64_t thr = 0ull;
    for (int e = 0; e < evict; ++e) {
      uint64_t m = ~0ull;
      for (int j = tid; j < n; j += kSelThreads) {
        const uint64_t key = cached ? s_key[j] : key_of(j);
        if (key > thr && key < m) m = key;  // key 0 (protected) is never > thr
      }
      m = wave_min_u64(m);
      if (lane == 0) s_wmin[wave] = m;
      __syncthreads();
      m = s_wmin[0];
      for (int w = 1; w < kSelThreads / 64; ++w) m = s_wmin[w] < m ? s_wmin[w] : m;
      thr = m;
      __syncthreads();
    }
    for (int j = tid; j < n; j += kSelThreads) {
      const uint64_t key = cached ? s_key[j] : key_of(j);
      const int k = key == 0ull ? 1 : key > thr;
      if (j < n8)
        keep8[j] = (uint8_t)k;
      else
        keep16[j - n8] = (uint8_t)k;
    }
    return;
  }
  if (tid == 0) {
    s_prefix = 0ull;
    s_mask = 0ull;
    s_rem = K;
    s_done = K == 0;
  }
  __syncthreads();
  for (int shift = 56; shift >= 0 && !s_done; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    const unsigned long long pre = s_prefix, msk = s_mask;
    for (int j = tid; j < n; j += kSelThreads) {
      const uint64_t key = cached ? s_key[j] : key_of(j);
      if (key != 0ull && (key & msk) == pre) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l covers bins 255-4l .. 252-4l; suffix sums from the top bin down
      unsigned hb[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hb[i] = hist[255 - 4 * lane - i];
        sum += hb[i];
      }
      unsigned incl = sum;
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      const unsigned excl = incl - sum;
      const unsigned rem = (unsigned)s_rem;
      if (excl < rem && rem <= incl) {
        unsigned cum = excl;
        int d = 255 - 4 * lane - 3;
        unsigned cnt = hb[3];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (cum + hb[i] >= rem) {
            d = 255 - 4 * lane - i;
            cnt = hb[i];
            break;
          }
          cum += hb[i];
        }
        const int rem2 = (int)(rem - cum);
        s_prefix = pre | ((unsigned long long)d << shift);
        s_mask = msk | (0xFFull << shift);
        s_rem = rem2;
        s_done = (rem2 == (int)cnt) || shift == 0;  // the whole bin is kept
      }
    }
    __syncthreads();
  }
  // keep every candidate whose key is >= the threshold prefix (its undecided low
  // bits at zero); when K = 0 no candidate is kept
  const unsigned long long kth = s_prefix;
  for (int j = tid; j < n; j += kSelThreads) {
    const uint64_t key = cached ? s_key[j] : key_of(j);
    const int k = key == 0ull ? 1 : (K > 0 && key >= kth);
    if (j < n8)
      keep8[j] = (uint8_t)k;
    else
      keep16[j - n8] = (uint8_t)k;
  }
}

void launch_select(const Dims& dm, const conf_cache& c, int layer0, int nl, const int32_t* budget,
                   uint8_t* keep, hipStream_t st) {
  hipLaunchKernelGGL(select_kernel, dim3(nl * dm.B), dim3(kSelThreads), 0, st, c, dm, layer0,
                     budget, keep);
}

}  // namespace confkv
