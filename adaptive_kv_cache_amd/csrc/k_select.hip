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
// MSB-first radix select (8 passes of 8 bits) with a 256-bin histogram in LDS;
// every candidate whose key is >= it is kept.
#include "common.hpp"

namespace confkv {

constexpr int kSelThreads = 256;

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
  const int tid = threadIdx.x;
  if (n <= N) {
    for (int j = tid; j < n8; j += kSelThreads) keep8[j] = 1;
    for (int j = tid; j < n16; j += kSelThreads) keep16[j] = 1;
    return;
  }
  __shared__ unsigned hist[256];
  __shared__ float s_emax;
  __shared__ int s_nprot;
  __shared__ unsigned long long s_prefix, s_mask;
  __shared__ int s_rem;
  const int prot_lo = t - dm.P;  // protected: pos > prot_lo
  float emax = 0.f;
  int nprot = 0;
  for (int j = tid; j < n; j += kSelThreads) {
    const float e = j < n8 ? ema8[j] : ema16[j - n8];
    const int p = j < n8 ? pos8[j] : pos16[j - n8];
    emax = fmaxf(emax, e);
    nprot += p > prot_lo;
  }
  for (int off = 32; off > 0; off >>= 1) {
    emax = fmaxf(emax, __shfl_xor(emax, off));
    nprot += __shfl_xor(nprot, off);
  }
  if (tid == 0) {
    s_emax = 0.f;
    s_nprot = 0;
    s_prefix = 0ull;
    s_mask = 0ull;
  }
  __syncthreads();
  if ((tid & 63) == 0) {
    atomicMax((unsigned*)&s_emax, __float_as_uint(emax));  // e >= 0: bits order like values
    atomicAdd(&s_nprot, nprot);
  }
  __syncthreads();
  const float em = s_emax;
  int K = N - s_nprot;
  if (K < 0) K = 0;
  if (tid == 0) s_rem = K;
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[tid] = 0u;
    __syncthreads();
    const unsigned long long pre = s_prefix, msk = s_mask;
    for (int j = tid; j < n; j += kSelThreads) {
      const int p = j < n8 ? pos8[j] : pos16[j - n8];
      if (p > prot_lo) continue;
      const float e = j < n8 ? ema8[j] : ema16[j - n8];
      const uint64_t key = sel_key(e, em, p, t, dm.s_ema, dm.s_rec);
      if ((key & msk) == pre) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int rem = s_rem;
      unsigned cum = 0;
      int d = 255;
      for (; d > 0; --d) {
        if ((int)(cum + hist[d]) >= rem) break;
        cum += hist[d];
      }
      s_rem = rem - (int)cum;
      s_prefix = pre | ((unsigned long long)d << shift);
      s_mask = msk | (0xFFull << shift);
    }
    __syncthreads();
  }
  const unsigned long long kth = s_prefix;
  for (int j = tid; j < n; j += kSelThreads) {
    const int p = j < n8 ? pos8[j] : pos16[j - n8];
    int k = 1;
    if (p <= prot_lo) {
      if (K == 0) {
        k = 0;
      } else {
        const float e = j < n8 ? ema8[j] : ema16[j - n8];
        k = sel_key(e, em, p, t, dm.s_ema, dm.s_rec) >= kth;
      }
    }
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
