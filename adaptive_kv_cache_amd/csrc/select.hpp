// (d) Rank and select, as a workgroup-wide device routine shared by the
// selection kernel and the fused selection + compaction kernel.
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
#pragma once

#include "common.hpp"

namespace confkv {

constexpr int kSelLdsKeys = 5632;  // keys cached in LDS (44 KB)
constexpr int kFewEvict = 8;       // evictions up to which minimum rounds replace the radix select
constexpr uint64_t kAllKept = ~0ull;  // sink key of a token kept without ranking (n <= N)

struct SelScratch {
  uint64_t key[kSelLdsKeys];
  unsigned hist[256];
};
struct SelMisc {
  float wmax[16];
  int wprot[16];
  unsigned long long wmin[16];
  unsigned long long prefix, mask;
  int rem, done;
};

__device__ inline uint64_t wave_min_u64(uint64_t x) {
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)x, off), hi = __shfl_xor((uint32_t)(x >> 32), off);
    const uint64_t y = ((uint64_t)hi << 32) | lo;
    x = y < x ? y : x;
  }
  return x;
}

// Retention key (CONF_POLICY_TRIM): s = (t - pos) * ln(beta) <= 0, one float32
// product, 0 for the newest token.  For m = -s >= 0 (with -0 made +0) the bits of
// m order like m, so ~bits(m) orders like s; with the position below it the key
// orders as (s desc, pos desc).
__device__ inline uint64_t retention_key(float log_beta, int pos, int t) {
#pragma clang fp contract(off)
  float m = 0.f;
  if (t != pos) m = -((float)(t - pos) * log_beta);
  const uint32_t bits = m == 0.f ? 0u : __float_as_uint(m);
  return ((uint64_t)~bits << 32) | (uint32_t)pos;
}

__device__ inline uint64_t sel_key(float e, float emax, int pos, int t, float s_ema, float s_rec,
                                   uint32_t tag) {
#pragma clang fp contract(off)
  const float ehat = emax > 0.f ? e / emax : 0.f;
  const float r = t > 0 ? (float)pos / (float)t : 1.0f;
  const float a = s_ema * ehat;
  const float b = s_rec * r;
  const float s = a + b;
  return ((uint64_t)__float_as_uint(s) << 32) | tag;
}

// The ranking shared by the per-sequence and the head-wise selection.  Tokens
// j < n each have (e, tag) from tok(j, e, tag); tag is the token's position, or
// in the head-wise (JOINT) form position * hw + head, so that the low key word
// is unique among the n tokens.  A token is protected when its position is
// above prot_lo.  keyf(e, e_max, tag) gives a candidate's 64-bit key; larger
// keys are kept first.  Keeps the protected tokens and the N - |protected|
// candidates with the largest keys, and calls sink(j, keep, key) once per j
// with key = the candidate's key + 1, 0 for a protected token (or kAllKept when
// n <= N and nothing is ranked).  The keys live in LDS (keys[key_cap], beside
// a 256-bin histogram) when n <= key_cap; otherwise each pass recomputes them.
// With PAIRS and use_pairs, keys[j] already holds (bits(e) << 32 | tag) for
// every j, written by thread j mod NT, whenever n <= key_cap.
template <int NT, bool PAIRS, bool JOINT, typename Tok, typename KeyFn, typename Sink>
__device__ void rank_core(int n, int N, int prot_lo, int hw, bool use_pairs, Tok tok, KeyFn keyf,
                          uint64_t* keys, unsigned* hist, int key_cap, SelMisc& M, Sink sink) {
  constexpr int kWaves = NT / 64;
  static_assert(kWaves <= 16, "SelMisc holds 16 wavefronts");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (n <= N) {
    for (int j = tid; j < n; j += NT) sink(j, 1, kAllKept);
    return;
  }
  auto pos_of = [&](uint32_t tag) -> int { return JOINT ? (int)(tag / (uint32_t)hw) : (int)tag; };
  const bool cached = n <= key_cap;
  // e_max over every token and the protected count; with the keys in LDS the
  // (e, tag) pairs wait there for the key pass (same thread, same index)
  float emax = 0.f;
  int nprot = 0;
  for (int j = tid; j < n; j += NT) {
    float e;
    uint32_t tag;
    if (PAIRS && cached && use_pairs) {
      const uint64_t v = keys[j];
      e = __uint_as_float((uint32_t)(v >> 32));
      tag = (uint32_t)v;
    } else {
      tok(j, e, tag);
      if (cached) keys[j] = ((uint64_t)__float_as_uint(e) << 32) | tag;
    }
    emax = fmaxf(emax, e);
    nprot += pos_of(tag) > prot_lo;
  }
  for (int off = 32; off > 0; off >>= 1) {
    emax = fmaxf(emax, __shfl_xor(emax, off));
    nprot += __shfl_xor(nprot, off);
  }
  if (lane == 0) {
    M.wmax[wave] = emax;
    M.wprot[wave] = nprot;
  }
  __syncthreads();
  float em = 0.f;
  int np = 0;
  for (int w = 0; w < kWaves; ++w) {
    em = fmaxf(em, M.wmax[w]);
    np += M.wprot[w];
  }
  int K = N - np;
  if (K < 0) K = 0;
  // candidate keys; protected tokens get key 0, which no candidate can have
  auto key_from = [&](float e, uint32_t tag) -> uint64_t {
    if (pos_of(tag) > prot_lo) return 0ull;
    return keyf(e, em, tag) + 1ull;
  };
  auto key_of = [&](int j) -> uint64_t {
    float e;
    uint32_t tag;
    tok(j, e, tag);
    return key_from(e, tag);
  };
  if (cached)
    for (int j = tid; j < n; j += NT) {
      const uint64_t v = keys[j];
      keys[j] = key_from(__uint_as_float((uint32_t)(v >> 32)), (uint32_t)v);
    }
  const int evict = (n - np) - K;  // candidates that go
  if (K > 0 && evict <= kFewEvict) {
    // the evict smallest candidate keys (keys are unique): after round e, thr is
    // the (e+1)-th smallest; the candidates above the last thr stay
    if (cached) __syncthreads();
    uint64_t thr = 0ull;
    for (int e = 0; e < evict; ++e) {
      uint64_t m = ~0ull;
      for (int j = tid; j < n; j += NT) {
        const uint64_t key = cached ? keys[j] : key_of(j);
        if (key > thr && key < m) m = key;  // key 0 (protected) is never > thr
      }
      m = wave_min_u64(m);
      if (lane == 0) M.wmin[wave] = m;
      __syncthreads();
      m = M.wmin[0];
      for (int w = 1; w < kWaves; ++w) m = M.wmin[w] < m ? M.wmin[w] : m;
      thr = m;
      __syncthreads();
    }
    for (int j = tid; j < n; j += NT) {
      const uint64_t key = cached ? keys[j] : key_of(j);
      sink(j, key == 0ull ? 1 : key > thr, key);
    }
    return;
  }
  if (tid == 0) {
    M.prefix = 0ull;
    M.mask = 0ull;
    M.rem = K;
    M.done = K == 0;
  }
  __syncthreads();
  for (int shift = 56; shift >= 0 && !M.done; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    const unsigned long long pre = M.prefix, msk = M.mask;
    for (int j = tid; j < n; j += NT) {
      const uint64_t key = cached ? keys[j] : key_of(j);
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
      const unsigned rem = (unsigned)M.rem;
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
        M.prefix = pre | ((unsigned long long)d << shift);
        M.mask = msk | (0xFFull << shift);
        M.rem = rem2;
        M.done = (rem2 == (int)cnt) || shift == 0;  // the whole bin is kept
      }
    }
    __syncthreads();
  }
  // keep every candidate whose key is >= the threshold prefix (its undecided low
  // bits at zero); when K = 0 no candidate is kept
  const unsigned long long kth = M.prefix;
  for (int j = tid; j < n; j += NT) {
    const uint64_t key = cached ? keys[j] : key_of(j);
    sink(j, key == 0ull ? 1 : (K > 0 && key >= kth), key);
  }
}

// Keep flags of one (layer, sequence) with n8 INT8 and n16 window tokens and
// budget N, over the index space j < n8 (INT8 slot j), j >= n8 (window slot
// j - n8).  Calls sink(j, keep, key) exactly once per index; key is the token's
// key + 1 (so a candidate's is never 0), 0 for a protected token, or kAllKept
// when n <= N and nothing is ranked.  All NT threads of the workgroup must call
// it; the sink calls are the last thing it does (no barrier follows them).
// With PAIRS, the caller has left each token's (bits(e) << 32 | pos) in X.key[j]
// whenever n8 + n16 <= kSelLdsKeys, written by the thread that owns j here
// (j mod NT), so the first pass reads no memory.
template <int NT, bool PAIRS = false, typename Sink>
__device__ void select_core(const conf_cache& c, const Dims& dm, int lb, int n8, int n16, int t,
                            int N, SelScratch& X, SelMisc& M, Sink sink) {
  const int n = n8 + n16;
  const int tid = threadIdx.x;
  const int32_t* pos8 = c.pos8 + (size_t)lb * dm.cap8;
  const float* ema8 = c.ema8 + (size_t)lb * dm.cap8;
  const int32_t* pos16 = c.pos16 + (size_t)lb * dm.cap16;
  const float* ema16 = c.ema16 + (size_t)lb * dm.cap16;
  // the sliding window keeps the newest W positions, (t-W, t], whatever the budget
  if (dm.policy == CONF_POLICY_WINDOW) {
    for (int j = tid; j < n; j += NT)
      sink(j, (j < n8 ? pos8[j] : pos16[j - n8]) > t - dm.W, kAllKept);
    return;
  }
  // full KV keeps everything, as CONF-KV does under its budget
  if (n <= N || dm.policy == CONF_POLICY_FULL) {
    for (int j = tid; j < n; j += NT) sink(j, 1, kAllKept);
    return;
  }
  auto tok = [&](int j, float& e, uint32_t& tag) {
    if (j < n8) {
      e = ema8[j];
      tag = (uint32_t)pos8[j];
    } else {
      e = ema16[j - n8];
      tag = (uint32_t)pos16[j - n8];
    }
  };
  const bool trim = dm.policy == CONF_POLICY_TRIM;
  const bool arkv = dm.policy == CONF_POLICY_ARKV;
  auto keyf = [&](float e, float em, uint32_t tag) -> uint64_t {
    if (trim) return retention_key(e, (int)tag, t);
    // ARKV ranks on its heavy-hitter EMA itself (e >= 0 orders like its bits)
    if (arkv) return ((uint64_t)__float_as_uint(e) << 32) | tag;
    return sel_key(e, em, (int)tag, t, dm.s_ema, dm.s_rec, tag);
  };
  rank_core<NT, PAIRS, false>(n, N, t - dm.P, 1, !trim, tok, keyf, X.key, X.hist, kSelLdsKeys, M,
                              sink);
}

}  // namespace confkv
