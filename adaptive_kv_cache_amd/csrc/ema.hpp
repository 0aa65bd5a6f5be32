// (c) EMA of per-token attention mass, as a device routine shared by the EMA
// kernel that follows the attention and by the fused EMA + selection +
// compaction kernel.
//
// CONF-KV explainer, Methodology, token ranking and eviction: each token keeps an
// exponential moving average of the attention mass it receives.
#pragma once

#include "common.hpp"

namespace confkv {

// ARKV's heavy-hitter score of a token [the ARKV page, Methodology: decoding-phase
// token ranking] from a = sum over the KV heads of its mass rows (each the sum of
// the head's G query heads' probabilities) and a2 = the sum of their squares,
// both in KV-head order: with m_k = row_k / G,
//   mean_k m_k + max(mean_k m_k^2 - (mean_k m_k)^2, 0),
// fp32, one rounding per operation.
__device__ inline float arkv_h(float a, float a2, const Dims& dm) {
#pragma clang fp contract(off)
  const float mean = a / (float)dm.Hq;
  const float gg_h = (float)dm.G * (float)dm.G * (float)dm.Hkv;
  const float var = fmaxf(a2 / gg_h - mean * mean, 0.f);
  return mean + var;
}

// ARKV's score EMA in the layout of ema_tokens below (same threads and tokens).
__device__ inline void arkv_tokens(const conf_cache& c, const Dims& dm, int lb,
                                   const float* __restrict__ massp_all, int n8, int nw, int t,
                                   int j0, int jstep) {
#pragma clang fp contract(off)
  const int appended = nw < dm.cap16;
  const int end = n8 + nw + appended;
  const float* rows = massp_all + (size_t)lb * dm.Hkv * dm.capt;
  float* ema8 = c.ema8 + (size_t)lb * dm.cap8;
  float* ema16 = c.ema16 + (size_t)lb * dm.cap16;
  for (int j = j0; j < end; j += jstep) {
    const int idx = j < n8 ? j : dm.cap8 + (j - n8);
    float a = 0.f, a2 = 0.f;
    for (int hk = 0; hk < dm.Hkv; ++hk) {
      const float r = rows[(size_t)hk * dm.capt + idx];
      a += r;
      a2 += r * r;
    }
    const float h = arkv_h(a, a2, dm);
    if (j < n8) {
      ema8[j] = dm.decay * ema8[j] + dm.one_minus_decay * h;
    } else if (j - n8 == nw) {
      ema16[nw] = dm.one_minus_decay * h;  // decay * 0 + (1 - decay) * h
      c.pos16[(size_t)lb * dm.cap16 + nw] = t + 1;
    } else {
      ema16[j - n8] = dm.decay * ema16[j - n8] + dm.one_minus_decay * h;
    }
  }
}

// EMA of the tokens of (layer, sequence) lb once every KV head's mass row is in
// massp: mass_j = (sum of the KV heads' rows, in index order) / Hq and
// e <- decay*e + (1-decay)*mass; the appended token (window slot nw, if the
// window had room) starts from e = 0 and takes position t+1.  (n8, nw, t) are
// the sizes before this step's append.  A thread takes tokens j0, j0 + jstep, ...
// The baseline policies keep no EMA: only the appended token's slot is set (EMA 0,
// position t+1), by the thread with j0 = 0.
__device__ inline void ema_tokens(const conf_cache& c, const Dims& dm, int lb,
                                  const float* __restrict__ massp_all, int n8, int nw, int t,
                                  int j0, int jstep) {
#pragma clang fp contract(off)
  const int appended = nw < dm.cap16;
  if (dm.policy == CONF_POLICY_ARKV) {
    arkv_tokens(c, dm, lb, massp_all, n8, nw, t, j0, jstep);
    return;
  }
  if (dm.policy != CONF_POLICY_CONFKV) {  // no EMA: the appended token's slot only
    if (j0 == 0 && appended) {
      c.ema16[(size_t)lb * dm.cap16 + nw] = 0.f;
      c.pos16[(size_t)lb * dm.cap16 + nw] = t + 1;
    }
    return;
  }
  const int end = n8 + nw + appended;
  const float* rows = massp_all + (size_t)lb * dm.Hkv * dm.capt;
  float* ema8 = c.ema8 + (size_t)lb * dm.cap8;
  float* ema16 = c.ema16 + (size_t)lb * dm.cap16;
  const float hq = (float)dm.Hq;
  // kT tokens per thread per round, every load of the round issued before the
  // arithmetic (a token past the end reads slot 0 and is not stored)
  constexpr int kT = 4;
  for (int jb = j0; jb < end; jb += kT * jstep) {
    int idx[kT];
    float a[kT], eo[kT];
#pragma unroll
    for (int k = 0; k < kT; ++k) {
      const int j = jb + k * jstep;
      idx[k] = j >= end ? 0 : j < n8 ? j : dm.cap8 + (j - n8);
      a[k] = 0.f;
    }
#pragma unroll 8
    for (int hk = 0; hk < dm.Hkv; ++hk)
#pragma unroll
      for (int k = 0; k < kT; ++k) a[k] += rows[(size_t)hk * dm.capt + idx[k]];
#pragma unroll
    for (int k = 0; k < kT; ++k) {
      const int j = jb + k * jstep;
      eo[k] = j < n8 ? ema8[idx[k]] : ema16[j >= end ? 0 : j - n8];
    }
#pragma unroll
    for (int k = 0; k < kT; ++k) {
      const int j = jb + k * jstep;
      if (j >= end) continue;
      const float m = a[k] / hq;
      if (j < n8) {
        ema8[j] = dm.decay * eo[k] + dm.one_minus_decay * m;
      } else if (j - n8 == nw) {
        ema16[nw] = dm.one_minus_decay * m;  // decay * 0 + (1 - decay) * mass
        c.pos16[(size_t)lb * dm.cap16 + nw] = t + 1;
      } else {
        ema16[j - n8] = dm.decay * eo[k] + dm.one_minus_decay * m;
      }
    }
  }
}

}  // namespace confkv
