// (c) EMA of per-token attention mass, as a device routine shared by the EMA
// kernel that follows the attention and by the fused EMA + selection +
// compaction kernel.
//
// CONF-KV explainer, Methodology, token ranking and eviction: each token keeps an
// exponential moving average of the attention mass it receives.
#pragma once

#include "common.hpp"

namespace confkv {

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
