// (b)+(c) Decode attention over the mixed-precision cache, and the per-token
// attention mass that feeds the EMA.
//
// CONF-KV explainer, Key contributions (system design): block-wise online-
// softmax attention; Methodology, implementation: dequantisation fused into the
// block-wise attention reads over a dense (compacted) layout; mixed-precision
// storage: INT8 codes with one scale per (KV head, channel), so the key scale
// folds into the query and the value scale into the output.
//
// One workgroup per unit (layer, sequence, KV head) covers the g = Hq/Hkv query
// heads that share the unit's keys and values, over n = n8 INT8 tokens followed by
// the n16 window tokens (the appended token is the last window slot).
#include "common.hpp"

namespace confkv {

constexpr int kAttnThreads = 256;

// ---------------------------------------------------------------------------
// Reference-structured kernel: two passes over the keys (pass A: per-head
// log-sum-exp; pass B: probabilities, token mass and the value sum).  Used for
// every shape the matrix-core kernel does not take.
// ---------------------------------------------------------------------------
template <int D>
__device__ inline void key_dot(const Dims& dm, int j, int n8, const int8_t* k8, const uint16_t* k16,
                               const float (*q8)[D], const float (*qw)[D], float* sig) {
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) sig[h] = 0.f;
  if (j < n8) {
    const int8_t* row = k8 + (size_t)j * D;
    for (int c0 = 0; c0 < D; c0 += 16) {
      const int4 v = *(const int4*)(row + c0);
      const int8_t* bytes = (const int8_t*)&v;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = (float)bytes[i];
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h)
          if (h < dm.G) sig[h] = fmaf(q8[h][c0 + i], x, sig[h]);
      }
    }
  } else {
    const uint16_t* row = k16 + (size_t)(j - n8) * D;
    for (int c0 = 0; c0 < D; c0 += 8) {
      const int4 v = *(const int4*)(row + c0);
      const uint16_t* hs = (const uint16_t*)&v;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = h16_to_f32(hs[i], dm.bf16);
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h)
          if (h < dm.G) sig[h] = fmaf(qw[h][c0 + i], x, sig[h]);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_ref_kernel(conf_cache c, Dims dm, int layer0,
                                                                const uint16_t* __restrict__ q_all,
                                                                float* __restrict__ out_all,
                                                                float* __restrict__ massp_all) {
  const int unit_local = blockIdx.x;
  const int hk = unit_local % dm.Hkv;
  const int lbl = unit_local / dm.Hkv;
  const int lb = layer0 * dm.B + lbl;
  const size_t u = (size_t)lb * dm.Hkv + hk;
  const int tid = threadIdx.x;
  const int G = dm.G;
  const int n8 = c.n8[lb];
  const int n16 = min(c.n16[lb] + 1, dm.cap16);
  const int n = n8 + n16;
  const int8_t* k8 = c.k8 + u * (size_t)dm.cap8 * D;
  const int8_t* v8 = c.v8 + u * (size_t)dm.cap8 * D;
  const uint16_t* k16 = (const uint16_t*)c.k16 + u * (size_t)dm.cap16 * D;
  const uint16_t* v16 = (const uint16_t*)c.v16 + u * (size_t)dm.cap16 * D;

  __shared__ float qw[kMaxGroup][D];
  __shared__ float q8[kMaxGroup][D];
  __shared__ float sv[D];
  __shared__ float lse[kMaxGroup];
  __shared__ float pch[kMaxGroup][kAttnThreads];
  __shared__ float redm[kAttnThreads / 64][kMaxGroup], reds[kAttnThreads / 64][kMaxGroup];

  const float rs = 1.0f / sqrtf((float)D);
  const uint16_t* qsrc = q_all + ((size_t)lbl * dm.Hq + (size_t)hk * G) * D;
  for (int i = tid; i < G * D; i += kAttnThreads) {
    const int h = i / D, ch = i % D;
    const float qv = h16_to_f32(qsrc[i], dm.bf16) * rs;
    qw[h][ch] = qv;
    q8[h][ch] = qv * (c.k_amax[u * D + ch] / 127.0f);
  }
  for (int ch = tid; ch < D; ch += kAttnThreads) sv[ch] = c.v_amax[u * D + ch] / 127.0f;
  __syncthreads();

  // pass A: running (max, sum) per head and thread
  float m[kMaxGroup], s[kMaxGroup], sig[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    m[h] = -INFINITY;
    s[h] = 0.f;
  }
  for (int j = tid; j < n; j += kAttnThreads) {
    key_dot<D>(dm, j, n8, k8, k16, q8, qw, sig);
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h < G) {
        if (sig[h] > m[h]) {
          s[h] = s[h] * expf(m[h] - sig[h]) + 1.0f;
          m[h] = sig[h];
        } else {
          s[h] += expf(sig[h] - m[h]);
        }
      }
    }
  }
  // reduce (max, sum) pairs: wave shuffles, then across waves
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h < G) {
      for (int off = 32; off > 0; off >>= 1) {
        const float om = __shfl_xor(m[h], off), os = __shfl_xor(s[h], off);
        const float M = fmaxf(m[h], om);
        float S = 0.f;
        if (m[h] > -INFINITY) S += s[h] * expf(m[h] - M);
        if (om > -INFINITY) S += os * expf(om - M);
        m[h] = M;
        s[h] = S;
      }
      if ((tid & 63) == 0) {
        redm[tid >> 6][h] = m[h];
        reds[tid >> 6][h] = s[h];
      }
    }
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int w = 0; w < kAttnThreads / 64; ++w) M = fmaxf(M, redm[w][tid]);
    float S = 0.f;
    for (int w = 0; w < kAttnThreads / 64; ++w)
      if (redm[w][tid] > -INFINITY) S += reds[w][tid] * expf(redm[w][tid] - M);
    lse[tid] = M + logf(S);
  }
  __syncthreads();

  // pass B: probabilities, mass and the value sums
  constexpr int kPer = (kMaxGroup * D + kAttnThreads - 1) / kAttnThreads;
  float acc8[kPer], acc16[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    acc8[r] = 0.f;
    acc16[r] = 0.f;
  }
  float* massp = massp_all + u * (size_t)dm.capt;
  for (int base = 0; base < n; base += kAttnThreads) {
    const int j = base + tid;
    if (j < n) {
      key_dot<D>(dm, j, n8, k8, k16, q8, qw, sig);
      float mass = 0.f;
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) {
        if (h < G) {
          const float p = expf(sig[h] - lse[h]);
          pch[h][tid] = p;
          mass += p;
        }
      }
      massp[j < n8 ? j : dm.cap8 + (j - n8)] = mass;
    } else {
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h)
        if (h < G) pch[h][tid] = 0.f;
    }
    __syncthreads();
    const int cnt = min(kAttnThreads, n - base);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int idx = tid + r * kAttnThreads;
      if (idx < G * D) {
        const int h = idx / D, ch = idx % D;
        float a8 = acc8[r], a16 = acc16[r];
        for (int jj = 0; jj < cnt; ++jj) {
          const int tok = base + jj;
          const float p = pch[h][jj];
          if (tok < n8)
            a8 = fmaf(p, (float)v8[vtile_off(tok, ch, D)], a8);
          else
            a16 = fmaf(p, h16_to_f32(v16[vtile_off(tok - n8, ch, D)], dm.bf16), a16);
        }
        acc8[r] = a8;
        acc16[r] = a16;
      }
    }
    __syncthreads();
  }
  float* out = out_all + ((size_t)lbl * dm.Hq + (size_t)hk * G) * D;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int idx = tid + r * kAttnThreads;
    if (idx < G * D) {
      const int ch = idx % D;
      out[idx] = fmaf(acc8[r], sv[ch], acc16[r]);
    }
  }
}

void launch_attn(const Dims& dm, const conf_cache& c, int layer0, int nl, const void* q, float* out,
                 float* massp, hipStream_t st) {
  const dim3 grid(nl * dm.B * dm.Hkv);
  if (dm.D == 64)
    hipLaunchKernelGGL(attn_ref_kernel<64>, grid, dim3(kAttnThreads), 0, st, c, dm, layer0,
                       (const uint16_t*)q, out, massp);
  else
    hipLaunchKernelGGL(attn_ref_kernel<128>, grid, dim3(kAttnThreads), 0, st, c, dm, layer0,
                       (const uint16_t*)q, out, massp);
}

}  // namespace confkv
