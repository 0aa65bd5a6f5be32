// (b)+(c) Decode attention over the mixed-precision cache, the per-token
// attention mass, and the EMA update, in one launch.
//
// CONF-KV explainer, Key contributions (system design): block-wise online-
// softmax attention; Methodology, implementation: dequantisation fused into the
// block-wise attention reads over a dense (compacted) layout; mixed-precision
// storage: INT8 codes with one scale per (KV head, channel), so the key scale
// folds into the query and the value scale into the output; token ranking: the
// EMA of each token's attention mass.
//
// One workgroup per unit (layer, sequence, KV head) covers the g = Hq/Hkv query
// heads sharing the unit's keys and values, over the n8 INT8 tokens, the window
// tokens and this step's token (read from the caller's k_new / v_new rows and
// also appended to the window).  Each unit writes the mass of its g heads per
// token; the last unit of a (layer, sequence) to arrive (arrival counter, device-
// scope fences) sums the KV heads in index order and applies the EMA.
#include "common.hpp"

namespace confkv {

constexpr int kAttnThreads = 256;

// Token view of one unit for this step: INT8 slots [0, n8), window slots
// [0, nw), then the new token (index n8 + nw) if it was appended.
struct UnitView {
  const int8_t* k8;
  const int8_t* v8;
  const uint16_t* k16;
  const uint16_t* v16;
  const uint16_t* knew;  // [D] row of this step's key
  const uint16_t* vnew;  // [D] row of this step's value
  int n8, nw, n;         // n = n8 + nw + appended
};

// Appends this step's key/value to window slot `slot` of the unit (data only).
__device__ inline void append_row(const Dims& dm, uint16_t* k16, uint16_t* v16, int slot,
                                  const uint16_t* knew, const uint16_t* vnew) {
  for (int ch = threadIdx.x; ch < dm.D; ch += blockDim.x) {
    k16[(size_t)slot * dm.D + ch] = knew[ch];
    v16[vtile_off(slot, ch, dm.D)] = vnew[ch];
  }
}

// EMA of one (layer, sequence) from the per-KV-head mass rows, run by the last
// unit to arrive.  mass_j = (sum over KV heads, in index order) / Hq;
// e <- decay*e + (1-decay)*mass; the appended token starts from e = 0 and takes
// position t+1; then n16 and t advance.
__device__ void ema_update_lb(const conf_cache& c, const Dims& dm, int lb, int n8, int nw,
                              int appended, int t, const float* mp) {
#pragma clang fp contract(off)
  const float hq = (float)dm.Hq;
  for (int j = threadIdx.x; j < n8 + nw + appended; j += blockDim.x) {
    const int idx = j < n8 ? j : dm.cap8 + (j - n8);
    float a = 0.f;
    for (int hk = 0; hk < dm.Hkv; ++hk) a += mp[(size_t)hk * dm.capt + idx];
    a = a / hq;
    if (j < n8) {
      float* e = c.ema8 + (size_t)lb * dm.cap8 + j;
      *e = dm.decay * (*e) + dm.one_minus_decay * a;
    } else {
      const int w = j - n8;
      float* e = c.ema16 + (size_t)lb * dm.cap16 + w;
      if (w == nw) {
        *e = dm.one_minus_decay * a;  // decay * 0 + (1 - decay) * mass
        c.pos16[(size_t)lb * dm.cap16 + w] = t + 1;
      } else {
        *e = dm.decay * (*e) + dm.one_minus_decay * a;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    c.n16[lb] = nw + appended;
    c.t[lb] = t + 1;
    c.arrive[lb] = 0;
  }
}

// Arrival protocol: every thread's mass stores are fenced at device scope
// before thread 0 counts the unit in; the unit that completes the count fences
// again (acquire) and runs the EMA for the (layer, sequence).
__device__ inline bool arrive_last(const conf_cache& c, const Dims& dm, int lb) {
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(c.arrive + lb, 1);
    s_last = prev == dm.Hkv - 1;
  }
  __syncthreads();
  const bool last = s_last != 0;
  if (last) __threadfence();
  return last;
}

// ---------------------------------------------------------------------------
// Two-pass kernel (pass A: per-head log-sum-exp; pass B: probabilities, token
// mass and the value sum), vector ALU only.
// ---------------------------------------------------------------------------
template <int D>
__device__ inline void key_dot(const Dims& dm, const UnitView& uv, int j, const float (*q8)[D],
                               const float (*qw)[D], float* sig) {
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) sig[h] = 0.f;
  if (j < uv.n8) {
    const int8_t* row = uv.k8 + (size_t)j * D;
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
    const uint16_t* row = (j - uv.n8 < uv.nw) ? uv.k16 + (size_t)(j - uv.n8) * D : uv.knew;
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
                                                                const uint16_t* __restrict__ knew_all,
                                                                const uint16_t* __restrict__ vnew_all,
                                                                float* __restrict__ out_all,
                                                                float* __restrict__ massp_all) {
  const int unit_local = blockIdx.x;
  const int hk = unit_local % dm.Hkv;
  const int lbl = unit_local / dm.Hkv;
  const int lb = layer0 * dm.B + lbl;
  const size_t u = (size_t)lb * dm.Hkv + hk;
  const int tid = threadIdx.x;
  const int G = dm.G;
  const int n8 = c.n8[lb], nw = c.n16[lb], t = c.t[lb];
  const int appended = nw < dm.cap16;
  UnitView uv;
  uv.k8 = c.k8 + u * (size_t)dm.cap8 * D;
  uv.v8 = c.v8 + u * (size_t)dm.cap8 * D;
  uv.k16 = (const uint16_t*)c.k16 + u * (size_t)dm.cap16 * D;
  uv.v16 = (const uint16_t*)c.v16 + u * (size_t)dm.cap16 * D;
  uv.knew = knew_all + (size_t)unit_local * D;
  uv.vnew = vnew_all + (size_t)unit_local * D;
  uv.n8 = n8;
  uv.nw = nw;
  uv.n = n8 + nw + appended;
  const int n = uv.n;
  if (appended) {
    append_row(dm, (uint16_t*)c.k16 + u * (size_t)dm.cap16 * D,
               (uint16_t*)c.v16 + u * (size_t)dm.cap16 * D, nw, uv.knew, uv.vnew);
  } else if (tid == 0 && hk == 0) {
    atomicOr(c.status, (int)CONF_ST_WINDOW_FULL);
  }

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
    key_dot<D>(dm, uv, j, q8, qw, sig);
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
  float* mp_lb = massp_all + (size_t)lb * dm.Hkv * dm.capt;
  float* massp = mp_lb + (size_t)hk * dm.capt;
  for (int base = 0; base < n; base += kAttnThreads) {
    const int j = base + tid;
    if (j < n) {
      key_dot<D>(dm, uv, j, q8, qw, sig);
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
          if (tok < n8) {
            a8 = fmaf(p, (float)uv.v8[vtile_off(tok, ch, D)], a8);
          } else {
            const int w = tok - n8;
            const uint16_t x = w < nw ? uv.v16[vtile_off(w, ch, D)] : uv.vnew[ch];
            a16 = fmaf(p, h16_to_f32(x, dm.bf16), a16);
          }
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
  if (arrive_last(c, dm, lb)) ema_update_lb(c, dm, lb, n8, nw, appended, t, mp_lb);
}

void launch_attn(const Dims& dm, const conf_cache& c, int layer0, int nl, const void* q,
                 const void* k_new, const void* v_new, float* out, float* massp, hipStream_t st) {
  const dim3 grid(nl * dm.B * dm.Hkv);
  if (dm.D == 64)
    hipLaunchKernelGGL(attn_ref_kernel<64>, grid, dim3(kAttnThreads), 0, st, c, dm, layer0,
                       (const uint16_t*)q, (const uint16_t*)k_new, (const uint16_t*)v_new, out,
                       massp);
  else
    hipLaunchKernelGGL(attn_ref_kernel<128>, grid, dim3(kAttnThreads), 0, st, c, dm, layer0,
                       (const uint16_t*)q, (const uint16_t*)k_new, (const uint16_t*)v_new, out,
                       massp);
}

}  // namespace confkv
