// (a) Confidence of each sequence's next-token logits and its per-layer budgets.
//
// CONF-KV explainer, Methodology, confidence estimation: c = w_H (1 - H^) +
// w_m sigma(m) + w_p p(1); adaptive budget selection: c >= tau -> N_high,
// else N_low; pyramidal budgets (CONF-KV-L) shrink the budget with depth.
//
// The vocabulary row (fp32, HBM-bound: 4 bytes per logit, read once) is split
// into chunks of 256 threads x kPer elements.  Each chunk keeps its elements in
// registers and reduces them to (M, S, T, top1, top2, non-finite count) with
// S = sum e^(z-M), T = sum e^(z-M)(z-M).  A second kernel merges the chunks of a
// row in a fixed order: with M* = max M_k, S = sum S_k e^(M_k-M*) and
// T = sum e^(M_k-M*)(T_k + (M_k-M*) S_k); then H = ln S - T/S and p(1) = 1/S.
#include "common.hpp"

namespace confkv {

constexpr int kConfThreads = 256;
constexpr int kConfPer = 16;  // logits per thread per chunk

// (a, b) = the two largest values seen, duplicates counted; z is never NaN.  Written
// with min/max: as a branch the compiler kept (a, b) in private memory and stored
// through a selected address.
__device__ inline void top2_push(float z, float& a, float& b) {
  b = fmaxf(b, fminf(a, z));
  a = fmaxf(a, z);
}
__device__ inline void top2_merge(float& a, float& b, float a2, float b2) {
  const float hi = fmaxf(a, a2), lo = fminf(a, a2);
  b = fmaxf(lo, fmaxf(b, b2));
  a = hi;
}

// VEC: every row starts 16-byte aligned (aligned base, V a multiple of 4), so a
// thread reads its 16 elements as four 16-byte loads.
template <bool VEC>
__global__ __launch_bounds__(kConfThreads) void conf_partial_kernel(const float* __restrict__ logits,
                                                                   float* __restrict__ part,
                                                                   int V, int n_chunks) {
#pragma clang fp contract(off)
  const int chunk = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const float* row = logits + (size_t)b * V;
  const int base = chunk * kConfThreads * kConfPer;
  // Every load is issued before the first use, unconditionally (an index past the
  // row reads the row's last element and is then discarded), so that the chunk
  // costs one memory round trip: with a branch around each load the compiler
  // waits for every load before issuing the next.
  float z[kConfPer];
  if constexpr (VEC) {
    // thread tid reads elements base + 4*(i*256 + tid) .. +3 (V is a multiple of 4)
#pragma unroll
    for (int i = 0; i < kConfPer / 4; ++i) {
      const int idx = base + 4 * (i * kConfThreads + tid);
      const float4 v4 = *(const float4*)(row + (idx < V ? idx : V - 4));
      z[4 * i] = v4.x;
      z[4 * i + 1] = v4.y;
      z[4 * i + 2] = v4.z;
      z[4 * i + 3] = v4.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kConfPer; ++i) z[i] = row[min(base + i * kConfThreads + tid, V - 1)];
  }
  float m = -INFINITY, a = -INFINITY, a2 = -INFINITY;
  int bad = 0;
#pragma unroll
  for (int i = 0; i < kConfPer; ++i) {
    const int idx = VEC ? base + 4 * ((i / 4) * kConfThreads + tid) + (i % 4)
                        : base + i * kConfThreads + tid;
    const bool ok = idx < V, fin = isfinite(z[i]);
    bad |= (ok && !fin) ? 1 : 0;
    const float v = (ok && fin) ? z[i] : -INFINITY;  // non-finite logits count as -inf
    top2_push(v, a, a2);
    z[i] = v;
    m = fmaxf(m, v);
  }
  __shared__ float red[kConfThreads / 64][6];
  __shared__ float bm;
  // block max
  float wm = m;
  for (int off = 32; off > 0; off >>= 1) wm = fmaxf(wm, __shfl_xor(wm, off));
  const int wave = tid >> 6, lane = tid & 63;
  if (lane == 0) red[wave][0] = wm;
  __syncthreads();
  if (tid == 0) {
    float x = red[0][0];
    for (int w = 1; w < kConfThreads / 64; ++w) x = fmaxf(x, red[w][0]);
    bm = x;
  }
  __syncthreads();
  const float M = bm;
  float S = 0.f, T = 0.f;
  if (M > -INFINITY) {
#pragma unroll
    for (int i = 0; i < kConfPer; ++i) {
      if (z[i] > -INFINITY) {
        const float d = z[i] - M;
        const float e = __expf(d);  // relative error ~1e-7, far inside c's tolerance
        S += e;
        T += e * d;
      }
    }
  }
  // block sums, top-2 and non-finite count
  for (int off = 32; off > 0; off >>= 1) {
    S += __shfl_xor(S, off);
    T += __shfl_xor(T, off);
    const float oa = __shfl_xor(a, off), ob = __shfl_xor(a2, off);
    top2_merge(a, a2, oa, ob);
    bad |= __shfl_xor(bad, off);
  }
  __syncthreads();
  if (lane == 0) {
    red[wave][1] = S;
    red[wave][2] = T;
    red[wave][3] = a;
    red[wave][4] = a2;
    red[wave][5] = (float)bad;
  }
  __syncthreads();
  if (tid == 0) {
    float s = 0.f, t = 0.f, x = -INFINITY, y = -INFINITY, nb = 0.f;
    for (int w = 0; w < kConfThreads / 64; ++w) {
      s += red[w][1];
      t += red[w][2];
      top2_merge(x, y, red[w][3], red[w][4]);
      nb += red[w][5];
    }
    float* o = part + ((size_t)b * n_chunks + chunk) * 8;
    o[0] = M;
    o[1] = s;
    o[2] = t;
    o[3] = x;
    o[4] = y;
    o[5] = nb;
  }
}

__global__ __launch_bounds__(64) void conf_final_kernel(const float* __restrict__ part,
                                                       int n_chunks, Dims dm,
                                                       float* __restrict__ c_out,
                                                       int32_t* __restrict__ budget) {
#pragma clang fp contract(off)
  const int b = blockIdx.x, lane = threadIdx.x;
  const float* pb = part + (size_t)b * n_chunks * 8;
  // global max over chunks
  float M = -INFINITY;
  for (int k = lane; k < n_chunks; k += 64) M = fmaxf(M, pb[k * 8 + 0]);
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float S = 0.f, T = 0.f, a = -INFINITY, a2 = -INFINITY, bad = 0.f;
  for (int k = lane; k < n_chunks; k += 64) {
    const float Mk = pb[k * 8 + 0], Sk = pb[k * 8 + 1], Tk = pb[k * 8 + 2];
    if (Mk > -INFINITY) {
      const float dk = Mk - M;
      const float f = expf(dk);
      S += Sk * f;
      T += f * (Tk + dk * Sk);
    }
    top2_merge(a, a2, pb[k * 8 + 3], pb[k * 8 + 4]);
    bad += pb[k * 8 + 5];
  }
  for (int off = 32; off > 0; off >>= 1) {
    S += __shfl_xor(S, off);
    T += __shfl_xor(T, off);
    const float oa = __shfl_xor(a, off), ob = __shfl_xor(a2, off);
    top2_merge(a, a2, oa, ob);
    bad += __shfl_xor(bad, off);
  }
  if (lane == 0) {
    float c;
    if (bad > 0.f) {
      c = __builtin_nanf("");
    } else {
      const float H = logf(S) - T / S;
      const float Hn = H / logf((float)dm.V);
      const float mgn = a - a2;
      const float sig = 1.0f / (1.0f + expf(-mgn));
      const float p1 = 1.0f / S;
      c = dm.w_H * (1.0f - Hn) + dm.w_m * sig + dm.w_p * p1;
    }
    c_out[b] = c;
    const int N = (c >= dm.tau) ? dm.n_high : dm.n_low;
    for (int l = 0; l < dm.L; ++l) budget[(size_t)b * dm.L + l] = layer_budget(N, l, dm.L, dm.pyramid);
  }
}

int conf_vchunks(int V) { return (V + kConfThreads * kConfPer - 1) / (kConfThreads * kConfPer); }

void launch_confidence(const Dims& dm, const float* logits, float* part, float* c, int32_t* budget,
                       hipStream_t st) {
  const int nch = conf_vchunks(dm.V);
  const bool vec = ((uintptr_t)logits & 15u) == 0 && (dm.V & 3) == 0;
  if (vec)
    hipLaunchKernelGGL(conf_partial_kernel<true>, dim3(nch, dm.B), dim3(kConfThreads), 0, st,
                       logits, part, dm.V, nch);
  else
    hipLaunchKernelGGL(conf_partial_kernel<false>, dim3(nch, dm.B), dim3(kConfThreads), 0, st,
                       logits, part, dm.V, nch);
  hipLaunchKernelGGL(conf_final_kernel, dim3(dm.B), dim3(64), 0, st, part, nch, dm, c, budget);
}

}  // namespace confkv
