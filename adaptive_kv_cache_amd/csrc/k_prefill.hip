// ARKV's prefill phase: layer-wise Original budgets from the statistics of the
// prefill attention.
//
// The ARKV page, Methodology, 1. prefill phase (layer-wise budget assignment):
// during the prefill each layer's attention pattern is measured by its entropy
// (spatial spread), variance (difference in token weights) and kurtosis (shape
// of the distribution); the layers more sensitive to precision loss get a larger
// share of full-precision (Original) tokens.  The page gives no formula; the
// reading used here (and by the CPU checker):
//   * a head's attention is the softmax, scale 1/sqrt(d), of its probe query (the
//     first query that attends to the whole prefill) over the 16-bit prefill keys;
//   * with d = p - 1/L0: H^ = H / ln L0, v^ = L0 sum d^2 / (L0 - 1),
//     k^ = ln(max(L0 sum d^4 / (sum d^2)^2, 1)) / ln L0 (0 for uniform weights);
//   * concentration = ((1 - H^) + v^ + k^) / 3, averaged over the layer's heads;
//     more concentrated counts as more sensitive;
//   * the OQ ratio runs linearly from 0.75 (the sequence's least concentrated
//     layer) to 0.95 (its most concentrated); N_O = max(P, ceil(r N)), N = n_high.
//
// Launches: one workgroup per (layer, sequence, KV head) computes its G heads in
// two passes over the keys (pass 1: the running max, sum and entropy sum; pass
// 2: the deviations' second and fourth powers, recomputing the scores the same
// way) and writes the sum of its heads' concentrations to the workspace; a small
// kernel averages each (layer, sequence) over its KV heads in a fixed order.  A
// second entry point turns the concentrations into the budgets.
#include "common.hpp"

namespace confkv {

constexpr int kPsThreads = 256;
constexpr int kPsWaves = kPsThreads / 64;

// Scores of key row `k` (16-bit, D channels) against the G probe queries in LDS.
template <int D>
__device__ inline void row_scores(const uint16_t* __restrict__ k, const float* sq, int G,
                                  int bf16, float rs, float z[kMaxGroup]) {
  float acc[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) acc[h] = 0.f;
  for (int c8 = 0; c8 < D / 8; ++c8) {
    const uint4 w = *(const uint4*)(k + 8 * c8);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    float kv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) kv[e] = h16_to_f32((uint16_t)(ww[e >> 1] >> (16 * (e & 1))), bf16);
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h >= G) break;
      const float* qh = sq + h * D + 8 * c8;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h] = fmaf(qh[e], kv[e], acc[h]);
    }
  }
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) z[h] = acc[h] * rs;
}

// (M, S, T) of a set of scores: M the max, S = sum e^(z-M), T = sum e^(z-M)(z-M).
// Merging two sets at M' = max: S' = S1 e^(M1-M') + S2 e^(M2-M'),
// T' = (T1 + (M1-M') S1) e^(M1-M') + (T2 + (M2-M') S2) e^(M2-M').
__device__ inline void mst_merge(float& M, float& S, float& T, float M2, float S2, float T2) {
  const float Mn = fmaxf(M, M2);
  if (Mn == -INFINITY) return;
  const float a = M == -INFINITY ? 0.f : expf(M - Mn), b = M2 == -INFINITY ? 0.f : expf(M2 - Mn);
  const float d1 = M == -INFINITY ? 0.f : M - Mn, d2 = M2 == -INFINITY ? 0.f : M2 - Mn;
  T = (T + d1 * S) * a + (T2 + d2 * S2) * b;
  S = S * a + S2 * b;
  M = Mn;
}

template <int D>
__global__ __launch_bounds__(kPsThreads) void arkv_stats_kernel(Dims dm, int layer0, int L0,
                                                                const uint16_t* __restrict__ q_all,
                                                                const uint16_t* __restrict__ k_all,
                                                                float* __restrict__ part) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int unit_local = blockIdx.x;
  const int hk = unit_local % dm.Hkv;
  const int lbl = unit_local / dm.Hkv;
  const size_t u = (size_t)(layer0 * dm.B + lbl) * dm.Hkv + hk;
  const int G = dm.G;
  const uint16_t* qsrc = q_all + ((size_t)lbl * dm.Hq + (size_t)hk * G) * D;
  const uint16_t* ksrc = k_all + (size_t)unit_local * L0 * D;
  const float rs = 1.0f / sqrtf((float)D);
  __shared__ float sq[kMaxGroup * D];
  __shared__ float red[kPsWaves][kMaxGroup][3];
  __shared__ float hst[kMaxGroup][3];  // per head: M, S, and H = ln S - T/S
  for (int i = tid; i < G * D; i += kPsThreads) sq[i] = h16_to_f32(qsrc[i], dm.bf16);
  __syncthreads();
  // ---- pass 1: running (M, S, T) per head
  float M[kMaxGroup], S[kMaxGroup], T[kMaxGroup], z[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    M[h] = -INFINITY;
    S[h] = 0.f;
    T[h] = 0.f;
  }
  for (int j = tid; j < L0; j += kPsThreads) {
    row_scores<D>(ksrc + (size_t)j * D, sq, G, dm.bf16, rs, z);
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) mst_merge(M[h], S[h], T[h], z[h], 1.f, 0.f);
  }
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    for (int off = 32; off > 0; off >>= 1) {
      const float m2 = __shfl_xor(M[h], off), s2 = __shfl_xor(S[h], off), t2 = __shfl_xor(T[h], off);
      mst_merge(M[h], S[h], T[h], m2, s2, t2);
    }
    if (lane == 0 && h < G) {
      red[wave][h][0] = M[h];
      red[wave][h][1] = S[h];
      red[wave][h][2] = T[h];
    }
  }
  __syncthreads();
  if (tid < G) {
    float m = -INFINITY, s = 0.f, t = 0.f;
    for (int w = 0; w < kPsWaves; ++w) mst_merge(m, s, t, red[w][tid][0], red[w][tid][1], red[w][tid][2]);
    hst[tid][0] = m;
    hst[tid][1] = s;
    hst[tid][2] = logf(s) - t / s;
  }
  __syncthreads();
  // ---- pass 2: sums of d^2 and d^4, d = p - 1/L0, p = e^(z-M)/S
  const float mu = 1.0f / (float)L0;
  float s2[kMaxGroup], s4[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) s2[h] = s4[h] = 0.f;
  for (int j = tid; j < L0; j += kPsThreads) {
    row_scores<D>(ksrc + (size_t)j * D, sq, G, dm.bf16, rs, z);
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h >= G) break;
      const float p = expf(z[h] - hst[h][0]) / hst[h][1];
      const float d = p - mu;
      const float d2 = d * d;
      s2[h] += d2;
      s4[h] += d2 * d2;
    }
  }
  __syncthreads();  // red[] is reused below
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    for (int off = 32; off > 0; off >>= 1) {
      s2[h] += __shfl_xor(s2[h], off);
      s4[h] += __shfl_xor(s4[h], off);
    }
    if (lane == 0 && h < G) {
      red[wave][h][0] = s2[h];
      red[wave][h][1] = s4[h];
    }
  }
  __syncthreads();
  if (tid == 0) {
    const float lnL = logf((float)L0);
    float sum = 0.f;
    for (int h = 0; h < G; ++h) {
      float a2 = 0.f, a4 = 0.f;
      for (int w = 0; w < kPsWaves; ++w) {
        a2 += red[w][h][0];
        a4 += red[w][h][1];
      }
      const float Hh = hst[h][2] / lnL;
      const float vh = (float)L0 * a2 / (float)(L0 - 1);
      float kh = 0.f;
      if (a2 > 0.f) {
        const float kurt = (float)L0 * a4 / (a2 * a2);
        kh = logf(fmaxf(kurt, 1.f)) / lnL;
      }
      sum += ((1.f - Hh) + vh + kh) / 3.f;
    }
    part[u] = sum;
  }
}

// conc[l][b] = (sum over the KV heads, in order, of their heads' sums) / Hq
__global__ void arkv_stats_final_kernel(Dims dm, int layer0, int nl, const float* __restrict__ part,
                                        float* __restrict__ conc) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nl * dm.B) return;
  const int lb = layer0 * dm.B + i;
  float s = 0.f;
  for (int hk = 0; hk < dm.Hkv; ++hk) s += part[(size_t)lb * dm.Hkv + hk];
  conc[lb] = s / (float)dm.Hq;
}

// n_orig[b][l] from conc[l][b]: one thread per sequence (the layers of a sequence
// are few), float32 one rounding at a time.
__global__ void arkv_budget_kernel(Dims dm, const float* __restrict__ conc,
                                   int32_t* __restrict__ n_orig) {
#pragma clang fp contract(off)
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= dm.B) return;
  float lo = INFINITY, hi = -INFINITY;
  for (int l = 0; l < dm.L; ++l) {
    const float c = conc[(size_t)l * dm.B + b];
    lo = fminf(lo, c);
    hi = fmaxf(hi, c);
  }
  const float r_lo = 0.75f, r_hi = 0.95f;
  const float span = hi - lo, width = r_hi - r_lo;
  for (int l = 0; l < dm.L; ++l) {
    float r;
    if (span > 0.f) {
      const float t = (conc[(size_t)l * dm.B + b] - lo) / span;
      r = r_lo + width * t;
    } else {
      r = (r_lo + r_hi) / 2.f;
    }
    int n = (int)ceilf(r * (float)dm.n_high);
    n_orig[(size_t)b * dm.L + l] = n > dm.P ? n : dm.P;
  }
}

void launch_arkv_stats(const Dims& dm, int layer0, int nl, int L0, const void* q,
                       const void* k_pre, float* part, float* conc, hipStream_t st) {
  const dim3 grid(nl * dm.B * dm.Hkv);
  if (dm.D == 64)
    hipLaunchKernelGGL(arkv_stats_kernel<64>, grid, dim3(kPsThreads), 0, st, dm, layer0, L0,
                       (const uint16_t*)q, (const uint16_t*)k_pre, part);
  else
    hipLaunchKernelGGL(arkv_stats_kernel<128>, grid, dim3(kPsThreads), 0, st, dm, layer0, L0,
                       (const uint16_t*)q, (const uint16_t*)k_pre, part);
  const int n = nl * dm.B;
  hipLaunchKernelGGL(arkv_stats_final_kernel, dim3((n + 255) / 256), dim3(256), 0, st, dm, layer0,
                     nl, part, conc);
}

void launch_arkv_budgets(const Dims& dm, const float* conc, int32_t* n_orig, hipStream_t st) {
  hipLaunchKernelGGL(arkv_budget_kernel, dim3((dm.B + 63) / 64), dim3(64), 0, st, dm, conc, n_orig);
}

}  // namespace confkv
