// Cache maintenance kernels: reset, prefill ingest, compaction + demotion, and
// export of one (layer, sequence).
//
// CONF-KV explainer, Methodology, system integration: the newest W tokens stay
// 16-bit, older kept tokens are INT8 per head and channel (mixed-precision
// storage); contiguous compaction keeps a dense layout with no indirection
// tables (implementation).  Token ranking and eviction: EMA attention mass.
#include "common.hpp"

namespace confkv {

// Per-unit base offsets.  A unit is one (layer, sequence, KV head); lb = l*B + b.
__device__ inline size_t unit_of(const Dims& dm, int lb, int hk) { return (size_t)lb * dm.Hkv + hk; }

// ---------------------------------------------------------------- reset
__global__ void reset_kernel(conf_cache c, Dims dm) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nlb = (size_t)dm.L * dm.B;
  const size_t namax = nlb * dm.Hkv * dm.D;
  if (i < nlb) {
    c.n8[i] = 0;
    c.n16[i] = 0;
    c.t[i] = -1;
  }
  if (i < namax) {
    c.k_amax[i] = 0.f;
    c.v_amax[i] = 0.f;
  }
  if (i == 0) c.status[0] = 0;
}

void launch_reset(const Dims& dm, const conf_cache& c, hipStream_t st) {
  const size_t n = (size_t)dm.L * dm.B * dm.Hkv * dm.D;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(reset_kernel, dim3((unsigned)blocks), dim3(256), 0, st, c, dm);
}

// ---------------------------------------------------------------- ingest
// Prefill of L0 tokens for one unit: positions < L0 - W become INT8 with the
// absmax over exactly those tokens; the rest go to the window.
__global__ __launch_bounds__(256) void ingest_kernel(conf_cache c, Dims dm, int layer0, int L0,
                                                     const uint16_t* __restrict__ kp,
                                                     const uint16_t* __restrict__ vp) {
#pragma clang fp contract(off)
  const int unit_local = blockIdx.x;
  const int hk = unit_local % dm.Hkv;
  const int lbl = unit_local / dm.Hkv;
  const int lb = layer0 * dm.B + lbl;
  const size_t u = unit_of(dm, lb, hk);
  const int D = dm.D;
  const int n8 = L0 > dm.W ? L0 - dm.W : 0;
  const int nw = L0 - n8;
  const uint16_t* ksrc = kp + (size_t)unit_local * L0 * D;
  const uint16_t* vsrc = vp + (size_t)unit_local * L0 * D;
  __shared__ float amk[256], amv[256];
  __shared__ float sk[128], sv[128];
  // absmax per channel: thread (ch, part) with 256/D parts striding over tokens
  const int parts = blockDim.x / D;
  const int ch = threadIdx.x % D, part = threadIdx.x / D;
  float mk = 0.f, mv = 0.f;
  if (part < parts) {
    for (int i = part; i < n8; i += parts) {
      mk = fmaxf(mk, fabsf(h16_to_f32(ksrc[(size_t)i * D + ch], dm.bf16)));
      mv = fmaxf(mv, fabsf(h16_to_f32(vsrc[(size_t)i * D + ch], dm.bf16)));
    }
  }
  amk[threadIdx.x] = mk;
  amv[threadIdx.x] = mv;
  __syncthreads();
  if (threadIdx.x < D) {
    float a = 0.f, b = 0.f;
    for (int p = 0; p < parts; ++p) {
      a = fmaxf(a, amk[p * D + threadIdx.x]);
      b = fmaxf(b, amv[p * D + threadIdx.x]);
    }
    c.k_amax[u * D + threadIdx.x] = a;
    c.v_amax[u * D + threadIdx.x] = b;
    sk[threadIdx.x] = a / 127.0f;
    sv[threadIdx.x] = b / 127.0f;
  }
  __syncthreads();
  int8_t* k8 = c.k8 + u * (size_t)dm.cap8 * D;
  int8_t* v8 = c.v8 + u * (size_t)dm.cap8 * D;
  for (size_t i = threadIdx.x; i < (size_t)n8 * D; i += blockDim.x) {
    const int tok = (int)(i / D), cc = (int)(i % D);
    k8[k8_off(tok, cc, D)] = quant_code(h16_to_f32(ksrc[i], dm.bf16), sk[cc]);
    v8[v8_off(tok, cc, D)] = quant_code(h16_to_f32(vsrc[i], dm.bf16), sv[cc]);
  }
  uint16_t* k16 = (uint16_t*)c.k16 + u * (size_t)dm.cap16 * D;
  uint16_t* v16 = (uint16_t*)c.v16 + u * (size_t)dm.cap16 * D;
  for (size_t i = threadIdx.x; i < (size_t)nw * D; i += blockDim.x) {
    const int w = (int)(i / D), cc = (int)(i % D);
    const size_t s = (size_t)(n8 + w) * D + cc;
    k16[k16_off(w, cc, D)] = ksrc[s];
    v16[v16_off(w, cc, D)] = vsrc[s];
  }
  if (hk == 0) {
    for (int i = threadIdx.x; i < n8; i += blockDim.x) {
      c.pos8[(size_t)lb * dm.cap8 + i] = i;
      c.ema8[(size_t)lb * dm.cap8 + i] = 0.f;
    }
    for (int w = threadIdx.x; w < nw; w += blockDim.x) {
      c.pos16[(size_t)lb * dm.cap16 + w] = n8 + w;
      c.ema16[(size_t)lb * dm.cap16 + w] = 0.f;
    }
    if (threadIdx.x == 0) {
      c.n8[lb] = n8;
      c.n16[lb] = nw;
      c.t[lb] = L0 - 1;
    }
  }
}

void launch_ingest(const Dims& dm, const conf_cache& c, int layer0, int nl, int L0, const void* k,
                   const void* v, hipStream_t st) {
  hipLaunchKernelGGL(ingest_kernel, dim3(nl * dm.B * dm.Hkv), dim3(256), 0, st, c, dm, layer0, L0,
                     (const uint16_t*)k, (const uint16_t*)v);
}

// ---------------------------------------------------------------- compaction plan
// One workgroup per (layer, sequence).  Window keep flags exclude the token at
// position t - W (it is demoted, not kept in place).  In each region the k-th
// hole below the new end receives the k-th survivor above it.  Metadata moves
// happen here; the plan tells the data kernel what to move.
// plan: [0] n8 new (before demotion) [1] moves8 [2] n16 new [3] moves16
//       [4] window slot of the demotee or -1 [5] INT8 slot it goes to or -1
constexpr int kPlanThreads = 256;

__device__ inline int block_excl_scan(int v, int* sh, int& total) {
  // Inclusive Hillis-Steele scan over 256 threads in shared memory.
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int x = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += x;
    __syncthreads();
  }
  total = sh[kPlanThreads - 1];
  const int r = sh[tid] - v;
  __syncthreads();
  return r;
}

__device__ void plan_region(const uint8_t* keep, int n, int n_new, int* mv, int* sh,
                            int32_t* pos, float* ema, int& n_moves_out) {
  // holes: i < n_new with !keep[i];  movers: n_new <= i < n with keep[i]
  int hole_base = 0;
  for (int base = 0; base < n_new; base += kPlanThreads) {
    const int i = base + threadIdx.x;
    const int is_hole = (i < n_new) && !keep[i];
    int tot;
    const int r = block_excl_scan(is_hole, sh, tot);
    if (is_hole) mv[2 * (hole_base + r) + 1] = i;
    hole_base += tot;
  }
  int mover_base = 0;
  for (int base = n_new; base < n; base += kPlanThreads) {
    const int i = base + threadIdx.x;
    const int is_mv = (i < n) && keep[i];
    int tot;
    const int r = block_excl_scan(is_mv, sh, tot);
    if (is_mv) mv[2 * (mover_base + r)] = i;
    mover_base += tot;
  }
  __syncthreads();
  n_moves_out = hole_base;  // == mover_base
  for (int k = threadIdx.x; k < hole_base; k += kPlanThreads) {
    const int src = mv[2 * k], dst = mv[2 * k + 1];
    pos[dst] = pos[src];
    ema[dst] = ema[src];
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(conf_cache c, Dims dm, int layer0,
                                                            const uint8_t* __restrict__ keep_all,
                                                            int32_t* __restrict__ plan_all,
                                                            int32_t* __restrict__ mv8_all,
                                                            int32_t* __restrict__ mv16_all,
                                                            uint8_t* __restrict__ wkeep_all) {
  const int lb = layer0 * dm.B + blockIdx.x;
  const int n8 = c.n8[lb], n16 = c.n16[lb], t = c.t[lb];
  const uint8_t* keep8 = keep_all + (size_t)lb * dm.capt;
  const uint8_t* keep16 = keep8 + dm.cap8;
  uint8_t* wkeep = wkeep_all + (size_t)lb * dm.cap16;
  int32_t* pos8 = c.pos8 + (size_t)lb * dm.cap8;
  float* ema8 = c.ema8 + (size_t)lb * dm.cap8;
  int32_t* pos16 = c.pos16 + (size_t)lb * dm.cap16;
  float* ema16 = c.ema16 + (size_t)lb * dm.cap16;
  __shared__ int sh[kPlanThreads];
  __shared__ int s_cnt8, s_cnt16, s_jd;
  if (threadIdx.x == 0) {
    s_cnt8 = 0;
    s_cnt16 = 0;
    s_jd = -1;
  }
  __syncthreads();
  const int target = t - dm.W;
  int c8 = 0, c16 = 0;
  for (int i = threadIdx.x; i < n8; i += kPlanThreads) c8 += keep8[i] ? 1 : 0;
  for (int w = threadIdx.x; w < n16; w += kPlanThreads) {
    int k = keep16[w] ? 1 : 0;
    if (k && target >= 0 && pos16[w] == target) {
      s_jd = w;  // at most one slot holds this position
      k = 0;
    }
    wkeep[w] = (uint8_t)k;
    c16 += k;
  }
  atomicAdd(&s_cnt8, c8);
  atomicAdd(&s_cnt16, c16);
  __syncthreads();
  const int n8n = s_cnt8, n16n = s_cnt16, jd = s_jd;
  int dpos = 0;
  float dema = 0.f;
  if (jd >= 0) {
    dpos = pos16[jd];
    dema = ema16[jd];
  }
  __syncthreads();
  int nm8 = 0, nm16 = 0;
  plan_region(keep8, n8, n8n, mv8_all + (size_t)lb * dm.cap8, sh, pos8, ema8, nm8);
  __syncthreads();
  plan_region(wkeep, n16, n16n, mv16_all + (size_t)lb * dm.cap16, sh, pos16, ema16, nm16);
  __syncthreads();
  if (threadIdx.x == 0) {
    int dest = -1;
    if (jd >= 0) {
      if (n8n < dm.cap8) {
        dest = n8n;
        pos8[dest] = dpos;
        ema8[dest] = dema;
      } else {
        atomicOr(c.status, (int)CONF_ST_INT8_FULL);
      }
    }
    int32_t* pl = plan_all + (size_t)lb * 16;
    pl[0] = n8n;
    pl[1] = nm8;
    pl[2] = n16n;
    pl[3] = nm16;
    pl[4] = jd;
    pl[5] = dest;
    c.n8[lb] = n8n + (dest >= 0 ? 1 : 0);
    c.n16[lb] = n16n;
  }
}

// ---------------------------------------------------------------- data moves + demotion
// One workgroup per unit.  Reads the demotee's 16-bit row first (a window move
// may overwrite its slot), moves INT8 and window rows/columns, then quantises the
// demotee into INT8 slot `dest` under the running absmax, requantising the
// channels whose absmax grows.
__global__ __launch_bounds__(256) void move_kernel(conf_cache c, Dims dm, int layer0,
                                                   const int32_t* __restrict__ plan_all,
                                                   const int32_t* __restrict__ mv8_all,
                                                   const int32_t* __restrict__ mv16_all) {
#pragma clang fp contract(off)
  const int unit_local = blockIdx.x;
  const int hk = unit_local % dm.Hkv;
  const int lb = layer0 * dm.B + unit_local / dm.Hkv;
  const size_t u = unit_of(dm, lb, hk);
  const int D = dm.D;
  const int32_t* pl = plan_all + (size_t)lb * 16;
  const int n8n = pl[0], nm8 = pl[1], nm16 = pl[3], jd = pl[4], dest = pl[5];
  int8_t* k8 = c.k8 + u * (size_t)dm.cap8 * D;
  int8_t* v8 = c.v8 + u * (size_t)dm.cap8 * D;
  uint16_t* k16 = (uint16_t*)c.k16 + u * (size_t)dm.cap16 * D;
  uint16_t* v16 = (uint16_t*)c.v16 + u * (size_t)dm.cap16 * D;
  __shared__ float xk[128], xv[128];
  __shared__ float s_old_k[128], s_new_k[128], s_old_v[128], s_new_v[128];
  __shared__ int grown_k[128], grown_v[128];
  __shared__ int n_grown_k, n_grown_v;
  if (threadIdx.x == 0) {
    n_grown_k = 0;
    n_grown_v = 0;
  }
  if (dest >= 0) {
    for (int ch = threadIdx.x; ch < D; ch += blockDim.x) {
      xk[ch] = h16_to_f32(k16[k16_off(jd, ch, D)], dm.bf16);
      xv[ch] = h16_to_f32(v16[v16_off(jd, ch, D)], dm.bf16);
    }
  }
  __syncthreads();
  const int32_t* mv8 = mv8_all + (size_t)lb * dm.cap8;
  for (int i = threadIdx.x; i < nm8 * D; i += blockDim.x) {
    const int k = i / D, ch = i % D;
    const int src = mv8[2 * k], dst = mv8[2 * k + 1];
    k8[k8_off(dst, ch, D)] = k8[k8_off(src, ch, D)];
    v8[v8_off(dst, ch, D)] = v8[v8_off(src, ch, D)];
  }
  const int32_t* mv16 = mv16_all + (size_t)lb * dm.cap16;
  for (int i = threadIdx.x; i < nm16 * D; i += blockDim.x) {
    const int k = i / D, ch = i % D;
    const int src = mv16[2 * k], dst = mv16[2 * k + 1];
    k16[k16_off(dst, ch, D)] = k16[k16_off(src, ch, D)];
    v16[v16_off(dst, ch, D)] = v16[v16_off(src, ch, D)];
  }
  __syncthreads();
  if (dest < 0) return;
  for (int ch = threadIdx.x; ch < D; ch += blockDim.x) {
    float* ak = c.k_amax + u * D + ch;
    float* av = c.v_amax + u * D + ch;
    const float ok = *ak, ov = *av;
    const float a_k = fabsf(xk[ch]), a_v = fabsf(xv[ch]);
    const int gk = a_k > ok, gv = a_v > ov;
    const float nk = gk ? a_k : ok, nv = gv ? a_v : ov;
    const float sk = nk / 127.0f, sv = nv / 127.0f;
    s_old_k[ch] = ok / 127.0f;
    s_new_k[ch] = sk;
    s_old_v[ch] = ov / 127.0f;
    s_new_v[ch] = sv;
    if (gk) grown_k[atomicAdd(&n_grown_k, 1)] = ch;
    if (gv) grown_v[atomicAdd(&n_grown_v, 1)] = ch;
    *ak = nk;
    *av = nv;
    k8[k8_off(dest, ch, D)] = quant_code(xk[ch], sk);
    v8[v8_off(dest, ch, D)] = quant_code(xv[ch], sv);
  }
  __syncthreads();
  // Requantise the stored codes (slots < n8n) of every channel whose absmax grew.
  const int ngk = n_grown_k, ngv = n_grown_v;
  for (int i = threadIdx.x; i < n8n * ngk; i += blockDim.x) {
    const int tok = i / ngk, ch = grown_k[i % ngk];
    int8_t* p = k8 + k8_off(tok, ch, D);
    *p = quant_code((float)(*p) * s_old_k[ch], s_new_k[ch]);
  }
  for (int i = threadIdx.x; i < n8n * ngv; i += blockDim.x) {
    const int tok = i / ngv, ch = grown_v[i % ngv];
    int8_t* p = v8 + v8_off(tok, ch, D);
    *p = quant_code((float)(*p) * s_old_v[ch], s_new_v[ch]);
  }
}

void launch_compact(const Dims& dm, const conf_cache& c, int layer0, int nl, const uint8_t* keep,
                    int32_t* plan, int32_t* mv8, int32_t* mv16, uint8_t* wkeep, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(nl * dm.B), dim3(kPlanThreads), 0, st, c, dm, layer0, keep,
                     plan, mv8, mv16, wkeep);
  hipLaunchKernelGGL(move_kernel, dim3(nl * dm.B * dm.Hkv), dim3(256), 0, st, c, dm, layer0, plan,
                     mv8, mv16);
}

// ---------------------------------------------------------------- export
__global__ void export_kernel(conf_cache c, Dims dm, int lb, int8_t* ok8, int8_t* ov8,
                              uint16_t* ok16, uint16_t* ov16) {
  const size_t n8tot = (size_t)dm.cap8 * dm.Hkv * dm.D;
  const size_t n16tot = (size_t)dm.cap16 * dm.Hkv * dm.D;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8tot + n16tot;
       i += (size_t)gridDim.x * blockDim.x) {
    if (i < n8tot) {
      const int ch = (int)(i % dm.D);
      const int hk = (int)((i / dm.D) % dm.Hkv);
      const int s = (int)(i / ((size_t)dm.D * dm.Hkv));
      const size_t u = unit_of(dm, lb, hk);
      ok8[i] = c.k8[u * dm.cap8 * dm.D + k8_off(s, ch, dm.D)];
      ov8[i] = c.v8[u * dm.cap8 * dm.D + v8_off(s, ch, dm.D)];
    } else {
      const size_t j = i - n8tot;
      const int ch = (int)(j % dm.D);
      const int hk = (int)((j / dm.D) % dm.Hkv);
      const int s = (int)(j / ((size_t)dm.D * dm.Hkv));
      const size_t u = unit_of(dm, lb, hk);
      ok16[j] = ((const uint16_t*)c.k16)[u * dm.cap16 * dm.D + k16_off(s, ch, dm.D)];
      ov16[j] = ((const uint16_t*)c.v16)[u * dm.cap16 * dm.D + v16_off(s, ch, dm.D)];
    }
  }
}

void launch_export(const Dims& dm, const conf_cache& c, int lb, int8_t* k8, int8_t* v8, void* k16,
                   void* v16, hipStream_t st) {
  hipLaunchKernelGGL(export_kernel, dim3(512), dim3(256), 0, st, c, dm, lb, k8, v8, (uint16_t*)k16,
                     (uint16_t*)v16);
}

}  // namespace confkv
