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

// ---------------------------------------------------------------- compaction + demotion
// One workgroup of 1024 threads per (layer, sequence).
//  1. Window keep flags exclude the token at position t - W (it is demoted, not
//     kept in place).  In each region the k-th hole below the new end receives
//     the k-th survivor above it (both in slot order), so the layout stays dense.
//  2. Positions and EMAs move; the demotee's metadata lands in INT8 slot n8'.
//  3. Key/value data of every KV head move the same way.
//  4. Per (KV head, channel), one thread quantises the demotee under the running
//     absmax; channels whose absmax grows first requantise their stored codes.
// plan: [0] n8' [1] INT8 moves [2] n16' [3] window moves [4] demotee's window
//       slot or -1 [5] its INT8 slot or -1  (kept in the workspace for inspection)
constexpr int kCompThreads = 1024;
constexpr int kCompWaves = kCompThreads / 64;
constexpr int kMaxGrown = 512;  // grown channels requantised by the whole workgroup

// Ordered ranks of the slots of [lo, hi) whose keep flag equals `want`:
// out[2*rank + off] = slot.  Returns their number.  Every thread must call it.
__device__ int rank_slots(int lo, int hi, const uint8_t* keep, bool want, int32_t* out, int off,
                          int* s_wcnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int base = 0;
  for (int c0 = lo; c0 < hi; c0 += kCompThreads) {
    const int i = c0 + tid;
    const bool f = i < hi && ((keep[i] != 0) == want);
    const unsigned long long bal = __ballot(f);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_wcnt[wave] = __popcll(bal);
    __syncthreads();
    int woff = 0, tot = 0;
    for (int w = 0; w < kCompWaves; ++w) {
      const int cw = s_wcnt[w];
      woff += w < wave ? cw : 0;
      tot += cw;
    }
    if (f) out[2 * (base + woff + before) + off] = i;
    base += tot;
    __syncthreads();
  }
  return base;
}


__global__ __launch_bounds__(kCompThreads) void compact_kernel(conf_cache c, Dims dm, int layer0,
                                                               const uint8_t* __restrict__ keep_all,
                                                               int32_t* __restrict__ plan_all,
                                                               int32_t* __restrict__ mv8_all,
                                                               int32_t* __restrict__ mv16_all,
                                                               uint8_t* __restrict__ wkeep_all) {
#pragma clang fp contract(off)
  const int lb = layer0 * dm.B + blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n8 = c.n8[lb], n16 = c.n16[lb], t = c.t[lb];
  const int D = dm.D;
  const uint8_t* keep8 = keep_all + (size_t)lb * dm.capt;
  const uint8_t* keep16 = keep8 + dm.cap8;
  uint8_t* wkeep = wkeep_all + (size_t)lb * dm.cap16;
  int32_t* pos8 = c.pos8 + (size_t)lb * dm.cap8;
  float* ema8 = c.ema8 + (size_t)lb * dm.cap8;
  int32_t* pos16 = c.pos16 + (size_t)lb * dm.cap16;
  float* ema16 = c.ema16 + (size_t)lb * dm.cap16;
  int32_t* mv8 = mv8_all + (size_t)lb * dm.cap8;
  int32_t* mv16 = mv16_all + (size_t)lb * dm.cap16;
  __shared__ int s_wcnt[kCompWaves];
  __shared__ int s_c8[kCompWaves], s_c16[kCompWaves];
  __shared__ int s_jd;
  __shared__ int s_ngrown;
  __shared__ int s_grown[kMaxGrown];
  __shared__ float s_gold[kMaxGrown], s_gnew[kMaxGrown];
  if (tid == 0) s_jd = -1;
  __syncthreads();
  // ---- 1. counts, the demotee, window keep flags
  const int target = t - dm.W;
  int c8 = 0, c16 = 0;
  for (int i = tid; i < n8; i += kCompThreads) c8 += keep8[i] ? 1 : 0;
  for (int w = tid; w < n16; w += kCompThreads) {
    int k = keep16[w] ? 1 : 0;
    if (k && target >= 0 && pos16[w] == target) {
      s_jd = w;  // at most one slot holds this position
      k = 0;
    }
    wkeep[w] = (uint8_t)k;
    c16 += k;
  }
  for (int off = 32; off > 0; off >>= 1) {
    c8 += __shfl_xor(c8, off);
    c16 += __shfl_xor(c16, off);
  }
  if (lane == 0) {
    s_c8[wave] = c8;
    s_c16[wave] = c16;
  }
  __syncthreads();
  int n8n = 0, n16n = 0;
  for (int w = 0; w < kCompWaves; ++w) {
    n8n += s_c8[w];
    n16n += s_c16[w];
  }
  const int jd = s_jd;
  const int dest = (jd >= 0 && n8n < dm.cap8) ? n8n : -1;
  int dpos = 0;
  float dema = 0.f;
  if (jd >= 0) {  // read before the window metadata moves
    dpos = pos16[jd];
    dema = ema16[jd];
  }
  // ---- 2. move lists: k-th hole below the new end <- k-th survivor above it
  const int nm8 = rank_slots(0, n8n, keep8, false, mv8, 1, s_wcnt);
  rank_slots(n8n, n8, keep8, true, mv8, 0, s_wcnt);
  const int nm16 = rank_slots(0, n16n, wkeep, false, mv16, 1, s_wcnt);
  rank_slots(n16n, n16, wkeep, true, mv16, 0, s_wcnt);
  __syncthreads();  // move lists complete (same workgroup: visible after the barrier)
  // ---- 3. metadata moves (holes and movers are disjoint slots)
  for (int k = tid; k < nm8; k += kCompThreads) {
    const int src = mv8[2 * k], dst = mv8[2 * k + 1];
    pos8[dst] = pos8[src];
    ema8[dst] = ema8[src];
  }
  for (int k = tid; k < nm16; k += kCompThreads) {
    const int src = mv16[2 * k], dst = mv16[2 * k + 1];
    pos16[dst] = pos16[src];
    ema16[dst] = ema16[src];
  }
  // ---- 4. INT8 data of every KV head (slot n8' is free once its mover has left)
  const int per = dm.Hkv * D;
  for (int i = tid; i < nm8 * per; i += kCompThreads) {
    const int k = i / per, r = i % per, hk = r / D, ch = r % D;
    const size_t ub = ((size_t)lb * dm.Hkv + hk) * (size_t)dm.cap8 * D;
    const int src = mv8[2 * k], dst = mv8[2 * k + 1];
    c.k8[ub + k8_off(dst, ch, D)] = c.k8[ub + k8_off(src, ch, D)];
    c.v8[ub + v8_off(dst, ch, D)] = c.v8[ub + v8_off(src, ch, D)];
  }
  __syncthreads();
  // ---- 5. demotion into INT8 slot `dest`, read from the untouched window slot jd.
  // One thread per (KV head, channel) and kind: a = |x|; a new maximum first
  // requantises that channel's stored codes (slots < n8'), then the token is coded
  // at the channel's absmax / 127.  Grown channels are listed in LDS and their
  // codes requantised by the whole workgroup (a list overflow, only possible when
  // very many channels grow at once, is handled by the owning thread).
  if (dest >= 0) {
    if (tid == 0) {
      pos8[dest] = dpos;
      ema8[dest] = dema;
      s_ngrown = 0;
    }
    __syncthreads();
    for (int pi = tid; pi < 2 * per; pi += kCompThreads) {
      const int kind = pi / per, hc = pi % per, hk = hc / D, ch = hc % D;
      const size_t u = (size_t)lb * dm.Hkv + hk;
      const float x = h16_to_f32(
          kind == 0 ? ((const uint16_t*)c.k16)[u * (size_t)dm.cap16 * D + k16_off(jd, ch, D)]
                    : ((const uint16_t*)c.v16)[u * (size_t)dm.cap16 * D + v16_off(jd, ch, D)],
          dm.bf16);
      int8_t* base = (kind == 0 ? c.k8 : c.v8) + u * (size_t)dm.cap8 * D;
      float* am = (kind == 0 ? c.k_amax : c.v_amax) + u * D + ch;
      const float old = *am, a = fabsf(x);
      const float amax = a > old ? a : old;
      const float s_new = amax / 127.0f;
      if (a > old) {
        *am = amax;
        const float s_old = old / 127.0f;
        const int slot = atomicAdd(&s_ngrown, 1);
        if (slot < kMaxGrown) {
          s_grown[slot] = pi;
          s_gold[slot] = s_old;
          s_gnew[slot] = s_new;
        } else {
          for (int tok = 0; tok < n8n; ++tok) {
            int8_t* p = base + (kind == 0 ? k8_off(tok, ch, D) : v8_off(tok, ch, D));
            *p = quant_code((float)(*p) * s_old, s_new);
          }
        }
      }
      base[kind == 0 ? k8_off(dest, ch, D) : v8_off(dest, ch, D)] = quant_code(x, s_new);
    }
    __syncthreads();
    const int ng = min(s_ngrown, kMaxGrown);
    for (int i = tid; i < ng * n8n; i += kCompThreads) {
      const int e = i % ng, tok = i / ng;
      const int pi = s_grown[e], kind = pi / per, hc = pi % per, hk = hc / D, ch = hc % D;
      const size_t u = (size_t)lb * dm.Hkv + hk;
      int8_t* p = (kind == 0 ? c.k8 + u * (size_t)dm.cap8 * D + k8_off(tok, ch, D)
                             : c.v8 + u * (size_t)dm.cap8 * D + v8_off(tok, ch, D));
      *p = quant_code((float)(*p) * s_gold[e], s_gnew[e]);
    }
  }
  __syncthreads();
  // ---- 6. window data of every KV head
  for (int i = tid; i < nm16 * per; i += kCompThreads) {
    const int k = i / per, r = i % per, hk = r / D, ch = r % D;
    const size_t ub = ((size_t)lb * dm.Hkv + hk) * (size_t)dm.cap16 * D;
    const int src = mv16[2 * k], dst = mv16[2 * k + 1];
    uint16_t* k16 = (uint16_t*)c.k16 + ub;
    uint16_t* v16 = (uint16_t*)c.v16 + ub;
    k16[k16_off(dst, ch, D)] = k16[k16_off(src, ch, D)];
    v16[v16_off(dst, ch, D)] = v16[v16_off(src, ch, D)];
  }
  if (tid == 0) {
    int32_t* pl = plan_all + (size_t)lb * 16;
    pl[0] = n8n;
    pl[1] = nm8;
    pl[2] = n16n;
    pl[3] = nm16;
    pl[4] = jd;
    pl[5] = dest;
    if (jd >= 0 && dest < 0) atomicOr(c.status, (int)CONF_ST_INT8_FULL);
    c.n8[lb] = n8n + (dest >= 0 ? 1 : 0);
    c.n16[lb] = n16n;
  }
}

void launch_compact(const Dims& dm, const conf_cache& c, int layer0, int nl, const uint8_t* keep,
                    int32_t* plan, int32_t* mv8, int32_t* mv16, uint8_t* wkeep, hipStream_t st) {
  hipLaunchKernelGGL(compact_kernel, dim3(nl * dm.B), dim3(kCompThreads), 0, st, c, dm, layer0,
                     keep, plan, mv8, mv16, wkeep);
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
