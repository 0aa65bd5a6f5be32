// (d) Rank and select: keep the protected window plus the top N - |protected|
// tokens by (composite score desc, position desc); one workgroup per (layer,
// sequence) writes the keep flags to global memory.  The selection itself is
// select_core (select.hpp), shared with the fused selection + compaction kernel.
//
// CONF-KV explainer, Methodology, token ranking and eviction.
#include <atomic>

#include "select.hpp"

namespace confkv {

constexpr int kSelThreads = 1024;

__global__ __launch_bounds__(kSelThreads) void select_kernel(conf_cache c, Dims dm, int layer0,
                                                             const int32_t* __restrict__ budget,
                                                             uint8_t* __restrict__ keep_all) {
  __shared__ SelScratch X;
  __shared__ SelMisc M;
  const int lb = layer0 * dm.B + blockIdx.x;
  const int l = lb / dm.B, b = lb % dm.B;
  const int n8 = c.n8[lb], n16 = c.n16[lb], t = c.t[lb];
  const int N = budget[(size_t)b * dm.L + l];
  uint8_t* keep8 = keep_all + (size_t)lb * dm.capt;
  uint8_t* keep16 = keep8 + dm.cap8;
  select_core<kSelThreads>(c, dm, lb, n8, n16, t, N, X, M, [&](int j, int k, uint64_t) {
    if (j < n8)
      keep8[j] = (uint8_t)k;
    else
      keep16[j - n8] = (uint8_t)k;
  });
}

void launch_select(const Dims& dm, const conf_cache& c, int layer0, int nl, const int32_t* budget,
                   uint8_t* keep, hipStream_t st) {
  hipLaunchKernelGGL(select_kernel, dim3(nl * dm.B), dim3(kSelThreads), 0, st, c, dm, layer0,
                     budget, keep);
}

// Head-wise keep sets: one workgroup per (layer, sequence) ranks the tokens of
// its hw KV heads together (each head is a cache of its own, sub-sequence
// (layer*nseq + b)*hw + h) against hw * budget[b][l] (token, head) pairs.  Each
// head's positions (t-P, t] are protected; the other pairs compete on the
// composite score with e_max over all hw heads, ties by position then head (the
// key's low word is pos*hw + h).  Writes every head's keep flags, which the
// per-head compaction then applies.  With EMA, the EMA update that an attention
// launch left pending comes first (sizes from the attention's snapshot, every
// head's n16 and t advanced here), and the updated (e, tag) pairs stay in the
// key cache for the ranking.  The key cache takes the dynamic LDS.
//
// CONF-KV explainer, Significance and claims: head-wise allocation composes with
// the method; Methodology, token ranking and eviction for the EMA and the score.
constexpr int kMaxHeadwise = 32;  // KV heads per sequence (n_kv_heads * head_dim <= 2048)

template <bool EMA>
__global__ __launch_bounds__(kSelThreads) void joint_select_kernel(
    conf_cache c, Dims dm, int layer0, const int32_t* __restrict__ budget,
    uint8_t* __restrict__ keep_all, const float* __restrict__ massp_all,
    const int32_t* __restrict__ snap, int key_cap) {
#pragma clang fp contract(off)
  extern __shared__ uint64_t dyn_keys[];  // [key_cap] keys, then the 256-bin histogram
  __shared__ SelMisc M;
  __shared__ int off[kMaxHeadwise + 1], n8s[kMaxHeadwise], nws[kMaxHeadwise];
  const int tid = threadIdx.x;
  const int ls = layer0 * dm.nseq + blockIdx.x;  // (layer, sequence)
  const int l = ls / dm.nseq, b = ls % dm.nseq;
  const int hw = dm.hw;
  const int sub0 = ls * hw;  // its first head's (layer, sub-sequence)
  if (tid == 0) {
    int acc = 0;
    for (int h = 0; h < hw; ++h) {
      int n8, n16;
      if constexpr (EMA) {
        n8 = snap[3 * (sub0 + h)];
        nws[h] = snap[3 * (sub0 + h) + 1];
        n16 = nws[h] + (nws[h] < dm.cap16);  // the append, unless the window was full
      } else {
        n8 = c.n8[sub0 + h];
        n16 = c.n16[sub0 + h];
      }
      off[h] = acc;
      n8s[h] = n8;
      acc += n8 + n16;
    }
    off[hw] = acc;
  }
  __syncthreads();
  const int n = off[hw];
  // every head of a sequence appends at each step
  const int t = EMA ? snap[3 * sub0 + 2] + 1 : c.t[sub0];
  const int N = budget[(size_t)b * dm.L + l] * hw;
  // the head holding index j: the last h with off[h] <= j (empty heads skipped)
  auto head_of = [&](int j) {
    int lo = 0, hi = hw;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= j) lo = mid; else hi = mid;
    }
    return lo;
  };
  if constexpr (EMA) {
    // e <- decay*e + (1-decay)*mass, mass = this head's mass row / G (one KV head
    // per cache), the appended token from e = 0 at position t; the same
    // operations as the EMA kernel
    const float hq = (float)dm.Hq;
    const bool cached = n <= key_cap;
    // kT tokens per thread per round, every load of the round issued before the
    // arithmetic (an index past the end reads head 0's first slot, not stored)
    constexpr int kT = 4;
    for (int jb = tid; jb < n; jb += kT * kSelThreads) {
      int hh[kT], jj[kT], po[kT];
      float mr[kT], eo[kT];
#pragma unroll
      for (int k = 0; k < kT; ++k) {
        const int j = jb + k * kSelThreads;
        const int h = j < n ? head_of(j) : 0;
        const int jl = j < n ? j - off[h] : 0;
        const size_t sub = (size_t)(sub0 + h);
        const int n8 = n8s[h];
        hh[k] = h;
        jj[k] = jl;
        mr[k] = massp_all[sub * dm.capt + (jl < n8 ? jl : dm.cap8 + (jl - n8))];
        eo[k] = jl < n8 ? c.ema8[sub * dm.cap8 + jl] : c.ema16[sub * dm.cap16 + (jl - n8)];
        po[k] = jl < n8 ? c.pos8[sub * dm.cap8 + jl] : c.pos16[sub * dm.cap16 + (jl - n8)];
      }
#pragma unroll
      for (int k = 0; k < kT; ++k) {
        const int j = jb + k * kSelThreads;
        if (j >= n) continue;
        const int h = hh[k], jl = jj[k], n8 = n8s[h];
        const size_t sub = (size_t)(sub0 + h);
        const float m = (0.f + mr[k]) / hq;
        float e;
        int p = po[k];
        if (jl < n8) {
          e = dm.decay * eo[k] + dm.one_minus_decay * m;
          c.ema8[sub * dm.cap8 + jl] = e;
        } else if (jl - n8 == nws[h]) {
          e = dm.one_minus_decay * m;  // decay * 0 + (1 - decay) * mass
          p = t;
          c.ema16[sub * dm.cap16 + nws[h]] = e;
          c.pos16[sub * dm.cap16 + nws[h]] = p;
        } else {
          e = dm.decay * eo[k] + dm.one_minus_decay * m;
          c.ema16[sub * dm.cap16 + (jl - n8)] = e;
        }
        if (cached)
          dyn_keys[j] = ((uint64_t)__float_as_uint(e) << 32) |
                        ((uint32_t)p * (uint32_t)hw + (uint32_t)h);
      }
    }
    if (tid < hw) {  // the per-head compaction reads the sizes from the cache
      c.n16[sub0 + tid] = off[tid + 1] - off[tid] - n8s[tid];
      c.t[sub0 + tid] = t;
    }
    __syncthreads();  // the EMA and the appended positions are in memory for the ranking
  }
  auto tok = [&](int j, float& e, uint32_t& tag) {
    const int h = head_of(j), jl = j - off[h];
    const size_t lb = (size_t)(sub0 + h);
    int p;
    if (jl < n8s[h]) {
      e = c.ema8[lb * dm.cap8 + jl];
      p = c.pos8[lb * dm.cap8 + jl];
    } else {
      e = c.ema16[lb * dm.cap16 + (jl - n8s[h])];
      p = c.pos16[lb * dm.cap16 + (jl - n8s[h])];
    }
    tag = (uint32_t)p * (uint32_t)hw + (uint32_t)h;
  };
  auto keyf = [&](float e, float em, uint32_t tag) -> uint64_t {
    return sel_key(e, em, (int)(tag / (uint32_t)hw), t, dm.s_ema, dm.s_rec, tag);
  };
  rank_core<kSelThreads, true, true>(n, N, t - dm.P, hw, EMA, tok, keyf, dyn_keys,
                                     (unsigned*)(dyn_keys + key_cap), key_cap, M,
                                     [&](int j, int k, uint64_t) {
    const int h = head_of(j), jl = j - off[h];
    uint8_t* keep = keep_all + (size_t)(sub0 + h) * dm.capt;
    keep[jl < n8s[h] ? jl : dm.cap8 + (jl - n8s[h])] = (uint8_t)k;
  });
}

// Dynamic LDS of the head-wise selection: as much of the workgroup's LDS as the
// device allows, less the static part and a margin.  Read and set once per device.
static int joint_dyn_bytes() {
  static std::atomic<int> bytes_of[kMaxDevices];  // 0: not yet set on that device
  const int slot = current_device_slot();
  if (slot >= 0) {
    const int b = bytes_of[slot].load(std::memory_order_acquire);
    if (b > 0) return b;
  }
  int dev = 0, max_lds = 65536;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
          hipSuccess)
    max_lds = 65536;
  const int want = max_lds - 2048;  // the static part (about 500 bytes) and a margin
  const int bytes = want < 32768 ? 32768 : want;
  (void)hipFuncSetAttribute((const void*)joint_select_kernel<true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  (void)hipFuncSetAttribute((const void*)joint_select_kernel<false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (slot >= 0) bytes_of[slot].store(bytes, std::memory_order_release);
  return bytes;
}

void launch_joint_select(const Dims& dm, const conf_cache& c, int layer0, int nl,
                         const int32_t* budget, uint8_t* keep, const float* massp,
                         const int32_t* snap, bool with_ema, hipStream_t st) {
  const int bytes = joint_dyn_bytes();
  const int key_cap = (bytes - 256 * (int)sizeof(unsigned)) / (int)sizeof(uint64_t);
  if (with_ema)
    hipLaunchKernelGGL(joint_select_kernel<true>, dim3(nl * dm.nseq), dim3(kSelThreads), bytes,
                       st, c, dm, layer0, budget, keep, massp, snap, key_cap);
  else
    hipLaunchKernelGGL(joint_select_kernel<false>, dim3(nl * dm.nseq), dim3(kSelThreads), bytes,
                       st, c, dm, layer0, budget, keep, massp, snap, key_cap);
}

}  // namespace confkv
