// (d) Rank and select: keep the protected window plus the top N - |protected|
// tokens by (composite score desc, position desc); one workgroup per (layer,
// sequence) writes the keep flags to global memory.  The selection itself is
// select_core (select.hpp), shared with the fused selection + compaction kernel.
//
// CONF-KV explainer, Methodology, token ranking and eviction.
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
// per-head compaction then applies.
//
// CONF-KV explainer, Significance and claims: head-wise allocation composes with
// the method; Methodology, token ranking and eviction for the score.
constexpr int kMaxHeadwise = 32;  // KV heads per sequence (n_kv_heads * head_dim <= 2048)

__global__ __launch_bounds__(kSelThreads) void joint_select_kernel(conf_cache c, Dims dm,
                                                                   int layer0,
                                                                   const int32_t* __restrict__ budget,
                                                                   uint8_t* __restrict__ keep_all) {
  __shared__ SelScratch X;
  __shared__ SelMisc M;
  __shared__ int off[kMaxHeadwise + 1], n8s[kMaxHeadwise];
  const int ls = layer0 * dm.nseq + blockIdx.x;  // (layer, sequence)
  const int l = ls / dm.nseq, b = ls % dm.nseq;
  const int hw = dm.hw;
  const int sub0 = ls * hw;  // its first head's (layer, sub-sequence)
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int h = 0; h < hw; ++h) {
      off[h] = acc;
      n8s[h] = c.n8[sub0 + h];
      acc += n8s[h] + c.n16[sub0 + h];
    }
    off[hw] = acc;
  }
  __syncthreads();
  const int n = off[hw];
  const int t = c.t[sub0];  // every head of a sequence appends at each step
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
  rank_core<kSelThreads, false, true>(n, N, t - dm.P, hw, false, tok, keyf, X, M,
                                      [&](int j, int k, uint64_t) {
    const int h = head_of(j), jl = j - off[h];
    uint8_t* keep = keep_all + (size_t)(sub0 + h) * dm.capt;
    keep[jl < n8s[h] ? jl : dm.cap8 + (jl - n8s[h])] = (uint8_t)k;
  });
}

void launch_joint_select(const Dims& dm, const conf_cache& c, int layer0, int nl,
                         const int32_t* budget, uint8_t* keep, hipStream_t st) {
  hipLaunchKernelGGL(joint_select_kernel, dim3(nl * dm.nseq), dim3(kSelThreads), 0, st, c, dm,
                     layer0, budget, keep);
}

}  // namespace confkv
