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

}  // namespace confkv
