// Cache maintenance kernels: reset, prefill ingest, compaction + demotion, and
// export of one (layer, sequence).
//
// CONF-KV explainer, Methodology, system integration: the newest W tokens stay
// 16-bit, older kept tokens are INT8 per head and channel (mixed-precision
// storage); contiguous compaction keeps a dense layout with no indirection
// tables (implementation).  Token ranking and eviction: EMA attention mass.
#include "ema.hpp"
#include "select.hpp"

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

// The 16-bit window arrays to zero.  The attention reads whole window halves and
// gives the slots past a unit's count probability 0, which only cancels a finite
// value; every later write into the window stores a caller-supplied or moved value.
__global__ void zero16_kernel(uint4* __restrict__ a, uint4* __restrict__ b, size_t n) {
  const uint4 z = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    a[i] = z;
    b[i] = z;
  }
}

void launch_reset(const Dims& dm, const conf_cache& c, hipStream_t st) {
  const size_t n = (size_t)dm.L * dm.B * dm.Hkv * dm.D;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(reset_kernel, dim3((unsigned)blocks), dim3(256), 0, st, c, dm);
  const size_t n16 = (size_t)dm.L * dm.B * dm.Hkv * dm.cap16 * dm.D * 2 / 16;
  const size_t zb = (n16 + 255) / 256;
  hipLaunchKernelGGL(zero16_kernel, dim3((unsigned)(zb < 4096 ? zb : 4096)), dim3(256), 0, st,
                     (uint4*)c.k16, (uint4*)c.v16, n16);
}

// ---------------------------------------------------------------- ingest
// Prefill of L0 tokens per unit: positions < L0 - W become INT8 (e4m3 under ARKV)
// with the absmax over exactly those tokens (a sliding window drops them); the
// rest go to the window.  Three launches, spread over the whole GPU rather than one
// workgroup per unit: the units' absmax rows are cleared; every chunk of
// kIngChunk tokens folds its per-channel |x| maxima into them with atomic maxima on
// the float bits (exact: for x >= 0 the bits order like the values); then every
// 64-token tile is quantised (or, for the window, copied) through LDS, so that
// each load and store is a 16-byte access.
constexpr int kIngThreads = 256;
constexpr int kIngChunk = 1024;  // tokens per absmax workgroup

struct IngGeom {
  int old, n8, nw;  // positions older than the window; INT8 tokens; window tokens
};
__host__ __device__ inline IngGeom ing_geom(const Dims& dm, int L0) {
  IngGeom g;
  g.old = L0 > dm.W ? L0 - dm.W : 0;
  g.n8 = dm.policy == CONF_POLICY_WINDOW ? 0 : g.old;
  g.nw = L0 - g.old;
  return g;
}

__global__ __launch_bounds__(kIngThreads) void ingest_clear_kernel(conf_cache c, Dims dm,
                                                                    int layer0, int nunits) {
  const size_t u0 = (size_t)layer0 * dm.B * dm.Hkv;
  const size_t n = (size_t)nunits * dm.D;
  for (size_t i = (size_t)blockIdx.x * kIngThreads + threadIdx.x; i < n;
       i += (size_t)gridDim.x * kIngThreads) {
    c.k_amax[u0 * dm.D + i] = 0.f;
    c.v_amax[u0 * dm.D + i] = 0.f;
  }
}

// grid (units, chunks): per-channel max |x| of tokens [kIngChunk*y, ...) below n8
__global__ __launch_bounds__(kIngThreads) void ingest_amax_kernel(conf_cache c, Dims dm,
                                                                   int layer0, int L0,
                                                                   const uint16_t* __restrict__ kp,
                                                                   const uint16_t* __restrict__ vp) {
  const int unit_local = blockIdx.x;
  const size_t u = (size_t)layer0 * dm.B * dm.Hkv + unit_local;
  const int D = dm.D, G8 = D / 8;  // 8-channel groups per token
  const IngGeom gm = ing_geom(dm, L0);
  const int t0 = blockIdx.y * kIngChunk, t1 = min(gm.n8, t0 + kIngChunk);
  const uint16_t* ks = kp + (size_t)unit_local * L0 * D;
  const uint16_t* vs = vp + (size_t)unit_local * L0 * D;
  const int cg = threadIdx.x % G8, rows = kIngThreads / G8;
  float mk[8], mv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mk[e] = mv[e] = 0.f;
  for (int tok = t0 + threadIdx.x / G8; tok < t1; tok += rows) {
    const uint4 a = *(const uint4*)(ks + (size_t)tok * D + 8 * cg);
    const uint4 b = *(const uint4*)(vs + (size_t)tok * D + 8 * cg);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mk[e] = fmaxf(mk[e], fabsf(h16_to_f32((uint16_t)(wa[e >> 1] >> (16 * (e & 1))), dm.bf16)));
      mv[e] = fmaxf(mv[e], fabsf(h16_to_f32((uint16_t)(wb[e >> 1] >> (16 * (e & 1))), dm.bf16)));
    }
  }
  // fold the rows that share a channel group: [row][D] in LDS, then one thread per channel
  __shared__ float sk[kIngThreads * 8], sv[kIngThreads * 8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    sk[(threadIdx.x / G8) * D + 8 * cg + e] = mk[e];
    sv[(threadIdx.x / G8) * D + 8 * cg + e] = mv[e];
  }
  __syncthreads();
  if ((int)threadIdx.x < D) {
    float a = 0.f, b = 0.f;
    for (int r = 0; r < rows; ++r) {
      a = fmaxf(a, sk[r * D + threadIdx.x]);
      b = fmaxf(b, sv[r * D + threadIdx.x]);
    }
    atomicMax((unsigned int*)&c.k_amax[u * D + threadIdx.x], __float_as_uint(a));
    atomicMax((unsigned int*)&c.v_amax[u * D + threadIdx.x], __float_as_uint(b));
  }
}

// grid (units, INT8 tiles + window tiles): one 64-token tile of one unit.  The
// tile's K and V rows are staged in LDS with 16-byte loads; a key tile is then
// written as 16-channel runs of one token, a value tile as 16-token runs of one
// channel (8 for the window), each one 16-byte store.
__global__ __launch_bounds__(kIngThreads) void ingest_tile_kernel(conf_cache c, Dims dm, int layer0,
                                                                   int L0,
                                                                   const uint16_t* __restrict__ kp,
                                                                   const uint16_t* __restrict__ vp) {
#pragma clang fp contract(off)
  const int unit_local = blockIdx.x;
  const int hk = unit_local % dm.Hkv;
  const int lb = layer0 * dm.B + unit_local / dm.Hkv;
  const size_t u = (size_t)lb * dm.Hkv + hk;
  const int D = dm.D;
  const IngGeom gm = ing_geom(dm, L0);
  const bool fp8 = dm.policy == CONF_POLICY_ARKV;  // ARKV quantises to e4m3
  const int nt8 = (gm.n8 + kTile - 1) / kTile;
  const bool i8 = (int)blockIdx.y < nt8;
  const int tile = i8 ? blockIdx.y : blockIdx.y - nt8;
  const int base = kTile * tile;                            // first slot of the tile
  const int cnt = min(kTile, (i8 ? gm.n8 : gm.nw) - base);  // slots of the tile in use
  const int src0 = (i8 ? 0 : gm.old) + base;                 // its first prefill position
  const uint16_t* ks = kp + ((size_t)unit_local * L0 + src0) * D;
  const uint16_t* vs = vp + ((size_t)unit_local * L0 + src0) * D;
  __shared__ uint4 tk[kTile * 128 / 8], tv[kTile * 128 / 8];  // [64][D] 16-bit, 16-byte chunks
  __shared__ float sk[128], sv[128];
  const int G8 = D / 8;
  for (int i = threadIdx.x; i < kTile * G8; i += kIngThreads) {
    const int r = i / G8;
    const uint4 z = {0u, 0u, 0u, 0u};
    tk[i] = r < cnt ? *(const uint4*)(ks + (size_t)i * 8) : z;
    tv[i] = r < cnt ? *(const uint4*)(vs + (size_t)i * 8) : z;
  }
  if (i8 && (int)threadIdx.x < D) {
    sk[threadIdx.x] = c.k_amax[u * D + threadIdx.x] / code_max(fp8);
    sv[threadIdx.x] = c.v_amax[u * D + threadIdx.x] / code_max(fp8);
  }
  __syncthreads();
  const uint16_t* hk16 = (const uint16_t*)tk;
  const uint16_t* hv16 = (const uint16_t*)tv;
  if (i8) {
    int8_t* k8 = c.k8 + u * (size_t)dm.cap8 * D;
    int8_t* v8 = c.v8 + u * (size_t)dm.cap8 * D;
    // keys: (token, 16-channel group), token fastest
    for (int i = threadIdx.x; i < kTile * (D / 16); i += kIngThreads) {
      const int r = i % kTile, cg = i / kTile;
      if (r >= cnt) continue;
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t x = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ch = 16 * cg + 4 * q + e;
          const int8_t code = quant8(h16_to_f32(hk16[r * D + ch], dm.bf16), sk[ch], fp8);
          x |= (uint32_t)(uint8_t)code << (8 * e);
        }
        w[q] = x;
      }
      *(uint4*)(k8 + k8_off(base + r, 16 * cg, D)) = (uint4){w[0], w[1], w[2], w[3]};
    }
    // values: (token group g, channel), channel fastest; the 16 bytes hold tokens
    // 32u + 16a + 4g + b at byte 8u + 4a + b (slots past cnt get code 0)
    for (int i = threadIdx.x; i < 4 * D; i += kIngThreads) {
      const int ch = i % D, g = i / D;
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t x = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int byte = 4 * q + e, uu = byte >> 3, a = (byte >> 2) & 1, b = byte & 3;
          const int r = 32 * uu + 16 * a + 4 * g + b;
          const int8_t code =
              r < cnt ? quant8(h16_to_f32(hv16[r * D + ch], dm.bf16), sv[ch], fp8) : (int8_t)0;
          x |= (uint32_t)(uint8_t)code << (8 * e);
        }
        w[q] = x;
      }
      // byte 0 of the run is slot 4g (u = a = b = 0)
      *(uint4*)(v8 + v8_off(base + 4 * g, ch, D)) = (uint4){w[0], w[1], w[2], w[3]};
    }
  } else {
    uint16_t* k16 = (uint16_t*)c.k16 + u * (size_t)dm.cap16 * D;
    uint16_t* v16 = (uint16_t*)c.v16 + u * (size_t)dm.cap16 * D;
    // keys: (token, 8-channel group) -> 16 contiguous bytes of the key tile
    for (int i = threadIdx.x; i < kTile * G8; i += kIngThreads) {
      const int r = i % kTile, cg = i / kTile;
      if (r >= cnt) continue;
      *(uint4*)(k16 + k16_off(base + r, 8 * cg, D)) = tk[r * G8 + cg];
    }
    // values: per 32-token half u, (token group g, channel) -> tokens 16a + 4g + b
    // at element 4a + b; only whole halves in use are written, a partial one
    // element by element (the slots past nw keep the zeros of the reset)
    for (int i = threadIdx.x; i < 2 * 4 * D; i += kIngThreads) {
      const int ch = i % D, g = (i / D) % 4, uu = i / (4 * D);
      uint16_t e16[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 32 * uu + 16 * (e >> 2) + 4 * g + (e & 3);
        e16[e] = r < cnt ? hv16[r * D + ch] : (uint16_t)0;
      }
      uint16_t* dst = v16 + v16_off(base + 32 * uu + 4 * g, ch, D);  // element 0 of the run
      if (32 * uu + 32 <= cnt) {
        *(uint4*)dst = (uint4){e16[0] | (uint32_t)e16[1] << 16, e16[2] | (uint32_t)e16[3] << 16,
                               e16[4] | (uint32_t)e16[5] << 16, e16[6] | (uint32_t)e16[7] << 16};
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 32 * uu + 16 * (e >> 2) + 4 * g + (e & 3);
          if (r < cnt) dst[e] = e16[e];
        }
      }
    }
  }
  // positions and EMA of the (layer, sequence), written by its KV head 0
  if (hk == 0) {
    for (int r = threadIdx.x; r < cnt; r += kIngThreads) {
      if (i8) {
        c.pos8[(size_t)lb * dm.cap8 + base + r] = base + r;
        c.ema8[(size_t)lb * dm.cap8 + base + r] = 0.f;
      } else {
        c.pos16[(size_t)lb * dm.cap16 + base + r] = gm.old + base + r;
        c.ema16[(size_t)lb * dm.cap16 + base + r] = 0.f;
      }
    }
    if (blockIdx.y == 0 && threadIdx.x == 0) {
      c.n8[lb] = gm.n8;
      c.n16[lb] = gm.nw;
      c.t[lb] = L0 - 1;
    }
  }
}

void launch_ingest(const Dims& dm, const conf_cache& c, int layer0, int nl, int L0, const void* k,
                   const void* v, hipStream_t st) {
  const int units = nl * dm.B * dm.Hkv;
  const IngGeom gm = ing_geom(dm, L0);
  const size_t na = (size_t)units * dm.D;
  const size_t cb = (na + kIngThreads - 1) / kIngThreads;
  hipLaunchKernelGGL(ingest_clear_kernel, dim3((unsigned)(cb < 1024 ? cb : 1024)),
                     dim3(kIngThreads), 0, st, c, dm, layer0, units);
  if (gm.n8 > 0)
    hipLaunchKernelGGL(ingest_amax_kernel, dim3(units, (gm.n8 + kIngChunk - 1) / kIngChunk),
                       dim3(kIngThreads), 0, st, c, dm, layer0, L0, (const uint16_t*)k,
                       (const uint16_t*)v);
  const int tiles = (gm.n8 + kTile - 1) / kTile + (gm.nw + kTile - 1) / kTile;
  if (tiles > 0)
    hipLaunchKernelGGL(ingest_tile_kernel, dim3(units, tiles), dim3(kIngThreads), 0, st, c, dm,
                       layer0, L0, (const uint16_t*)k, (const uint16_t*)v);
}

// ---------------------------------------------------------------- compaction + demotion
// One workgroup of 512 threads per (layer, sequence), built to need few global
// round trips (one token or so moves per step in the steady state):
//  1. Keep flags are read once (into LDS).  The window flag of the token at
//     position t - W is cleared: it is demoted, not kept in place.
//  2. In each region the k-th hole below the new end receives the k-th survivor
//     above it (both in slot order), so the layout stays dense; a demotee takes
//     the first INT8 hole itself.  The move lists come from ballot ranks, in LDS
//     (the workspace holds what does not fit).
//  3. INT8 moves (data, position, EMA) run while every (KV head, channel, K|V)
//     thread of the demotion reads its 16-bit value and absmax and works out the
//     new absmax and code.
//  4. After a barrier: the demotee's codes and metadata land in its INT8 slot,
//     window moves (data, position, EMA; the demotee's window slot has been
//     read), and channels whose absmax grew requantise their stored codes
//     (listed in LDS and spread over the workgroup; an overflow of the list is
//     handled by the owning threads).
// plan: [0] n8' (kept INT8 tokens) [1] INT8 moves [2] n16' [3] window moves
//       [4] demotee's window slot or -1 [5] its INT8 slot or -1  (kept in the
//       workspace for inspection; the INT8 region ends at n8' + (demoted))
constexpr int kCompThreads = 512;  // every (layer, sequence) workgroup resident at once
typedef uint32_t cu4 __attribute__((ext_vector_type(4)));  // a 16-byte chunk
constexpr int kCompWaves = kCompThreads / 64;
constexpr int kMaxGrown = 512;    // grown channels requantised by the whole workgroup
constexpr int kLdsFlags8 = 4096;  // INT8 keep flags cached in LDS (beyond: global memory)
constexpr int kLdsFlags16 = 2048; // window keep flags cached in LDS (beyond: workspace)
constexpr int kLdsMoves = 2048;   // move-list pairs per region kept in LDS (beyond: workspace)

// A compaction configuration: threads per workgroup and the LDS capacities of the
// flag caches, move lists and grown-channel list (what does not fit goes to
// global memory).  A workgroup spreads the 2*Hkv*d (K|V, KV head, channel)
// triples of a demotion over its threads, at most eight each.
template <int NT_, int F8_, int F16_, int MV_, int MG_>
struct CompCfg {
  static constexpr int NT = NT_, W = NT_ / 64, F8 = F8_, F16 = F16_, MV = MV_, MG = MG_;
};
// one (layer, sequence) with all its KV heads
using CompBig = CompCfg<kCompThreads, kLdsFlags8, kLdsFlags16, kLdsMoves, kMaxGrown>;
// one (sequence, KV head) of a head-wise cache: 2*d <= 256 triples, and little LDS,
// so that many workgroups share a compute unit
using CompSmall = CompCfg<128, 2048, 1024, 256, 256>;

template <class C>
struct CompFlagsT {  // keep flags cached in LDS
  uint8_t k8[C::F8];
  uint8_t k16[C::F16];
};
template <class C>
struct CompScratchT {  // move lists and the grown-channel list
  int mv8[2 * C::MV];   // (source, destination) pairs
  int mv16[2 * C::MV];
  int grown[C::MG];
  float gold[C::MG], gnew[C::MG];
};
template <class C>
struct CompMiscT {
  int wcnt[2][C::W];
  int c8[C::W], c16[C::W];
  int jd, ngrown, first_hole;
};
using CompFlags = CompFlagsT<CompBig>;
using CompScratch = CompScratchT<CompBig>;
using CompMisc = CompMiscT<CompBig>;

// Ordered ranks of the slots of [0, max(n, nnew)) that are holes (slot < nnew,
// not kept; slots >= n count as not kept) or survivors (slot >= nnew, kept).  The
// first `skip` holes are set aside (the first one's slot goes to *first_hole);
// hole skip + k receives survivor k: pair k = (survivor k, hole skip + k).
// `flag(i)` reads slot i's keep flag (i < n).  Returns the number of pairs.
// With ntb > 0, tile_base[T] (T < ntb) receives the number of holes in slots
// [0, 64T), set-aside ones included.  Every thread must call it.
//
// Each wavefront takes a contiguous range of 64-slot tiles.  It counts its holes
// and survivors with ballots, one barrier exchanges the counts, and a second walk
// over its tiles writes the pairs from its offsets: two barriers in all, where a
// workgroup-wide pass per 512 slots took two per pass (the steady state's caches
// have a hole or two in thousands of slots).  The flags of four tiles are read
// together.
template <class C, typename Flag>
__device__ int build_moves(int n, int nnew, int skip, Flag flag, int* lds_mv, int32_t* gl_mv,
                           int (*wcnt)[C::W], int* first_hole, int32_t* tile_base = nullptr,
                           int ntb = 0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int end = n > nnew ? n : nnew;
  const int ntiles = (end + 63) >> 6;
  const int t0 = (int)((long long)ntiles * wave / C::W);
  const int t1 = (int)((long long)ntiles * (wave + 1) / C::W);
  const unsigned long long below = (1ull << lane) - 1ull;
  constexpr int kU = 4;
  auto tile_masks = [&](int T0, unsigned long long (&bh)[kU], unsigned long long (&bs)[kU]) {
    bool kk[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = 64 * (T0 + u) + lane;
      kk[u] = T0 + u < t1 && i < n && flag(i);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = 64 * (T0 + u) + lane;
      const bool in = T0 + u < t1;
      bh[u] = __ballot(in && i < nnew && !kk[u]);
      bs[u] = __ballot(in && i >= nnew && kk[u]);
    }
  };
  int ch = 0, cs = 0;
  for (int T0 = t0; T0 < t1; T0 += kU) {
    unsigned long long bh[kU], bs[kU];
    tile_masks(T0, bh, bs);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      ch += __popcll(bh[u]);
      cs += __popcll(bs[u]);
    }
  }
  if (lane == 0) {
    wcnt[0][wave] = ch;
    wcnt[1][wave] = cs;
  }
  __syncthreads();
  int hb = 0, sb = 0, th = 0;
  for (int w = 0; w < C::W; ++w) {
    const int a = wcnt[0][w], b = wcnt[1][w];
    hb += w < wave ? a : 0;
    sb += w < wave ? b : 0;
    th += a;
  }
  for (int T0 = t0; T0 < t1; T0 += kU) {
    unsigned long long bh[kU], bs[kU];
    tile_masks(T0, bh, bs);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (T0 + u >= t1) break;  // uniform
      const int i = 64 * (T0 + u) + lane;
      if (lane == 0 && T0 + u < ntb) tile_base[T0 + u] = hb;
      if ((bh[u] >> lane) & 1ull) {
        const int r = hb + __popcll(bh[u] & below) - skip;
        if (r < 0) {
          if (r == -skip) *first_hole = i;
        } else if (r < C::MV) {
          lds_mv[2 * r + 1] = i;
        } else {
          gl_mv[2 * r + 1] = i;
        }
      }
      if ((bs[u] >> lane) & 1ull) {
        const int r = sb + __popcll(bs[u] & below);
        if (r < C::MV) lds_mv[2 * r] = i; else gl_mv[2 * r] = i;
      }
      hb += __popcll(bh[u]);
      sb += __popcll(bs[u]);
    }
  }
  __syncthreads();  // the lists, the first hole and the tile counts are complete
  return th - skip;  // holes below the new end, less those set aside = survivors above it
}

template <class C>
__device__ inline int mv_at(const int* lds_mv, const int32_t* gl_mv, int e) {
  return e < 2 * C::MV ? lds_mv[e] : gl_mv[e];
}

// Bulk copy of `total` elements, element i from src(i) to dst(i), spread over the
// workgroup: each thread loads a batch of NB elements into registers and only
// then stores them.  Sources are survivors above the new end and destinations
// holes below it, so no store of a batch can feed a load of a later one; batching
// keeps the loads of a batch in flight together (a plain loop waits on every load,
// since the compiler cannot prove the store does not alias the next load).
template <int NT, int NB, typename T, typename Src, typename Dst>
__device__ inline void bulk_copy(int total, Src src, Dst dst) {
  for (int i0 = threadIdx.x; i0 < total; i0 += NT * NB) {
    T v[NB];
#pragma unroll
    for (int e = 0; e < NB; ++e) {
      const int i = i0 + e * NT;
      if (i < total) v[e] = *src(i);
    }
#pragma unroll
    for (int e = 0; e < NB; ++e) {
      const int i = i0 + e * NT;
      if (i < total) *dst(i) = v[e];
    }
  }
}

// Bulk INT8 value moves by destination run.  A value tile keeps the 16 tokens of
// each group g in one 16-byte run per channel, so a moved token's bytes lie one per
// run, 16 bytes apart: moved token by token, every byte is a store of its own into
// a line it shares with 15 other tokens.  Here each wavefront takes one (KV head,
// destination tile) at a time and rebuilds the tile's runs whole: it reads a run,
// puts each hole's byte from the survivor that fills it (byte loads, every one of
// a run issued before the first wait, those of slots that receive nothing at
// kNoItem) and writes the run back, so that the stores are 16 bytes per lane and
// contiguous over the lanes.  Hole r (over all holes in slot order, less the
// `skip` set aside) takes survivor r: its rank is tile_base[T] plus the tile's holes
// below it.  Each run belongs to one item; the bytes of slots that receive nothing
// are written back as read (survivors in the last tile, which are sources, keep
// their values).  All threads call it; no barrier.
template <class C, typename Flag>
__device__ void v8_moves_by_run(const conf_cache& c, const Dims& dm, int lb, int n8, int n8end,
                                int skip, Flag flag, const int* lds_mv, const int32_t* gl_mv,
                                const int32_t* tile_base) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int D = dm.D;
  const int ntiles = (n8end + 63) >> 6;
  const uint32_t tile_bytes = (uint32_t)(kTile * D);
  for (int item = wave; item < ntiles * dm.Hkv; item += C::W) {
    const int T = item / dm.Hkv, hk = item % dm.Hkv;
    const int s = 64 * T + lane;
    const bool hole = s < n8end && !(s < n8 && flag(s));
    const unsigned long long bh = __ballot(hole);
    const int rank = tile_base[T] + __popcll(bh & ((1ull << lane) - 1ull)) - skip;
    const int src = hole && rank >= 0 ? mv_at<C>(lds_mv, gl_mv, 2 * rank) : -1;
    if (__ballot(src >= 0) == 0ull) continue;  // nothing lands in this tile
    const rsrc_t rv = make_rsrc(c.v8 + ((size_t)lb * dm.Hkv + hk) * (size_t)dm.cap8 * D,
                                (uint32_t)dm.cap8 * D);
    // lane `lane` takes the runs (g, ch) = divmod(lane + 64 i, D), i = 0 .. 4D/64 - 1
    for (int i = 0; i < 4 * D / 64; ++i) {
      const int g = (64 * i) / D, ch = (64 * i) % D + lane;  // g is uniform
      const uint32_t ro = (uint32_t)T * tile_bytes + (uint32_t)(g * D + ch) * 16u;
      cu4 run = __builtin_bit_cast(cu4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)ro, 0, 0));
      uint32_t by[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        // byte x of a run is slot 32u + 16a + 4g + b of the tile, x = 8u + 4a + b
        const int j = 32 * (x >> 3) + 16 * ((x >> 2) & 1) + 4 * g + (x & 3);
        const int sx = __builtin_amdgcn_readlane(src, j);
        const uint32_t off = sx >= 0 ? (uint32_t)v8_off(sx, ch, D) : kNoItem;
        by[x] = __builtin_amdgcn_raw_buffer_load_b8(rv, (int)off, 0, 0);
      }
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int j = 32 * (x >> 3) + 16 * ((x >> 2) & 1) + 4 * g + (x & 3);
        if (__builtin_amdgcn_readlane(src, j) >= 0) {
          const int sh = 8 * (x & 3);
          run[x >> 2] = (run[x >> 2] & ~(0xffu << sh)) | ((by[x] & 0xffu) << sh);
        }
      }
      __builtin_amdgcn_raw_buffer_store_b128(run, rv, (int)ro, 0, 0);
    }
  }
}

// Steps 2-4 of the compaction for one (layer, sequence), once the keep flags are
// known: F holds those of slots below kLdsFlags8 / kLdsFlags16, keep8 / wkeep (in
// global memory) the others; the window flag of the demotee (window slot jd, or
// -1) is already cleared, and n8n / n16n count the kept INT8 / window tokens.
// M.ngrown must be 0.  All kCompThreads threads call it.
template <class C>
__device__ void compact_core(const conf_cache& c, const Dims& dm, int lb, int n8, int n16,
                             int n8n, int n16n, int jd, const uint8_t* keep8, const uint8_t* wkeep,
                             CompFlagsT<C>& F, CompScratchT<C>& X, CompMiscT<C>& M, int32_t* plan_all,
                             int32_t* mv8_all, int32_t* mv16_all) {
#pragma clang fp contract(off)
  const int tid = threadIdx.x;
  const int D = dm.D;
  const bool fp8 = dm.policy == CONF_POLICY_ARKV;  // e4m3 codes in place of INT8
  const float cmax = code_max(fp8);
  int32_t* pos8 = c.pos8 + (size_t)lb * dm.cap8;
  float* ema8 = c.ema8 + (size_t)lb * dm.cap8;
  int32_t* pos16 = c.pos16 + (size_t)lb * dm.cap16;
  float* ema16 = c.ema16 + (size_t)lb * dm.cap16;
  int32_t* mv8 = mv8_all + (size_t)lb * dm.cap8;
  int32_t* mv16 = mv16_all + (size_t)lb * dm.cap16;
  // ---- 2. move lists.  With a demotee, the INT8 region grows to n8' + 1 and the
  // demotee takes its first hole (in the steady state: the slot of the evicted
  // INT8 token, so nothing moves); without one it ends at n8'.
  const bool demote = jd >= 0 && n8n < dm.cap8;
  const int n8end = n8n + (demote ? 1 : 0);
  auto flag8 = [&](int i) { return i < C::F8 ? F.k8[i] != 0 : keep8[i] != 0; };
  // per-tile hole counts for the run-based value moves, in the part of the
  // workspace move list that the LDS list stands for (entries below 2 * C::MV)
  const int ntiles8 = (n8end + 63) >> 6;
  const int ntb = ntiles8 <= 2 * C::MV ? ntiles8 : 0;
  const int nm8 = build_moves<C>(n8, n8end, demote ? 1 : 0, flag8, X.mv8, mv8, M.wcnt,
                                 &M.first_hole, mv8, ntb);
  const int nm16 = build_moves<C>(
      n16, n16n, 0, [&](int w) { return w < C::F16 ? F.k16[w] != 0 : wkeep[w] != 0; },
      X.mv16, mv16, M.wcnt, &M.first_hole);
  const int dest = demote ? M.first_hole : -1;  // written by build_moves before its last barrier
  // ---- 3. INT8 moves; the demotion's reads and arithmetic; window-move reads.
  // Steady state (a move or so per region): every load is issued before any
  // store, from registers.  Bulk steps (step 0 after a long prefill) loop.
  const int per = dm.Hkv * D;
  constexpr int kMv = 2;       // move elements per thread in the register path
  constexpr int kDemPer = 8;   // (K|V, KV head, channel) triples per thread: 2*Hkv*d <= 4096 (host-checked)
  const bool fast = nm8 * per <= kMv * C::NT && nm16 * per <= kMv * C::NT &&
                    nm8 <= C::NT && nm16 <= C::NT;
  // loaded values are held widened to 32 bits: packing 8- or 16-bit values into
  // shared registers would make each load wait before the next one issues
  int32_t mk[kMv], mvv[kMv];
  uint32_t wk[kMv], wv[kMv];
  int32_t mp8 = 0, mp16 = 0;
  float me8 = 0.f, me16 = 0.f;
  if (fast) {
#pragma unroll
    for (int e = 0; e < kMv; ++e) {
      const int i = tid + e * C::NT;
      if (i < nm8 * per) {
        const int k = i / per, r = i % per, hk = r / D, ch = r % D;
        const size_t ub = ((size_t)lb * dm.Hkv + hk) * (size_t)dm.cap8 * D;
        const int src = mv_at<C>(X.mv8, mv8, 2 * k);
        mk[e] = c.k8[ub + k8_off(src, ch, D)];
        mvv[e] = c.v8[ub + v8_off(src, ch, D)];
      }
      if (i < nm16 * per) {
        const int k = i / per, r = i % per, hk = r / D, ch = r % D;
        const size_t ub = ((size_t)lb * dm.Hkv + hk) * (size_t)dm.cap16 * D;
        const int src = mv_at<C>(X.mv16, mv16, 2 * k);
        wk[e] = ((const uint16_t*)c.k16)[ub + k16_off(src, ch, D)];
        wv[e] = ((const uint16_t*)c.v16)[ub + v16_off(src, ch, D)];
      }
    }
    if (tid < nm8) {
      const int src = mv_at<C>(X.mv8, mv8, 2 * tid);
      mp8 = pos8[src];
      me8 = ema8[src];
    }
    if (tid < nm16) {
      const int src = mv_at<C>(X.mv16, mv16, 2 * tid);
      mp16 = pos16[src];
      me16 = ema16[src];
    }
  } else {
    for (int k = tid; k < nm8; k += C::NT) {
      const int src = mv_at<C>(X.mv8, mv8, 2 * k), dst = mv_at<C>(X.mv8, mv8, 2 * k + 1);
      pos8[dst] = pos8[src];
      ema8[dst] = ema8[src];
    }
    // Bulk moves: keys as 16-byte chunks (16 channels are contiguous in a key
    // tile), the move index fastest; values byte by byte with the channel fastest:
    // one token's bytes lie 16 bytes apart in its tile, so a wavefront's 64 channels
    // of one token fall in eight 128-byte lines (with the move index fastest each
    // lane touched a line of its own, one request per byte).
    const int kg = D / 16;
    bulk_copy<C::NT, 2, cu4>(
        nm8 * dm.Hkv * kg,
        [&](int i) {
          const int k = i % nm8, r = i / nm8;
          const size_t ub = ((size_t)lb * dm.Hkv + r / kg) * (size_t)dm.cap8 * D;
          return (const cu4*)(c.k8 + ub + k8_off(mv_at<C>(X.mv8, mv8, 2 * k), 16 * (r % kg), D));
        },
        [&](int i) {
          const int k = i % nm8, r = i / nm8;
          const size_t ub = ((size_t)lb * dm.Hkv + r / kg) * (size_t)dm.cap8 * D;
          return (cu4*)(c.k8 + ub + k8_off(mv_at<C>(X.mv8, mv8, 2 * k + 1), 16 * (r % kg), D));
        });
    // Values: by destination run once the moves average four or more per tile
    // (whole runs then cost less than single-byte stores), else byte by byte.
    if (ntb > 0 && 16 * nm8 >= n8end)
      v8_moves_by_run<C>(c, dm, lb, n8, n8end, demote ? 1 : 0, flag8, X.mv8, mv8, mv8);
    else
      bulk_copy<C::NT, 8, int8_t>(
          nm8 * per,
          [&](int i) {
            const int k = i / per, r = i % per;
            const size_t ub = ((size_t)lb * dm.Hkv + r / D) * (size_t)dm.cap8 * D;
            return (const int8_t*)(c.v8 + ub + v8_off(mv_at<C>(X.mv8, mv8, 2 * k), r % D, D));
          },
          [&](int i) {
            const int k = i / per, r = i % per;
            const size_t ub = ((size_t)lb * dm.Hkv + r / D) * (size_t)dm.cap8 * D;
            return c.v8 + ub + v8_off(mv_at<C>(X.mv8, mv8, 2 * k + 1), r % D, D);
          });
  }
  int8_t code[kDemPer];
  float amax_new[kDemPer], s_old[kDemPer];
  bool grew[kDemPer], listed[kDemPer];
  int dpos = 0;
  float dema = 0.f;
  if (dest >= 0) {
    if (tid == 0) {  // read before the window metadata moves of phase 4
      dpos = pos16[jd];
      dema = ema16[jd];
    }
    // every load first (each thread's triples are clamped into range, so no
    // branch separates them), then the arithmetic: one memory round trip
    uint32_t xr[kDemPer];
    float oldr[kDemPer];
#pragma unroll
    for (int e = 0; e < kDemPer; ++e) {
      if (e * C::NT >= 2 * per) break;  // uniform
      const int pi = min(tid + e * C::NT, 2 * per - 1);
      const int kind = pi / per, hc = pi % per, hk = hc / D, ch = hc % D;
      const size_t u = (size_t)lb * dm.Hkv + hk;
      xr[e] = kind == 0 ? ((const uint16_t*)c.k16)[u * (size_t)dm.cap16 * D + k16_off(jd, ch, D)]
                        : ((const uint16_t*)c.v16)[u * (size_t)dm.cap16 * D + v16_off(jd, ch, D)];
      oldr[e] = (kind == 0 ? c.k_amax : c.v_amax)[u * D + ch];
    }
#pragma unroll
    for (int e = 0; e < kDemPer; ++e) {
      const int pi = tid + e * C::NT;
      grew[e] = false;
      listed[e] = false;
      if (pi < 2 * per) {
        const float x = h16_to_f32((uint16_t)xr[e], dm.bf16);
        const float old = oldr[e];
        const float a = fabsf(x);
        const float am = a > old ? a : old;
        amax_new[e] = am;
        code[e] = quant8(x, am / cmax, fp8);
        s_old[e] = old / cmax;
        if (a > old) {
          grew[e] = true;
          const int slot = atomicAdd(&M.ngrown, 1);
          if (slot < C::MG) {
            listed[e] = true;
            X.grown[slot] = pi;
            X.gold[slot] = s_old[e];
            X.gnew[slot] = am / cmax;
          }
        }
      }
    }
  }
  if (fast) {
    // INT8 stores go to holes below n8', which no load of this phase reads
#pragma unroll
    for (int e = 0; e < kMv; ++e) {
      const int i = tid + e * C::NT;
      if (i < nm8 * per) {
        const int k = i / per, r = i % per, hk = r / D, ch = r % D;
        const size_t ub = ((size_t)lb * dm.Hkv + hk) * (size_t)dm.cap8 * D;
        const int dst = mv_at<C>(X.mv8, mv8, 2 * k + 1);
        c.k8[ub + k8_off(dst, ch, D)] = (int8_t)mk[e];
        c.v8[ub + v8_off(dst, ch, D)] = (int8_t)mvv[e];
      }
    }
    if (tid < nm8) {
      const int dst = mv_at<C>(X.mv8, mv8, 2 * tid + 1);
      pos8[dst] = mp8;
      ema8[dst] = me8;
    }
  }
  __syncthreads();  // INT8 moves done, the demotee's window slot read
  // ---- 4. demotee codes and metadata; window moves; requantisation of grown channels
  if (dest >= 0) {
    if (tid == 0) {
      pos8[dest] = dpos;
      ema8[dest] = dema;
    }
#pragma unroll
    for (int e = 0; e < kDemPer; ++e) {
      const int pi = tid + e * C::NT;
      if (pi < 2 * per) {
        const int kind = pi / per, hc = pi % per, hk = hc / D, ch = hc % D;
        const size_t u = (size_t)lb * dm.Hkv + hk;
        int8_t* base = (kind == 0 ? c.k8 : c.v8) + u * (size_t)dm.cap8 * D;
        base[kind == 0 ? k8_off(dest, ch, D) : v8_off(dest, ch, D)] = code[e];
        if (grew[e]) (kind == 0 ? c.k_amax : c.v_amax)[u * D + ch] = amax_new[e];
      }
    }
  }
  if (fast) {
#pragma unroll
    for (int e = 0; e < kMv; ++e) {
      const int i = tid + e * C::NT;
      if (i < nm16 * per) {
        const int k = i / per, r = i % per, hk = r / D, ch = r % D;
        const size_t ub = ((size_t)lb * dm.Hkv + hk) * (size_t)dm.cap16 * D;
        const int dst = mv_at<C>(X.mv16, mv16, 2 * k + 1);
        ((uint16_t*)c.k16)[ub + k16_off(dst, ch, D)] = (uint16_t)wk[e];
        ((uint16_t*)c.v16)[ub + v16_off(dst, ch, D)] = (uint16_t)wv[e];
      }
    }
    if (tid < nm16) {
      const int dst = mv_at<C>(X.mv16, mv16, 2 * tid + 1);
      pos16[dst] = mp16;
      ema16[dst] = me16;
    }
  } else {
    for (int k = tid; k < nm16; k += C::NT) {
      const int src = mv_at<C>(X.mv16, mv16, 2 * k), dst = mv_at<C>(X.mv16, mv16, 2 * k + 1);
      pos16[dst] = pos16[src];
      ema16[dst] = ema16[src];
    }
    // bulk window moves: keys as 16-byte chunks (8 channels), the move index
    // fastest; values element by element, the channel fastest (as above)
    const int wg = D / 8;
    uint16_t* k16a = (uint16_t*)c.k16;
    uint16_t* v16a = (uint16_t*)c.v16;
    bulk_copy<C::NT, 2, cu4>(
        nm16 * dm.Hkv * wg,
        [&](int i) {
          const int k = i % nm16, r = i / nm16;
          const size_t ub = ((size_t)lb * dm.Hkv + r / wg) * (size_t)dm.cap16 * D;
          return (const cu4*)(k16a + ub + k16_off(mv_at<C>(X.mv16, mv16, 2 * k), 8 * (r % wg), D));
        },
        [&](int i) {
          const int k = i % nm16, r = i / nm16;
          const size_t ub = ((size_t)lb * dm.Hkv + r / wg) * (size_t)dm.cap16 * D;
          return (cu4*)(k16a + ub + k16_off(mv_at<C>(X.mv16, mv16, 2 * k + 1), 8 * (r % wg), D));
        });
    bulk_copy<C::NT, 8, uint16_t>(
        nm16 * per,
        [&](int i) {
          const int k = i / per, r = i % per;
          const size_t ub = ((size_t)lb * dm.Hkv + r / D) * (size_t)dm.cap16 * D;
          return (const uint16_t*)(v16a + ub + v16_off(mv_at<C>(X.mv16, mv16, 2 * k), r % D, D));
        },
        [&](int i) {
          const int k = i / per, r = i % per;
          const size_t ub = ((size_t)lb * dm.Hkv + r / D) * (size_t)dm.cap16 * D;
          return v16a + ub + v16_off(mv_at<C>(X.mv16, mv16, 2 * k + 1), r % D, D);
        });
  }
  if (dest >= 0) {
    // codes of every other INT8 slot of each grown channel: c = clamp(rne((c * s_old) / s_new))
    const int ng = M.ngrown;
    const int ngl = ng < C::MG ? ng : C::MG;
    for (int i = tid; i < ngl * n8end; i += C::NT) {
      const int e = i % ngl, tok = i / ngl;
      if (tok == dest) continue;
      const int pi = X.grown[e], kind = pi / per, hc = pi % per, hk = hc / D, ch = hc % D;
      const size_t u = (size_t)lb * dm.Hkv + hk;
      int8_t* p = (kind == 0 ? c.k8 + u * (size_t)dm.cap8 * D + k8_off(tok, ch, D)
                             : c.v8 + u * (size_t)dm.cap8 * D + v8_off(tok, ch, D));
      *p = quant8(code_value(*p, fp8) * X.gold[e], X.gnew[e], fp8);
    }
    // a list overflow (very many channels grew at once): the owner requantises
#pragma unroll
    for (int e = 0; e < kDemPer; ++e) {
      if (!grew[e] || listed[e]) continue;
      const int pi = tid + e * C::NT;
      const int kind = pi / per, hc = pi % per, hk = hc / D, ch = hc % D;
      int8_t* base = (kind == 0 ? c.k8 : c.v8) + ((size_t)lb * dm.Hkv + hk) * (size_t)dm.cap8 * D;
      const float s_new = amax_new[e] / cmax;
      for (int tok = 0; tok < n8end; ++tok) {
        if (tok == dest) continue;
        int8_t* q = base + (kind == 0 ? k8_off(tok, ch, D) : v8_off(tok, ch, D));
        *q = quant8(code_value(*q, fp8) * s_old[e], s_new, fp8);
      }
    }
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
    c.n8[lb] = n8end;
    c.n16[lb] = n16n;
  }
}

// Sums per-thread counts of kept INT8 and window tokens over the workgroup.
template <class C>
__device__ inline void count_kept(int c8, int c16, CompMiscT<C>& M, int& n8n, int& n16n) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int off = 32; off > 0; off >>= 1) {
    c8 += __shfl_xor(c8, off);
    c16 += __shfl_xor(c16, off);
  }
  if (lane == 0) {
    M.c8[wave] = c8;
    M.c16[wave] = c16;
  }
  __syncthreads();
  n8n = 0;
  n16n = 0;
  for (int w = 0; w < C::W; ++w) {
    n8n += M.c8[w];
    n16n += M.c16[w];
  }
}

template <class C>
__global__ __launch_bounds__(C::NT) void compact_kernel(conf_cache c, Dims dm, int layer0,
                                                               const uint8_t* __restrict__ keep_all,
                                                               int32_t* __restrict__ plan_all,
                                                               int32_t* __restrict__ mv8_all,
                                                               int32_t* __restrict__ mv16_all,
                                                               uint8_t* __restrict__ wkeep_all) {
  __shared__ CompFlagsT<C> F;
  __shared__ CompScratchT<C> X;
  __shared__ CompMiscT<C> M;
  const int lb = layer0 * dm.B + blockIdx.x;
  const int tid = threadIdx.x;
  const int n8 = c.n8[lb], n16 = c.n16[lb], t = c.t[lb];
  const uint8_t* keep8 = keep_all + (size_t)lb * dm.capt;
  const uint8_t* keep16 = keep8 + dm.cap8;
  uint8_t* wkeep = wkeep_all + (size_t)lb * dm.cap16;
  const int32_t* pos16 = c.pos16 + (size_t)lb * dm.cap16;
  if (tid == 0) {
    M.jd = -1;
    M.ngrown = 0;
  }
  __syncthreads();
  // ---- 1. keep flags (one read), counts, the demotee
  // the token that leaves the window (the baselines and retention eviction demote
  // nothing: their tokens stay 16-bit)
  const int target = dm.policy == CONF_POLICY_FULL || dm.policy == CONF_POLICY_TRIM ||
                             dm.policy == CONF_POLICY_WINDOW
                         ? -1
                         : t - dm.W;
  int c8 = 0, c16 = 0;
  for (int i = tid; i < n8; i += C::NT) {
    const uint8_t k = keep8[i] ? 1 : 0;
    if (i < C::F8) F.k8[i] = k;
    c8 += k;
  }
  for (int w = tid; w < n16; w += C::NT) {
    uint8_t k = keep16[w] ? 1 : 0;
    if (k && target >= 0 && pos16[w] == target) {
      M.jd = w;  // at most one slot holds this position
      k = 0;
    }
    if (w < C::F16) F.k16[w] = k; else wkeep[w] = k;
    c16 += k;
  }
  int n8n, n16n;
  count_kept(c8, c16, M, n8n, n16n);
  compact_core(c, dm, lb, n8, n16, n8n, n16n, M.jd, keep8, wkeep, F, X, M, plan_all, mv8_all,
               mv16_all);
}

// The EMA update of (layer, sequence) lb, as ema_tokens computes it (same
// arithmetic, same order over the KV heads), by a kCompThreads workgroup whose
// thread tid takes tokens tid, tid + kCompThreads, ...  Each round issues the loads
// of five tokens (EMA, position, then the mass rows two heads at a time) before
// the arithmetic.  With the
// selection's keys in LDS, each token's new (bits(e) << 32 | pos) is left in
// X.key[j] for select_core, which then reads no memory in its first pass.
__device__ inline void ema_pairs(const conf_cache& c, const Dims& dm, int lb,
                                 const float* __restrict__ massp_all, int n8, int nw, int t,
                                 float log_beta, SelScratch& X) {
#pragma clang fp contract(off)
  const int appended = nw < dm.cap16;
  if (dm.policy != CONF_POLICY_CONFKV) {  // no EMA: the appended token's slot only
    if (threadIdx.x == 0 && appended) {   // (retention eviction keeps its ln(beta) there)
      c.ema16[(size_t)lb * dm.cap16 + nw] = dm.policy == CONF_POLICY_TRIM ? log_beta : 0.f;
      c.pos16[(size_t)lb * dm.cap16 + nw] = t + 1;
    }
    return;
  }
  const int end = n8 + nw + appended;
  const bool cached = end <= kSelLdsKeys;
  const float* rows = massp_all + (size_t)lb * dm.Hkv * dm.capt;
  float* ema8 = c.ema8 + (size_t)lb * dm.cap8;
  float* ema16 = c.ema16 + (size_t)lb * dm.cap16;
  const int32_t* pos8 = c.pos8 + (size_t)lb * dm.cap8;
  int32_t* pos16 = c.pos16 + (size_t)lb * dm.cap16;
  const float hq = (float)dm.Hq;
  // Four tokens per thread and round; the mass rows of up to eight KV heads are
  // loaded together with the EMA and positions, and only then summed (in head
  // order): one memory round trip per round and eight heads, within 80 VGPRs
  // (6 waves/SIMD).  (A loop over the heads that summed as it loaded waited once
  // per unrolled pair of heads.)
  constexpr int kT = 4, kHC = 8;
  for (int jb = threadIdx.x; jb < end; jb += kT * kCompThreads) {
    int idx[kT], po[kT];
    float a[kT], eo[kT];
#pragma unroll
    for (int k = 0; k < kT; ++k) {
      const int j = jb + k * kCompThreads;
      idx[k] = j >= end ? 0 : j < n8 ? j : dm.cap8 + (j - n8);
      const int w = j >= end ? 0 : j - n8;
      eo[k] = j < n8 ? ema8[idx[k]] : ema16[w];
      po[k] = j < n8 ? pos8[idx[k]] : pos16[w];
      a[k] = 0.f;
    }
    for (int h0 = 0; h0 < dm.Hkv; h0 += kHC) {
      float r[kHC][kT];
#pragma unroll
      for (int i = 0; i < kHC; ++i) {
        // heads past the last read the last one's row again and are not added
        const int hk = min(h0 + i, dm.Hkv - 1);
#pragma unroll
        for (int k = 0; k < kT; ++k) r[i][k] = rows[(size_t)hk * dm.capt + idx[k]];
      }
#pragma unroll
      for (int i = 0; i < kHC; ++i)
        if (h0 + i < dm.Hkv) {
#pragma unroll
          for (int k = 0; k < kT; ++k) a[k] += r[i][k];
        }
    }
#pragma unroll
    for (int k = 0; k < kT; ++k) {
      const int j = jb + k * kCompThreads;
      if (j >= end) continue;
      const float m = a[k] / hq;
      float e;
      int p = po[k];
      if (j < n8) {
        e = dm.decay * eo[k] + dm.one_minus_decay * m;
        ema8[j] = e;
      } else if (j - n8 == nw) {
        e = dm.one_minus_decay * m;  // decay * 0 + (1 - decay) * mass
        p = t + 1;
        ema16[nw] = e;
        pos16[nw] = p;
      } else {
        e = dm.decay * eo[k] + dm.one_minus_decay * m;
        ema16[j - n8] = e;
      }
      if (cached) X.key[j] = ((uint64_t)__float_as_uint(e) << 32) | (uint32_t)p;
    }
  }
}

// (d)+(e) in one launch: the selection's keep flags go straight into the LDS
// flag cache (INT8 flags beyond it into keep_all, window flags beyond it into
// the window flag spill), the demotee is recognised from its ranking key (whose
// low bits hold the position), and the compaction follows in the same
// workgroup.  The selection's key cache and the compaction's move lists share
// LDS.  Results are those of select_kernel followed by compact_kernel.
// With EMA, (c) comes first, in place of the EMA kernel after an attention launch
// that left it pending: the sizes before the step's append come from the
// attention's snapshot, every token's EMA is updated (and the appended token's
// position written), and n16 and t advance.
template <bool EMA>
// (six wavefronts per SIMD: three workgroups per CU, which the LDS allows too)
__global__ __launch_bounds__(kCompThreads, 6) void evict_kernel(conf_cache c, Dims dm, int layer0,
                                                             const int32_t* __restrict__ budget,
                                                             uint8_t* __restrict__ keep_all,
                                                             int32_t* __restrict__ plan_all,
                                                             int32_t* __restrict__ mv8_all,
                                                             int32_t* __restrict__ mv16_all,
                                                             uint8_t* __restrict__ wkeep_all,
                                                             const float* __restrict__ massp_all,
                                                             const int32_t* __restrict__ snap,
                                                             const float* __restrict__ log_beta) {
  // 52 KB of LDS in all, so that three workgroups fit on a CU
  __shared__ CompFlags F;
  __shared__ union {
    SelScratch sel;
    CompScratch comp;
  } U;
  __shared__ SelMisc SM;
  __shared__ CompMisc M;
  const int lb = layer0 * dm.B + blockIdx.x;
  const int l = lb / dm.B, b = lb % dm.B;
  const int tid = threadIdx.x;
  int n8, n16, t;
  if constexpr (EMA) {
    n8 = snap[3 * lb];
    const int nw = snap[3 * lb + 1], t0 = snap[3 * lb + 2];
    n16 = nw + (nw < dm.cap16);
    t = t0 + 1;
    ema_pairs(c, dm, lb, massp_all, n8, nw, t0, log_beta ? log_beta[blockIdx.x] : 0.f, U.sel);
    if (tid == 0) c.t[lb] = t;  // n16 is written by the compaction
    __syncthreads();  // the EMA and the appended position are in memory for the selection
  } else {
    n8 = c.n8[lb];
    n16 = c.n16[lb];
    t = c.t[lb];
  }
  const int N = budget[(size_t)b * dm.L + l];
  uint8_t* keep8 = keep_all + (size_t)lb * dm.capt;
  uint8_t* wkeep = wkeep_all + (size_t)lb * dm.cap16;
  const int32_t* pos16 = c.pos16 + (size_t)lb * dm.cap16;
  if (tid == 0) {
    M.jd = -1;
    M.ngrown = 0;
  }
  __syncthreads();
  // the token that leaves the window (the baselines and retention eviction demote
  // nothing: their tokens stay 16-bit)
  const int target = dm.policy == CONF_POLICY_FULL || dm.policy == CONF_POLICY_TRIM ||
                             dm.policy == CONF_POLICY_WINDOW
                         ? -1
                         : t - dm.W;
  int c8 = 0, c16 = 0;
  // (both counts advance on every token: with the increment inside each branch the
  // compiler kept the two counts in private memory and added through a selected
  // address, one scratch round trip per token)
  select_core<kCompThreads, EMA>(c, dm, lb, n8, n16, t, N, U.sel, SM, [&](int j, int k, uint64_t key) {
    const bool is8 = j < n8;
    if (is8) {
      if (j < kLdsFlags8) F.k8[j] = (uint8_t)k; else keep8[j] = (uint8_t)k;
    } else {
      const int w = j - n8;
      if (k && target >= 0) {
        // a protected token (key 0) is newer than t - W
        const int p = key == kAllKept ? pos16[w] : key ? (int)(uint32_t)(key - 1ull) : -1;
        if (p == target) {
          M.jd = w;  // at most one slot holds this position
          k = 0;
        }
      }
      if (w < kLdsFlags16) F.k16[w] = (uint8_t)k; else wkeep[w] = (uint8_t)k;
    }
    c8 += is8 ? k : 0;
    c16 += is8 ? 0 : k;
  });
  int n8n, n16n;
  count_kept(c8, c16, M, n8n, n16n);  // its barrier also ends the key cache's use
  compact_core(c, dm, lb, n8, n16, n8n, n16n, M.jd, keep8, wkeep, F, U.comp, M, plan_all,
               mv8_all, mv16_all);
}

// ARKV's pending score update (the ARKV page, Methodology: decoding-phase token
// ranking) for (layer, sequence) lb: over the KV heads k, with m_k = row_k / G
// the token's attention averaged over head k's query heads,
//   h = mean_k m_k + (mean_k m_k^2 - (mean_k m_k)^2, at least 0),
//   e <- decay*e + (1-decay)*h   (the appended token from e = 0 at position t+1),
// fp32, one rounding per operation.  Each token's (bits(e) << 32 | pos) is left in
// X.key[j] for select_core when the keys fit in LDS.
__device__ inline void arkv_pairs(const conf_cache& c, const Dims& dm, int lb,
                                  const float* __restrict__ massp_all, int n8, int nw, int t,
                                  SelScratch& X) {
#pragma clang fp contract(off)
  const int appended = nw < dm.cap16;
  const int end = n8 + nw + appended;
  const bool cached = end <= kSelLdsKeys;
  const float* rows = massp_all + (size_t)lb * dm.Hkv * dm.capt;
  float* ema8 = c.ema8 + (size_t)lb * dm.cap8;
  float* ema16 = c.ema16 + (size_t)lb * dm.cap16;
  const int32_t* pos8 = c.pos8 + (size_t)lb * dm.cap8;
  int32_t* pos16 = c.pos16 + (size_t)lb * dm.cap16;
  constexpr int kT = 4;
  for (int jb = threadIdx.x; jb < end; jb += kT * kCompThreads) {
    int idx[kT], po[kT];
    float a[kT], a2[kT], eo[kT];
#pragma unroll
    for (int k = 0; k < kT; ++k) {
      const int j = jb + k * kCompThreads;
      idx[k] = j >= end ? 0 : j < n8 ? j : dm.cap8 + (j - n8);
      const int w = j >= end ? 0 : j - n8;
      eo[k] = j < n8 ? ema8[idx[k]] : ema16[w];
      po[k] = j < n8 ? pos8[idx[k]] : pos16[w];
      a[k] = 0.f;
      a2[k] = 0.f;
    }
    // up to eight KV heads' rows loaded together, then summed in head order (as in
    // ema_pairs)
    constexpr int kHC = 8;
    for (int h0 = 0; h0 < dm.Hkv; h0 += kHC) {
      float r[kHC][kT];
#pragma unroll
      for (int i = 0; i < kHC; ++i) {
        const int hk = min(h0 + i, dm.Hkv - 1);
#pragma unroll
        for (int k = 0; k < kT; ++k) r[i][k] = rows[(size_t)hk * dm.capt + idx[k]];
      }
#pragma unroll
      for (int i = 0; i < kHC; ++i)
        if (h0 + i < dm.Hkv) {
#pragma unroll
          for (int k = 0; k < kT; ++k) {
            a[k] += r[i][k];
            a2[k] += r[i][k] * r[i][k];
          }
        }
    }
#pragma unroll
    for (int k = 0; k < kT; ++k) {
      const int j = jb + k * kCompThreads;
      if (j >= end) continue;
      const float h = arkv_h(a[k], a2[k], dm);
      float e;
      int p = po[k];
      if (j < n8) {
        e = dm.decay * eo[k] + dm.one_minus_decay * h;
        ema8[j] = e;
      } else if (j - n8 == nw) {
        e = dm.one_minus_decay * h;  // decay * 0 + (1 - decay) * h
        p = t + 1;
        ema16[nw] = e;
        pos16[nw] = p;
      } else {
        e = dm.decay * eo[k] + dm.one_minus_decay * h;
        ema16[j - n8] = e;
      }
      if (cached) X.key[j] = ((uint64_t)__float_as_uint(e) << 32) | (uint32_t)p;
    }
  }
}

// One ARKV step's cache update, one workgroup per (layer, sequence) [the ARKV
// page, Methodology: three-state assignment]:
//  1. with EMA (after conf_attend), the score update above (sizes from the
//     attention's snapshot; t advances); without, the EMA kernel has applied it;
//  2. keep the newest P positions and the budget's best others by (EMA desc,
//     position desc) (select_core);
//  3. with more than N_O kept tokens Original (16-bit), the lowest-ranked
//     unprotected one becomes Quantized: compact_core's demotion, with e4m3
//     codes, together with the eviction.  Any further demotion the step needs
//     is arkv_rounds_kernel's.
template <bool EMA>
__global__ __launch_bounds__(kCompThreads) void arkv_kernel(
    conf_cache c, Dims dm, int layer0, const int32_t* __restrict__ budget,
    const int32_t* __restrict__ n_orig, uint8_t* __restrict__ keep_all,
    int32_t* __restrict__ plan_all, int32_t* __restrict__ mv8_all, int32_t* __restrict__ mv16_all,
    uint8_t* __restrict__ wkeep_all, const float* __restrict__ massp_all,
    const int32_t* __restrict__ snap) {
  __shared__ CompFlags F;
  __shared__ union {
    SelScratch sel;
    CompScratch comp;
  } U;
  __shared__ SelMisc SM;
  __shared__ CompMisc M;
  const int lb = layer0 * dm.B + blockIdx.x;
  const int l = lb / dm.B, b = lb % dm.B;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int n8, n16, t;
  if constexpr (EMA) {
    n8 = snap[3 * lb];
    const int nw = snap[3 * lb + 1], t0 = snap[3 * lb + 2];
    n16 = nw + (nw < dm.cap16);
    t = t0 + 1;
    arkv_pairs(c, dm, lb, massp_all, n8, nw, t0, U.sel);
    if (tid == 0) c.t[lb] = t;  // n8 and n16 are written by the compaction
  } else {
    n8 = c.n8[lb];
    n16 = c.n16[lb];
    t = c.t[lb];
  }
  if (tid == 0) {
    M.jd = -1;
    M.ngrown = 0;
  }
  __syncthreads();  // scores and the appended position are in memory for the selection
  const int N = budget[(size_t)b * dm.L + l];
  const int NO = n_orig[(size_t)b * dm.L + l];
  const int prot_lo = t - dm.P;
  uint8_t* keep8 = keep_all + (size_t)lb * dm.capt;
  uint8_t* wkeep = wkeep_all + (size_t)lb * dm.cap16;
  const int32_t* pos16 = c.pos16 + (size_t)lb * dm.cap16;
  const float* ema16 = c.ema16 + (size_t)lb * dm.cap16;
  // ranking key + 1 of window slot w, or 0 when it is protected
  auto win_key = [&](int w) -> uint64_t {
    const int p = pos16[w];
    if (p > prot_lo) return 0ull;
    return (((uint64_t)__float_as_uint(ema16[w]) << 32) | (uint32_t)p) + 1ull;
  };
  // the kept unprotected Original with the smallest key: (key, slot) per thread
  uint64_t mn = ~0ull;
  int ms = -1;
  int c8 = 0, c16 = 0;
  select_core<kCompThreads, EMA>(c, dm, lb, n8, n16, t, N, U.sel, SM, [&](int j, int k, uint64_t key) {
    const bool is8 = j < n8;  // both counts advance on every token (no private-memory counts)
    if (is8) {
      if (j < kLdsFlags8) F.k8[j] = (uint8_t)k; else keep8[j] = (uint8_t)k;
    } else {
      const int w = j - n8;
      if (k) {
        const uint64_t kk = key == kAllKept ? win_key(w) : key;
        if (kk != 0ull && kk < mn) {
          mn = kk;
          ms = w;
        }
      }
      if (w < kLdsFlags16) F.k16[w] = (uint8_t)k; else wkeep[w] = (uint8_t)k;
    }
    c8 += is8 ? k : 0;
    c16 += is8 ? 0 : k;
  });
  int n8n, n16n;
  count_kept(c8, c16, M, n8n, n16n);  // its barrier also ends the key cache's use
  // the demotee, if more than N_O Original tokens remain
  int jd = -1;
  if (n16n > NO) {
    const uint64_t wm = wave_min_u64(mn);
    if (lane == 0) SM.wmin[wave] = wm;
    __syncthreads();
    uint64_t gm = SM.wmin[0];
    for (int w = 1; w < kCompWaves; ++w) gm = SM.wmin[w] < gm ? SM.wmin[w] : gm;
    if (gm != ~0ull && mn == gm) {  // keys are unique: one thread
      M.jd = ms;
      if (ms < kLdsFlags16) F.k16[ms] = 0; else wkeep[ms] = 0;
    }
    __syncthreads();
    jd = M.jd;
    if (jd >= 0) --n16n;
  }
  compact_core(c, dm, lb, n8, n16, n8n, n16n, jd, keep8, wkeep, F, U.comp, M, plan_all,
               mv8_all, mv16_all);
}

// Further ARKV demotions of a step whose N_O fell by more than one token (or the
// first step after a prefill whose window holds more than N_O): one round per
// token, each the lowest-ranked unprotected Original of the cache as it stands,
// moved by compact_core with every other token kept.  A workgroup whose cache is
// within N_O returns at once, so in the steady state this launch does nothing.
// Registers are bounded to 128 (the loop spills): a workgroup that needs the
// whole register file waits for a compute unit with no attention workgroup on
// it, even to return at once.
__global__ __launch_bounds__(kCompThreads, 4) void arkv_rounds_kernel(
    conf_cache c, Dims dm, int layer0, const int32_t* __restrict__ n_orig,
    uint8_t* __restrict__ keep_all, int32_t* __restrict__ plan_all, int32_t* __restrict__ mv8_all,
    int32_t* __restrict__ mv16_all, uint8_t* __restrict__ wkeep_all) {
  __shared__ CompFlags F;
  __shared__ CompScratch X;
  __shared__ CompMisc M;
  __shared__ unsigned long long wmin[kCompWaves];
  const int lb = layer0 * dm.B + blockIdx.x;
  const int l = lb / dm.B, b = lb % dm.B;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NO = n_orig[(size_t)b * dm.L + l];
  int n8 = c.n8[lb], n16 = c.n16[lb];
  const int t = c.t[lb];
  if (n16 <= NO) return;  // uniform over the workgroup
  const int prot_lo = t - dm.P;
  uint8_t* keep8 = keep_all + (size_t)lb * dm.capt;
  uint8_t* wkeep = wkeep_all + (size_t)lb * dm.cap16;
  const int32_t* pos16 = c.pos16 + (size_t)lb * dm.cap16;
  const float* ema16 = c.ema16 + (size_t)lb * dm.cap16;
  while (n16 > NO) {
    uint64_t mn = ~0ull;
    int ms = -1;
    for (int i = tid; i < n8; i += kCompThreads)
      if (i < kLdsFlags8) F.k8[i] = 1; else keep8[i] = 1;
    for (int w = tid; w < n16; w += kCompThreads) {
      if (w < kLdsFlags16) F.k16[w] = 1; else wkeep[w] = 1;
      const int p = pos16[w];
      if (p > prot_lo) continue;
      const uint64_t kk = ((uint64_t)__float_as_uint(ema16[w]) << 32) | (uint32_t)p;
      if (kk < mn) {
        mn = kk;
        ms = w;
      }
    }
    if (tid == 0) {
      M.jd = -1;
      M.ngrown = 0;
    }
    const uint64_t wm = wave_min_u64(mn);
    if (lane == 0) wmin[wave] = wm;
    __syncthreads();
    uint64_t gm = wmin[0];
    for (int w = 1; w < kCompWaves; ++w) gm = wmin[w] < gm ? wmin[w] : gm;
    if (gm != ~0ull && mn == gm) {
      M.jd = ms;
      if (ms < kLdsFlags16) F.k16[ms] = 0; else wkeep[ms] = 0;
    }
    __syncthreads();
    const int jd = M.jd;
    if (jd < 0) break;  // every Original token is protected
    compact_core(c, dm, lb, n8, n16, n8, n16 - 1, jd, keep8, wkeep, F, X, M, plan_all,
                 mv8_all, mv16_all);
    // the demotee took the INT8 region's first free slot (or was dropped when it was full)
    n8 += n8 < dm.cap8 ? 1 : 0;
    n16 -= 1;
    __syncthreads();  // this round's moves are in memory
  }
}

void launch_arkv(const Dims& dm, const conf_cache& c, int layer0, int nl, const int32_t* budget,
                 const int32_t* n_orig, uint8_t* keep, int32_t* plan, int32_t* mv8, int32_t* mv16,
                 uint8_t* wkeep, const float* massp, const int32_t* snap, bool with_ema,
                 hipStream_t st) {
  if (with_ema)
    hipLaunchKernelGGL(arkv_kernel<true>, dim3(nl * dm.B), dim3(kCompThreads), 0, st, c, dm,
                       layer0, budget, n_orig, keep, plan, mv8, mv16, wkeep, massp, snap);
  else
    hipLaunchKernelGGL(arkv_kernel<false>, dim3(nl * dm.B), dim3(kCompThreads), 0, st, c, dm,
                       layer0, budget, n_orig, keep, plan, mv8, mv16, wkeep, massp, snap);
  hipLaunchKernelGGL(arkv_rounds_kernel, dim3(nl * dm.B), dim3(kCompThreads), 0, st, c, dm,
                     layer0, n_orig, keep, plan, mv8, mv16, wkeep);
}

void launch_compact(const Dims& dm, const conf_cache& c, int layer0, int nl, const uint8_t* keep,
                    int32_t* plan, int32_t* mv8, int32_t* mv16, uint8_t* wkeep, hipStream_t st) {
  // a head-wise cache compacts one KV head per workgroup: small workgroups with
  // little LDS, many of them resident per compute unit
  if (dm.headwise && 2 * dm.Hkv * dm.D <= 8 * CompSmall::NT)
    hipLaunchKernelGGL(compact_kernel<CompSmall>, dim3(nl * dm.B), dim3(CompSmall::NT), 0, st, c,
                       dm, layer0, keep, plan, mv8, mv16, wkeep);
  else
    hipLaunchKernelGGL(compact_kernel<CompBig>, dim3(nl * dm.B), dim3(CompBig::NT), 0, st, c, dm,
                       layer0, keep, plan, mv8, mv16, wkeep);
}

void launch_evict(const Dims& dm, const conf_cache& c, int layer0, int nl, const int32_t* budget,
                  uint8_t* keep, int32_t* plan, int32_t* mv8, int32_t* mv16, uint8_t* wkeep,
                  const float* massp, const int32_t* snap, const float* log_beta, bool with_ema,
                  hipStream_t st) {
  if (with_ema)
    hipLaunchKernelGGL(evict_kernel<true>, dim3(nl * dm.B), dim3(kCompThreads), 0, st, c, dm,
                       layer0, budget, keep, plan, mv8, mv16, wkeep, massp, snap, log_beta);
  else
    hipLaunchKernelGGL(evict_kernel<false>, dim3(nl * dm.B), dim3(kCompThreads), 0, st, c, dm,
                       layer0, budget, keep, plan, mv8, mv16, wkeep, massp, snap, log_beta);
}

// ln(beta) of an ingested prefill (retention eviction): window slot w holds
// position w, since the prefill fits the window.  log_beta [nl*B][L0].
__global__ void set_retention_kernel(conf_cache c, Dims dm, int layer0, const float* log_beta,
                                     int L0) {
  const int lb = layer0 * dm.B + blockIdx.x;
  for (int w = threadIdx.x; w < L0; w += blockDim.x)
    c.ema16[(size_t)lb * dm.cap16 + w] = log_beta[(size_t)blockIdx.x * L0 + w];
}

void launch_set_retention(const Dims& dm, const conf_cache& c, int layer0, int nl,
                          const float* log_beta, int L0, hipStream_t st) {
  hipLaunchKernelGGL(set_retention_kernel, dim3(nl * dm.B), dim3(256), 0, st, c, dm, layer0,
                     log_beta, L0);
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
