// (b)+(c) Decode attention on the CDNA4 matrix cores, with the per-token
// attention mass and the EMA update, in one launch per step.
//
// CONF-KV explainer, Key contributions (system design): block-wise online-
// softmax attention; Methodology, implementation: dequantisation fused into the
// block-wise attention reads over a dense (compacted) layout; mixed-precision
// storage: INT8 codes with one scale per (KV head, channel).
//
// Work split: one workgroup (4 wavefronts) per unit (layer, sequence, KV head);
// a wavefront takes whole 64-token blocks, round-robin.  For a block it forms
//   S^T[16 tokens x 16 heads] = K[16 x d] . Q^T[d x 16]   (v_mfma_f32_16x16x32)
// four times (64 tokens), so each lane holds one query head (lane % 16) and four
// tokens per 16-token row block; that is exactly the A-operand layout of
//   O[16 heads x 16 channels] += P[16 x 32 tokens] . V[32 tokens x 16 channels]
// so P never leaves registers, and the tiled value layout (see tile_col) hands
// each lane its 16 tokens of one channel in one 16-byte load.  Heads beyond
// g = Hq/Hkv are zero padding of the 16-wide tile.
//
// Precision.  INT8 codes become fp16 exactly.  The key scale folds into the
// query: q' = q * amax_K/127, scaled by a power of two per head so its largest
// entry sits in [2^14, 2^15), then split into fp16 hi + lo parts (two MFMAs,
// ~22 significant bits).  Window keys meet the 16-bit query as stored (exact
// products).  P is rounded to fp16 for INT8 values and fp16 windows; for
// bfloat16 windows it is split into bf16 hi + lo parts.  All sums are fp32.
//
// Scores of the whole unit stay in LDS (fp32) when they fit; then the per-token
// mass is formed after the softmax normaliser is final.  Otherwise (the first
// step after a long prefill) the kernel makes two passes over the keys: the
// first finds each head's log-sum-exp, the second forms probabilities, mass and
// the value sums directly.
#include "common.hpp"

namespace confkv {

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



typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kMfmaThreads = kWaves * 64;
constexpr int kLdsScoreBytes = 76 * 1024;  // dynamic LDS budget of one workgroup

enum { MODE_ONLINE = 0, MODE_LSE = 1, MODE_FINAL = 2 };

__device__ inline f4 mma_f16(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ inline f4 mma_bf16(bf8 a, bf8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16 signed INT8 codes -> two groups of 8 exact fp16 values.  x ^ 0x80 is the
// code + 128; the fp16 bit pattern 0x64XX is 1024 + XX; subtracting 1152 leaves
// the code.
__device__ inline h2 bias_pair(uint32_t w, uint32_t sel) {
  const uint32_t v = __builtin_amdgcn_perm(0x64646464u, w, sel);
  return __builtin_bit_cast(h2, v) - (h2){(_Float16)1152.0f, (_Float16)1152.0f};
}
__device__ inline void codes_to_f16(u4 raw, h8& a0, h8& a1) {
  const uint32_t w0 = raw.x ^ 0x80808080u, w1 = raw.y ^ 0x80808080u;
  const uint32_t w2 = raw.z ^ 0x80808080u, w3 = raw.w ^ 0x80808080u;
  const h2 p0 = bias_pair(w0, 0x04010400u), p1 = bias_pair(w0, 0x04030402u);
  const h2 p2 = bias_pair(w1, 0x04010400u), p3 = bias_pair(w1, 0x04030402u);
  const h2 p4 = bias_pair(w2, 0x04010400u), p5 = bias_pair(w2, 0x04030402u);
  const h2 p6 = bias_pair(w3, 0x04010400u), p7 = bias_pair(w3, 0x04030402u);
  a0 = (h8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
  a1 = (h8){p4.x, p4.y, p5.x, p5.y, p6.x, p6.y, p7.x, p7.y};
}

__device__ inline u4 ld16(const void* p) { return *(const u4*)p; }

template <int D>
struct WaveAcc {
  float m;             // running max of this lane's head
  float l;             // running sum
  f4 o[D / 16];        // O tile: lane = channel 16*cb + lane%16, rows = heads 4*(lane/16)+i
};

template <int D, bool BF16>
struct QOps {
  u4 qw[D / 32];       // 16-bit query as stored, for window keys
  h8 qh[D / 32];       // fp16 hi part of the scaled INT8 query
  h8 ql[D / 32];       // fp16 lo part
};

// S^T of one 64-token block: acc[r][i] = score of token 16r + 4*(lane/16) + i
// for head lane%16 (before scaling).
template <int D, bool BF16>
__device__ inline void block_scores_i8(const int8_t* k8blk, const QOps<D, BF16>& q, f4 acc[4]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, row = lane & 15;
  u4 raw[4][D / 64];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int hh = 0; hh < D / 64; ++hh) raw[r][hh] = ld16(k8blk + (16 * r + row) * D + 64 * hh + 16 * g);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    f4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hh = 0; hh < D / 64; ++hh) {
      h8 k0, k1;
      codes_to_f16(raw[r][hh], k0, k1);
      a = mma_f16(k0, q.qh[2 * hh], a);
      a = mma_f16(k0, q.ql[2 * hh], a);
      a = mma_f16(k1, q.qh[2 * hh + 1], a);
      a = mma_f16(k1, q.ql[2 * hh + 1], a);
    }
    acc[r] = a;
  }
}

template <int D, bool BF16>
__device__ inline void block_scores_16(const uint16_t* k16blk, const QOps<D, BF16>& q, f4 acc[4]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, row = lane & 15;
  u4 raw[4][D / 32];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int s = 0; s < D / 32; ++s) raw[r][s] = ld16(k16blk + (16 * r + row) * D + 32 * s + 8 * g);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    f4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      if constexpr (BF16)
        a = mma_bf16(__builtin_bit_cast(bf8, raw[r][s]), __builtin_bit_cast(bf8, q.qw[s]), a);
      else
        a = mma_f16(__builtin_bit_cast(h8, raw[r][s]), __builtin_bit_cast(h8, q.qw[s]), a);
    }
    acc[r] = a;
  }
}

// O += P . V for one 64-token block.  p[r][i]: probability of token
// 16r + 4g + i for head lane%16 (already 0 for masked tokens and padding heads).
template <int D>
__device__ inline void block_pv_i8(const int8_t* v8blk, const float p[4][4], f4* o) {
  const int lane = threadIdx.x & 63, g = lane >> 4, col = lane & 15;
  h8 pa[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) pa[u][e] = (_Float16)p[2 * u + (e >> 2)][e & 3];
#pragma unroll
  for (int cb = 0; cb < D / 16; ++cb) {
    const u4 raw = ld16(v8blk + (16 * cb + col) * kTile + 16 * g);
    h8 v0, v1;
    codes_to_f16(raw, v0, v1);
    o[cb] = mma_f16(pa[0], v0, o[cb]);
    o[cb] = mma_f16(pa[1], v1, o[cb]);
  }
}

template <int D, bool BF16>
__device__ inline void block_pv_16(const uint16_t* v16blk, const float p[4][4], f4* o) {
  const int lane = threadIdx.x & 63, g = lane >> 4, col = lane & 15;
  if constexpr (BF16) {
    bf8 ph[2], pl[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = p[2 * u + (e >> 2)][e & 3];
        const __bf16 hi = (__bf16)x;
        ph[u][e] = hi;
        pl[u][e] = (__bf16)(x - (float)hi);
      }
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) {
      const uint16_t* rowp = v16blk + (16 * cb + col) * kTile + 16 * g;
      const bf8 v0 = __builtin_bit_cast(bf8, ld16(rowp));
      const bf8 v1 = __builtin_bit_cast(bf8, ld16(rowp + 8));
      o[cb] = mma_bf16(ph[0], v0, o[cb]);
      o[cb] = mma_bf16(pl[0], v0, o[cb]);
      o[cb] = mma_bf16(ph[1], v1, o[cb]);
      o[cb] = mma_bf16(pl[1], v1, o[cb]);
    }
  } else {
    h8 pa[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) pa[u][e] = (_Float16)p[2 * u + (e >> 2)][e & 3];
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) {
      const uint16_t* rowp = v16blk + (16 * cb + col) * kTile + 16 * g;
      o[cb] = mma_f16(pa[0], __builtin_bit_cast(h8, ld16(rowp)), o[cb]);
      o[cb] = mma_f16(pa[1], __builtin_bit_cast(h8, ld16(rowp + 8)), o[cb]);
    }
  }
}

// max / sum over the four lanes that hold the same head (lane, lane^16, lane^32, lane^48)
__device__ inline float head_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ inline float head_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}
// sum over the 16 heads held by one 16-lane group
__device__ inline float group_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  return x + __shfl_xor(x, 8);
}

struct BlockCtx {
  int n_valid;     // valid tokens in this block (1..64)
  int tok0;        // unit-level token index of the block's first slot
  int mass_idx0;   // massp index of the block's first slot
  float scale;     // score scale of this lane's head
  int head_ok;     // lane's head < g
};

// One 64-token block in the given mode.  sc: LDS scores [h][stride] (MODE_ONLINE);
// lse: this lane's head log-sum-exp (MODE_FINAL).
template <int D, bool BF16, bool INT8, int MODE>
__device__ inline void do_block(const void* kblk, const void* vblk, const QOps<D, BF16>& q,
                                const BlockCtx& bc, WaveAcc<D>& wa, float* sc, int stride,
                                float lse, float* massp) {
  const int lane = threadIdx.x & 63, g = lane >> 4, h = lane & 15;
  f4 acc[4];
  if constexpr (INT8)
    block_scores_i8<D, BF16>((const int8_t*)kblk, q, acc);
  else
    block_scores_16<D, BF16>((const uint16_t*)kblk, q, acc);
  float sig[4][4];
  float mloc = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tk = 16 * r + 4 * g + i;
      const bool ok = bc.head_ok && tk < bc.n_valid;
      sig[r][i] = ok ? acc[r][i] * bc.scale : -INFINITY;
      mloc = fmaxf(mloc, sig[r][i]);
    }
  float p[4][4];
  if constexpr (MODE == MODE_FINAL) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[r][i] = sig[r][i] > -INFINITY ? __expf(sig[r][i] - lse) : 0.f;
    // token mass of this KV head's query group: sum over the 16 lanes of the group
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = group_sum(p[r][i]);
        const int tk = 16 * r + 4 * g + i;
        if (h == 0 && tk < bc.n_valid) massp[bc.mass_idx0 + tk] = s;
      }
  } else {
    const float mnew = fmaxf(wa.m, head_max(mloc));
    const float corr = wa.m > -INFINITY ? __expf(wa.m - mnew) : 0.f;
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[r][i] = sig[r][i] > -INFINITY ? __expf(sig[r][i] - mnew) : 0.f;
        lsum += p[r][i];
      }
    wa.l = wa.l * corr + head_sum(lsum);
    wa.m = mnew;
    if constexpr (MODE == MODE_LSE) return;
    // keep the raw scores for the mass pass
    if (bc.head_ok) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tk = 16 * r + 4 * g + i;
          if (tk < bc.n_valid) sc[h * stride + bc.tok0 + tk] = sig[r][i];
        }
    }
    // rescale O rows (heads 4g+i) by their head's correction
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ci = __shfl(corr, 4 * g + i);
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) wa.o[cb][i] *= ci;
    }
  }
  if constexpr (INT8)
    block_pv_i8<D>((const int8_t*)vblk, p, wa.o);
  else
    block_pv_16<D, BF16>((const uint16_t*)vblk, p, wa.o);
}

// Appends this step's key/value to window slot `slot` of the unit (data only).
__device__ inline void append_row_m(int D, uint16_t* k16, uint16_t* v16, int slot,
                                    const uint16_t* knew, const uint16_t* vnew) {
  for (int ch = threadIdx.x; ch < D; ch += blockDim.x) {
    k16[(size_t)slot * D + ch] = knew[ch];
    v16[vtile_off(slot, ch, D)] = vnew[ch];
  }
}


// value scale of the INT8 part: lane's O channels are 16*cb + lane%16
template <int D>
__device__ inline void apply_vscale(WaveAcc<D>& wa, const float* sv) {
  const int hl = threadIdx.x & 15;
#pragma unroll
  for (int cb = 0; cb < D / 16; ++cb) {
    const float s = sv[16 * cb + hl];
    wa.o[cb] *= s;
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(kMfmaThreads, 2) void attn_mfma_kernel(
    conf_cache c, Dims dm, int layer0, const uint16_t* __restrict__ q_all,
    const uint16_t* __restrict__ knew_all, const uint16_t* __restrict__ vnew_all,
    float* __restrict__ out_all, float* __restrict__ massp_all, int score_cap) {
  // Dynamic LDS: first the fp32 query staging [G][D], then (after the operands
  // are in registers) the scores [G][score_cap + 1], then the O merge buffer.
  extern __shared__ float smem[];
  __shared__ float s_qscale[kMaxGroup];    // power-of-two scale of the INT8 query
  __shared__ float s_snew[kMaxGroup];      // score of this step's token
  __shared__ float s_m[kWaves][kMaxGroup], s_l[kWaves][kMaxGroup];
  __shared__ float s_lse[kMaxGroup], s_pnew[kMaxGroup], s_f[kWaves][kMaxGroup];
  __shared__ float s_sv[D];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, hl = lane & 15;
  const int unit_local = blockIdx.x;
  const int hk = unit_local % dm.Hkv;
  const int lbl = unit_local / dm.Hkv;
  const int lb = layer0 * dm.B + lbl;
  const size_t u = (size_t)lb * dm.Hkv + hk;
  const int G = dm.G;
  const int n8 = c.n8[lb], nw = c.n16[lb], t = c.t[lb];
  const int appended = nw < dm.cap16;
  const int n = n8 + nw + appended;
  const int8_t* k8 = c.k8 + u * (size_t)dm.cap8 * D;
  const int8_t* v8 = c.v8 + u * (size_t)dm.cap8 * D;
  uint16_t* k16 = (uint16_t*)c.k16 + u * (size_t)dm.cap16 * D;
  uint16_t* v16 = (uint16_t*)c.v16 + u * (size_t)dm.cap16 * D;
  const uint16_t* knew = knew_all + (size_t)unit_local * D;
  const uint16_t* vnew = vnew_all + (size_t)unit_local * D;
  const uint16_t* qsrc = q_all + ((size_t)lbl * dm.Hq + (size_t)hk * G) * D;
  float* mp_lb = massp_all + (size_t)lb * dm.Hkv * dm.capt;
  float* massp = mp_lb + (size_t)hk * dm.capt;
  const float rs = 1.0f / sqrtf((float)D);

  if (appended)
    append_row_m(D, k16, v16, nw, knew, vnew);
  else if (tid == 0 && hk == 0)
    atomicOr(c.status, (int)CONF_ST_WINDOW_FULL);

  // ---- query set-up
  float* s_q = smem;
  for (int i = tid; i < G * D; i += kMfmaThreads) s_q[i] = h16_to_f32(qsrc[i], dm.bf16);
  for (int ch = tid; ch < D; ch += kMfmaThreads) s_sv[ch] = c.v_amax[u * D + ch] / 127.0f;
  __syncthreads();
  if (tid < G) {
    float s = 0.f;
    for (int ch = 0; ch < D; ++ch) s = fmaf(s_q[tid * D + ch], h16_to_f32(knew[ch], dm.bf16), s);
    s_snew[tid] = s * rs;
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kMfmaThreads) s_q[i] *= c.k_amax[u * D + i % D] / 127.0f;
  __syncthreads();
  if (tid < G) {
    float mx = 0.f;
    for (int ch = 0; ch < D; ++ch) mx = fmaxf(mx, fabsf(s_q[tid * D + ch]));
    s_qscale[tid] = mx > 0.f ? ldexpf(1.0f, 14 - ilogbf(mx)) : 1.0f;
  }
  __syncthreads();
  const int head_ok = hl < G;
  QOps<D, BF16> q;
  {
    const float al = head_ok ? s_qscale[hl] : 1.0f;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      q.qw[s] = head_ok ? ld16(qsrc + (size_t)hl * D + 32 * s + 8 * g) : (u4){0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ch = 64 * (s >> 1) + 16 * g + 8 * (s & 1) + e;
        const float x = head_ok ? s_q[hl * D + ch] * al : 0.f;
        const _Float16 hi = (_Float16)x;
        q.qh[s][e] = hi;
        q.ql[s][e] = (_Float16)(x - (float)hi);
      }
    }
  }
  const float scale8 = head_ok ? rs / s_qscale[hl] : 0.f;
  const float scale16 = head_ok ? rs : 0.f;
  __syncthreads();  // the staging area becomes the score store

  const int nb8 = (n8 + kTile - 1) / kTile, nbw = (nw + kTile - 1) / kTile;
  const int nblk = nb8 + nbw;
  const int stride = score_cap + 1;
  const bool in_lds = n <= score_cap;
  WaveAcc<D> wa;
  wa.m = -INFINITY;
  wa.l = 0.f;
#pragma unroll
  for (int cb = 0; cb < D / 16; ++cb) wa.o[cb] = (f4){0.f, 0.f, 0.f, 0.f};

  auto ctx = [&](int bi, BlockCtx& bc) {
    if (bi < nb8) {
      bc.n_valid = min(kTile, n8 - bi * kTile);
      bc.tok0 = bi * kTile;
      bc.mass_idx0 = bi * kTile;
      bc.scale = scale8;
    } else {
      const int wb = bi - nb8;
      bc.n_valid = min(kTile, nw - wb * kTile);
      bc.tok0 = n8 + wb * kTile;
      bc.mass_idx0 = dm.cap8 + wb * kTile;
      bc.scale = scale16;
    }
    bc.head_ok = head_ok;
  };
  // Each wavefront meets its INT8 blocks before its window blocks; the value
  // scale of the INT8 codes is applied to the accumulator once, in between.
  bool vscaled = false;

  if (in_lds) {
    float* sc = smem;
    for (int bi = wave; bi < nblk; bi += kWaves) {
      BlockCtx bc;
      ctx(bi, bc);
      if (bi < nb8) {
        do_block<D, BF16, true, MODE_ONLINE>(k8 + (size_t)bi * kTile * D, v8 + (size_t)bi * kTile * D,
                                              q, bc, wa, sc, stride, 0.f, nullptr);
      } else {
        if (!vscaled) {
          apply_vscale<D>(wa, s_sv);
          vscaled = true;
        }
        do_block<D, BF16, false, MODE_ONLINE>(k16 + (size_t)(bi - nb8) * kTile * D,
                                               v16 + (size_t)(bi - nb8) * kTile * D, q, bc, wa, sc,
                                               stride, 0.f, nullptr);
      }
    }
    if (appended && tid < G) sc[tid * stride + n - 1] = s_snew[tid];
  } else {
    for (int bi = wave; bi < nblk; bi += kWaves) {
      BlockCtx bc;
      ctx(bi, bc);
      if (bi < nb8)
        do_block<D, BF16, true, MODE_LSE>(k8 + (size_t)bi * kTile * D, nullptr, q, bc, wa, nullptr,
                                           0, 0.f, nullptr);
      else
        do_block<D, BF16, false, MODE_LSE>(k16 + (size_t)(bi - nb8) * kTile * D, nullptr, q, bc, wa,
                                            nullptr, 0, 0.f, nullptr);
    }
  }
  // ---- merge the running (max, sum) of the waves and add this step's token
  if (lane < 16) {
    s_m[wave][lane] = wa.m;
    s_l[wave][lane] = wa.l;
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][tid]);
    if (appended) M = fmaxf(M, s_snew[tid]);
    float S = 0.f;
    for (int w = 0; w < kWaves; ++w)
      if (s_m[w][tid] > -INFINITY) S += s_l[w][tid] * expf(s_m[w][tid] - M);
    if (appended) S += expf(s_snew[tid] - M);
    const float lse = M + logf(S);
    s_lse[tid] = lse;
    s_pnew[tid] = appended ? expf(s_snew[tid] - lse) : 0.f;
    // weight of each wave's O in the final, normalised sum
    for (int w = 0; w < kWaves; ++w)
      s_f[w][tid] = s_m[w][tid] > -INFINITY ? expf(s_m[w][tid] - lse) : 0.f;
  }
  __syncthreads();

  if (in_lds) {
    // per-token mass of this query group from the stored scores
    const float* sc = smem;
    for (int j = tid; j < n; j += kMfmaThreads) {
      float s = 0.f;
      for (int h = 0; h < G; ++h) s += __expf(sc[h * stride + j] - s_lse[h]);
      massp[j < n8 ? j : dm.cap8 + (j - n8)] = s;
    }
    __syncthreads();
  } else {
    // second pass: probabilities with the final normaliser, mass and values
    const float lse = head_ok ? s_lse[hl] : 0.f;
    for (int bi = wave; bi < nblk; bi += kWaves) {
      BlockCtx bc;
      ctx(bi, bc);
      if (bi < nb8) {
        do_block<D, BF16, true, MODE_FINAL>(k8 + (size_t)bi * kTile * D, v8 + (size_t)bi * kTile * D,
                                             q, bc, wa, nullptr, 0, lse, massp);
      } else {
        if (!vscaled) {
          apply_vscale<D>(wa, s_sv);
          vscaled = true;
        }
        do_block<D, BF16, false, MODE_FINAL>(k16 + (size_t)(bi - nb8) * kTile * D,
                                              v16 + (size_t)(bi - nb8) * kTile * D, q, bc, wa,
                                              nullptr, 0, lse, massp);
      }
    }
    if (appended && tid == 0) {
      float s = 0.f;
      for (int h = 0; h < G; ++h) s += s_pnew[h];
      massp[dm.cap8 + nw] = s;
    }
  }
  if (!vscaled) apply_vscale<D>(wa, s_sv);

  // ---- merge the waves' O tiles in LDS (the score region is free again)
  float* ob = smem;  // [kWaves][G][D]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * g + i;
    if (hh < G) {
      const float f = in_lds ? s_f[wave][hh] : 1.0f;
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) ob[(wave * G + hh) * D + 16 * cb + hl] = wa.o[cb][i] * f;
    }
  }
  __syncthreads();
  float* out = out_all + ((size_t)lbl * dm.Hq + (size_t)hk * G) * D;
  for (int i = tid; i < G * D; i += kMfmaThreads) {
    const int hh = i / D, ch = i % D;
    float s = 0.f;
    for (int w = 0; w < kWaves; ++w) s += ob[(w * G + hh) * D + ch];
    out[i] = fmaf(s_pnew[hh], h16_to_f32(vnew[ch], dm.bf16), s);
  }
  if (arrive_last(c, dm, lb)) ema_update_lb(c, dm, lb, n8, nw, appended, t, mp_lb);
}

int attn_score_cap(const Dims& dm) {
  const int cap = kLdsScoreBytes / (4 * dm.G) - 1;
  return cap < dm.capt + 1 ? cap : dm.capt + 1;
}

size_t attn_dyn_lds(const Dims& dm) {
  const size_t sc = (size_t)dm.G * (attn_score_cap(dm) + 1) * 4;
  const size_t ob = (size_t)kWaves * dm.G * dm.D * 4;
  return sc > ob ? sc : ob;
}

template <int D, bool BF16>
static void launch_t(const Dims& dm, const conf_cache& c, int layer0, int nl, const void* q,
                     const void* k_new, const void* v_new, float* out, float* massp, hipStream_t st) {
  const size_t lds = attn_dyn_lds(dm);
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void*)attn_mfma_kernel<D, BF16>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsScoreBytes);
    attr_set = true;
  }
  hipLaunchKernelGGL((attn_mfma_kernel<D, BF16>), dim3(nl * dm.B * dm.Hkv), dim3(kMfmaThreads), lds,
                     st, c, dm, layer0, (const uint16_t*)q, (const uint16_t*)k_new,
                     (const uint16_t*)v_new, out, massp, attn_score_cap(dm));
}

void launch_attn(const Dims& dm, const conf_cache& c, int layer0, int nl, const void* q,
                 const void* k_new, const void* v_new, float* out, float* massp, hipStream_t st) {
  if (dm.D == 64) {
    if (dm.bf16) launch_t<64, true>(dm, c, layer0, nl, q, k_new, v_new, out, massp, st);
    else launch_t<64, false>(dm, c, layer0, nl, q, k_new, v_new, out, massp, st);
  } else {
    if (dm.bf16) launch_t<128, true>(dm, c, layer0, nl, q, k_new, v_new, out, massp, st);
    else launch_t<128, false>(dm, c, layer0, nl, q, k_new, v_new, out, massp, st);
  }
}

}  // namespace confkv
