// (b)+(c) Decode attention on the CDNA4 matrix cores, the per-token attention
// mass and the EMA update.
//
// CONF-KV explainer, Key contributions (system design): block-wise online-
// softmax attention; Methodology, implementation: dequantisation fused into the
// block-wise attention reads over a dense (compacted) layout; mixed-precision
// storage: INT8 codes with one scale per (KV head, channel); token ranking: the
// EMA of each token's attention mass.
//
// Two launches.  The attention kernel writes, per unit, the mass of its query
// group for every token to the workspace; a small kernel then sums the KV heads
// in index order and applies the EMA.  (A kernel boundary is the cheap way to
// order that: a device-scope fence per workgroup would write back the per-XCD
// L2 caches.)
//
// Work split.  One workgroup (4 wavefronts) per unit (layer, sequence, KV head)
// covers the g = Hq/Hkv query heads that share the unit's keys and values.  The
// unit's tokens are cut into work items of equal byte size: 64-token INT8 blocks
// and 32-token halves of the 64-token window tiles.  Wavefront w takes items w,
// w+4, ...; while it computes item i, the values of item i and the keys of
// item i+4 are in flight.  For an item it forms
//   S^T[16 tokens x 16 heads] = K[16 x d] . Q^T[d x 16]          (v_mfma_f32_16x16x32)
// per 16-token row block, so a lane holds one query head (lane % 16) and four
// tokens per row block; that is the A-operand layout of
//   O[16 heads x 16 channels] += P[16 x 32 tokens] . V[32 tokens x 16 channels]
// so P never leaves registers, and the tiled value layout hands each lane its
// tokens of one channel in one 16-byte load.  Heads beyond g are zero padding.
//
// Precision.  INT8 codes become fp16 exactly, and so do e4m3 codes (ARKV's
// Quantized state), scaled by 2^-8.  The key scale folds into the
// query: q' = q * amax_K/127, times a power of two per head that puts its largest
// entry in [2^14, 2^15), split into fp16 hi + lo parts (two MFMAs, ~22 bits).
// Window keys meet the 16-bit query as stored (exact products).  P is rounded to
// fp16 for INT8 values and fp16 windows, and split into bf16 hi + lo for bfloat16
// windows.  Accumulation is fp32 throughout.  The INT8 value scale multiplies the
// accumulator once, between a wavefront's INT8 items and its window items.
//
// One pass over the keys and values in every case.  The raw scores of the unit
// (fp32) are kept for the per-token mass, which is formed once the softmax
// normaliser is final: in LDS while they fit, and from the first item that does
// not fit on (a cache longer than the LDS rows, such as the first steps after a
// long prefill) in per-unit rows of the workspace.  That costs 4*g bytes per
// token written and read back, against the 2*d (INT8) or 4*d (16-bit) bytes of
// keys and values the unit streams for it.  At d = 128, a cache whose scores do
// not all fit the LDS rows keeps those of its window halves in the wavefronts'
// registers (up to four halves each, a 512-token window), so that the rows hold
// the INT8 tokens only: the 4097-token caches after a long prefill then spill
// nothing.
#include <atomic>

#include "ema.hpp"

namespace confkv {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kAttnThreads = kWaves * 64;
// Dynamic LDS of one workgroup.  At d = 128 as much as lets two workgroups share
// a compute unit (160 KB) beside their static arrays (2 KB each), so that the
// 4097-token caches after a long prefill keep more of their scores on chip.  At
// d = 64 the kernel needs 128 registers, so four workgroups can share a compute
// unit when each takes 38 KB: the units of a d = 64 cache are small (about 1000
// tokens of 128 bytes), their fixed phases (set-up, merge, mass) weigh more, and
// more resident workgroups hide them (measured: attention 0.51 -> 0.55 of 8 TB/s
// on the gpt-oss-20b-shaped cache, against two 76 KB workgroups).
__host__ __device__ constexpr int lds_dyn_bytes(int D) { return D == 64 ? 38 * 1024 : 79360; }
// resident workgroups per compute unit the register budget is set for
__host__ __device__ constexpr int attn_min_blocks(int D) { return D == 64 ? 4 : 2; }

// ONLINE: scores kept in LDS for the mass; SPILL: the same, with the items from
// the first one that does not fit in LDS writing their scores to the workspace;
// PLAIN: no scores kept, for a policy that needs no mass.
enum { MODE_ONLINE = 0, MODE_SPILL = 1, MODE_PLAIN = 2 };

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
// 16 e4m3 codes -> two groups of 8 exact fp16 values, each the code's value / 256:
// a code b placed in the high byte of a 16-bit half keeps its sign bit where fp16
// has it, and one right shift puts its four exponent and three mantissa bits on
// fp16's (exponent bias 15 against e4m3's 7: a factor 2^-8; e4m3 subnormals land
// on fp16 subnormals with the same factor).
__device__ inline uint32_t fp8_pair(uint32_t w, uint32_t sel) {
  const uint32_t x = __builtin_amdgcn_perm(0u, w, sel);
  return (x & 0x80008000u) | ((x >> 1) & 0x3F803F80u);
}

template <bool FP8>
__device__ inline void codes_to_f16(u4 raw, h8& a0, h8& a1) {
  if constexpr (FP8) {
    // selector 0x0c gives a zero byte: halves (byte 0 | byte 1 ...) << 8
    const uint32_t lo = 0x010C000Cu, hi = 0x030C020Cu;
    const uint32_t r0 = fp8_pair(raw.x, lo), r1 = fp8_pair(raw.x, hi);
    const uint32_t r2 = fp8_pair(raw.y, lo), r3 = fp8_pair(raw.y, hi);
    const uint32_t r4 = fp8_pair(raw.z, lo), r5 = fp8_pair(raw.z, hi);
    const uint32_t r6 = fp8_pair(raw.w, lo), r7 = fp8_pair(raw.w, hi);
    a0 = __builtin_bit_cast(h8, (u4){r0, r1, r2, r3});
    a1 = __builtin_bit_cast(h8, (u4){r4, r5, r6, r7});
    return;
  }
  const uint32_t w0 = raw.x ^ 0x80808080u, w1 = raw.y ^ 0x80808080u;
  const uint32_t w2 = raw.z ^ 0x80808080u, w3 = raw.w ^ 0x80808080u;
  const h2 p0 = bias_pair(w0, 0x04010400u), p1 = bias_pair(w0, 0x04030402u);
  const h2 p2 = bias_pair(w1, 0x04010400u), p3 = bias_pair(w1, 0x04030402u);
  const h2 p4 = bias_pair(w2, 0x04010400u), p5 = bias_pair(w2, 0x04030402u);
  const h2 p6 = bias_pair(w3, 0x04010400u), p7 = bias_pair(w3, 0x04030402u);
  a0 = (h8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
  a1 = (h8){p4.x, p4.y, p5.x, p5.y, p6.x, p6.y, p7.x, p7.y};
}

// The factor that turns a converted 8-bit code into its value: the INT8 scale
// amax/127, or for e4m3 the scale amax/448 times the 2^8 the conversion took off.
template <bool FP8>
__device__ inline float code_scale(float amax) {
#pragma clang fp contract(off)
  if constexpr (FP8) return (amax / 448.0f) * 256.0f;
  return amax / 127.0f;
}

__device__ inline u4 ld16(const void* p) { return *(const u4*)p; }

// ---------------------------------------------------------------- work items
template <int D>
struct Buf {
  // one item's keys (INT8 block: [row block r][64-channel half hh]; window half:
  // [r][32-channel step s]) or values ([16-channel block cb])
  u4 x[D / 16];
};

template <int D>
struct WaveAcc {
  float m;        // running max of this lane's head
  float l;        // running sum
  f4 o[D / 16];   // O: lane holds channel 16*cb + lane%16, heads 4*(lane/16) + i
};

// Query operands of one lane (head lane%16, lane group lane/16), kept in LDS as
// [32-channel step s][3] x 16 bytes: the 16-bit query as stored (window keys),
// then the fp16 hi and lo parts of the scaled query (INT8 keys).  Lanes of
// padding heads point at a shared all-zero block.
typedef __attribute__((address_space(3))) const u4 lds_u4;  // a 16-byte LDS chunk

template <int D, bool BF16>
struct QOps {
  const lds_u4* p;  // LDS pointer: stays an LDS read when laundered through asm
  __device__ u4 qw(int s) const { return p[3 * s]; }
  __device__ h8 qh(int s) const { return __builtin_bit_cast(h8, p[3 * s + 1]); }
  __device__ h8 ql(int s) const { return __builtin_bit_cast(h8, p[3 * s + 2]); }
};
template <int D>
__host__ __device__ constexpr int qops_u4(int G) { return (4 * G + 1) * (D / 32) * 3; }

struct Item {
  bool i8;        // INT8 block (64 tokens) or window half-tile (32 tokens)
  int blk;        // INT8 block index, or window item index j (tokens 32j .. 32j+31)
  int n_valid;    // valid tokens in the item
  int tok0;       // unit token index of the first slot (scores in LDS)
  int mass0;      // mass-row index of the first slot
  bool held;      // window half whose raw scores stay in the wavefront's registers
};

// Window halves whose raw scores a wavefront keeps in registers until the
// normaliser is final, when every window half of the unit fits (nw <= 128 * NK):
// s[m] holds the wavefront's m-th newest window half, in the score layout of
// softmax_item (row block r, token 16r + 4*(lane/16) + i, head lane%16).
template <int NK>
struct Held {
  float s[NK > 0 ? NK : 1][2][4];
  int n;  // window halves held (wave-uniform)
};
// At d = 128 the four halves of a 512-token window (32 registers); at d = 64 the
// two of a 256-token window (16 registers).
__host__ __device__ constexpr int held_halves(int D) { return D == 128 ? 4 : 0; }

// lane H of this lane's 16-lane row (DPP row broadcast, a VALU operand)
template <int H>
__device__ inline float row_lane(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + H, 0xF, 0xF, false));
}

// Every item's keys and values are read as D/16 loads of 16 bytes per lane.
// Keys: load i reads the 1 KB run at 1 KB * i, a lane at 16 * lane inside it.
// Values: load i reads 16 channels (16i .. 16i+15) of the four token groups g,
// a lane at 16*D*(lane / 16) + 16*(lane % 16) + 256*i: four 256-byte pieces.
// That holds for INT8 blocks and window halves alike (both are 64 * D bytes), so
// one straight-line load sequence serves both.
//
// The item loads go through buffer descriptors (one per region of the
// unit: INT8 keys, INT8 values, window keys, window values); an item that does
// not exist is loaded at kNoItem (a zero-returning offset past the range), so
// every stage issues the same load instructions with no branch around them.

// Keys and values are read once per step: the loads carry the non-temporal cache
// policy (cache-policy bit 1), which keeps 2.7 GB of single-use data per step
// from churning the L2 and last-level caches (measured: 13% faster than the
// default policy on the 32K, batch-8 cache).
constexpr int kStreamPolicy = 2;

template <int D, int STEP = 1024>
__device__ inline void load_run_rs(rsrc_t r, uint32_t off, int lane_off, Buf<D>& R) {
#pragma unroll
  for (int i = 0; i < D / 16; ++i)
    R.x[i] = __builtin_bit_cast(
        u4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + lane_off + i * STEP), 0,
                                                  kStreamPolicy));
}

// Raw S^T: acc[r][i] is the score of item token 16r + 4*(lane/16) + i for head lane%16.
template <int D, bool BF16, bool FP8>
__device__ inline void scores_i8(const Buf<D>& R, const QOps<D, BF16>& q, f4 acc[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    f4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hh = 0; hh < D / 64; ++hh) {
      h8 k0, k1;
      codes_to_f16<FP8>(R.x[r * (D / 64) + hh], k0, k1);
      a = mma_f16(k0, q.qh(2 * hh), a);
      a = mma_f16(k0, q.ql(2 * hh), a);
      a = mma_f16(k1, q.qh(2 * hh + 1), a);
      a = mma_f16(k1, q.ql(2 * hh + 1), a);
    }
    acc[r] = a;
    // keep one row block's converted codes live at a time
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D, bool BF16>
__device__ inline void scores_16(const Buf<D>& R, const QOps<D, BF16>& q, f4 acc[2]) {
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    f4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      if constexpr (BF16)
        a = mma_bf16(__builtin_bit_cast(bf8, R.x[r * (D / 32) + s]), __builtin_bit_cast(bf8, q.qw(s)),
                     a);
      else
        a = mma_f16(__builtin_bit_cast(h8, R.x[r * (D / 32) + s]), __builtin_bit_cast(h8, q.qw(s)), a);
    }
    acc[r] = a;
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O += P . V.  p[r][i]: probability of item token 16r + 4g + i for head lane%16.
template <int D, bool FP8>
__device__ inline void pv_i8(const Buf<D>& R, const float p[4][4], f4* o) {
  h8 pa[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) pa[u][e] = (_Float16)p[2 * u + (e >> 2)][e & 3];
#pragma unroll
  for (int cb = 0; cb < D / 16; ++cb) {
    h8 v0, v1;
    codes_to_f16<FP8>(R.x[cb], v0, v1);
    o[cb] = mma_f16(pa[0], v0, o[cb]);
    o[cb] = mma_f16(pa[1], v1, o[cb]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O += P . V over a window half.  Slots past the item's end meet p = 0; their
// values are read too, so they must be finite (0 * NaN is NaN in the matrix
// core): conf_cache_reset zeroes the window, and every later write stores a
// caller-supplied or moved value.  (8-bit codes always convert to finite values.)
template <int D, bool BF16>
__device__ inline void pv_16(const Buf<D>& R, const float p[2][4], f4* o) {
  if constexpr (BF16) {
    bf8 ph, pl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = p[e >> 2][e & 3];
      const __bf16 hi = (__bf16)x;
      ph[e] = hi;
      pl[e] = (__bf16)(x - (float)hi);
    }
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) {
      const bf8 v = __builtin_bit_cast(bf8, R.x[cb]);
      o[cb] = mma_bf16(ph, v, o[cb]);
      o[cb] = mma_bf16(pl, v, o[cb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    h8 pa;
#pragma unroll
    for (int e = 0; e < 8; ++e) pa[e] = (_Float16)p[e >> 2][e & 3];
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) o[cb] = mma_f16(pa, __builtin_bit_cast(h8, R.x[cb]), o[cb]);
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
__device__ inline float wave_sum(float x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}
__device__ inline float wave_max(float x) {
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// Where a unit's raw scores go: LDS rows [G][stride] indexed by the unit's token
// index for the items before token `jsp`, and from there on the workspace rows
// [G][capt] fp32, indexed by slot like the mass rows (INT8 slot i at i, window
// slot w at cap8 + w), so that every stored row block is 16-byte aligned.
struct ScoreSink {
  float* lds;
  int stride;
  rsrc_t spill;
  int capt;
  int jsp;
};

// Softmax bookkeeping of one item with R row blocks (R = 4 INT8, 2 window):
// update the running (max, sum), keep the scores (MODE_ONLINE, MODE_SPILL),
// rescale O and fill p.
template <int R, int MODE, int D>
__device__ inline void softmax_item(const f4* acc, float scale, bool head_ok, const Item& I,
                                    WaveAcc<D>& wa, const ScoreSink& sk, float p[R][4],
                                    float sig[R][4]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, h = lane & 15;
  float mloc = -INFINITY;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tk = 16 * r + 4 * g + i;
      sig[r][i] = (head_ok && tk < I.n_valid) ? acc[r][i] * scale : -INFINITY;
      mloc = fmaxf(mloc, sig[r][i]);
    }
  const float mnew = fmaxf(wa.m, head_max(mloc));
  const float corr = wa.m > -INFINITY ? __expf(wa.m - mnew) : 0.f;
  float lsum = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[r][i] = sig[r][i] > -INFINITY ? __expf(sig[r][i] - mnew) : 0.f;
      lsum += p[r][i];
    }
  wa.l = wa.l * corr + head_sum(lsum);
  wa.m = mnew;
  if constexpr (MODE != MODE_PLAIN) {
    // wave-uniform; a held window half goes neither to LDS nor to the workspace
    const bool to_lds = !I.held && (MODE == MODE_ONLINE || I.tok0 < sk.jsp);
    if (to_lds && head_ok) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tk = 16 * r + 4 * g + i;
          if (tk < I.n_valid) sk.lds[h * sk.stride + I.tok0 + tk] = sig[r][i];
        }
    }
    if constexpr (MODE == MODE_SPILL) {
      // one 16-byte store per row block: this lane's four tokens of its head.
      // Every item issues them; those of an item kept in LDS and of padding heads
      // go to an offset past the rows' range and are dropped, so no branch
      // surrounds a store and the wait counts of the loads in flight stay exact.
      // Tokens past the item's end store -inf into their own (unused) slots.
      const uint32_t base = (!to_lds && !I.held && head_ok)
                                ? 4u * (uint32_t)(h * sk.capt + I.mass0 + 4 * g)
                                : kNoItem;
#pragma unroll
      for (int r = 0; r < R; ++r)
        __builtin_amdgcn_raw_buffer_store_b128(
            (u4){__float_as_uint(sig[r][0]), __float_as_uint(sig[r][1]),
                 __float_as_uint(sig[r][2]), __float_as_uint(sig[r][3])},
            sk.spill, (int)(base + 64u * r), 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float ci = __shfl(corr, 4 * g + i);
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) wa.o[cb][i] *= ci;
  }
}

template <int D, bool BF16, int MODE, bool FP8>
__device__ inline void compute_item(const Item& I, Buf<D>& K, const Buf<D>& V,
                                    const QOps<D, BF16>& q, float scale8, float scale16,
                                    bool head_ok, WaveAcc<D>& wa, const ScoreSink& sk, rsrc_t kr,
                                    uint32_t koff, int klane, float hs[2][4]) {
  // Re-read the query operands from LDS for every item instead of letting the
  // compiler hoist 48 registers' worth of them out of the item loop.
  QOps<D, BF16> ql = q;
  __asm__ volatile("" : "+v"(ql.p));
  if (I.i8) {
    f4 acc[4];
    scores_i8<D, BF16, FP8>(K, ql, acc);
    load_run_rs<D>(kr, koff, klane, K);  // the keys are used: the next item's start loading
    float p[4][4], sig[4][4];
    softmax_item<4, MODE, D>(acc, scale8, head_ok, I, wa, sk, p, sig);
    __builtin_amdgcn_sched_barrier(0);
    pv_i8<D, FP8>(V, p, wa.o);
  } else {
    f4 acc[2];
    scores_16<D, BF16>(K, ql, acc);
    load_run_rs<D>(kr, koff, klane, K);
    float p[2][4];
    softmax_item<2, MODE, D>(acc, scale16, head_ok, I, wa, sk, p, hs);
    __builtin_amdgcn_sched_barrier(0);
    pv_16<D, BF16>(V, p, wa.o);
  }
}

// This wavefront's O tile into the merge buffer ob [4][G][D]: lane (g, hl) holds
// heads 4g .. 4g+3 of channels 16*cb + hl.
template <int D>
__device__ inline void store_o(const WaveAcc<D>& wa, float* ob, int G) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, hl = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * g + i;
    if (hh < G) {
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) ob[(wave * G + hh) * D + 16 * cb + hl] = wa.o[cb][i];
    }
  }
}

// value scale of the INT8 part: the lane's O channels are 16*cb + lane%16
template <int D>
__device__ inline void apply_vscale(WaveAcc<D>& wa, const float* sv) {
  const int hl = threadIdx.x & 15;
#pragma unroll
  for (int cb = 0; cb < D / 16; ++cb) wa.o[cb] *= sv[16 * cb + hl];
}

// sum[r][i] += e[r][i] of heads 0, 1, ..., G-1 in that order: every lane of a
// 16-lane row (one token group, head = lane % 16) ends with its row's sum
template <int H = 0>
__device__ inline void add_heads_in_order(const float (&e)[2][4], float (&sum)[2][4], int G) {
  if constexpr (H < kMaxGroup) {
    if (H < G) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[r][i] += row_lane<H>(e[r][i]);
      add_heads_in_order<H + 1>(e, sum, G);
    }
  }
}

// One pass of a wavefront over its items (it = wave, wave + 4, ...), software
// pipelined on one key and one value buffer: an item's values load from the
// start of its stage, and the next item's keys as soon as this item's scores
// are formed.  The key load is issued for every stage (an item past the end
// reads at kNoItem), so no branch surrounds a load.  The INT8 items and the
// window items run as two loops: each loop body is straight-line code, so the
// compiler's wait counts stay exact (with both item kinds in one loop body it
// merged the two paths' counts and waited for the values before the scores).
// `kb` holds (or is receiving) the keys of item `wave`.  With `hold` every window
// half of the wavefront (at most NK) keeps its raw scores in `held`.
struct UnitRs {
  rsrc_t k8, v8, k16, v16;  // the unit's four regions
};

template <int D, bool BF16, int MODE, bool FP8, int NK>
__device__ inline void wave_pass(int nitems, int nb8, int n8, int nw, int cap8, const UnitRs& rs,
                                 const QOps<D, BF16>& q, float scale8, float scale16, bool head_ok,
                                 WaveAcc<D>& wa, const float* sv, const ScoreSink& sk,
                                 Buf<D>& kb, bool hold, Held<NK>& held) {
  // wave-uniform, so that the descriptor choice per item is a scalar select
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int klane = 16 * lane, vlane = 16 * D * (lane >> 4) + 16 * (lane & 15);
  const uint32_t ib = (uint32_t)kTile * D;  // bytes per item in every region
  Buf<D> V;
  int it = wave;
  for (; it < nb8; it += kWaves) {  // INT8 blocks
    load_run_rs<D, 256>(rs.v8, (uint32_t)it * ib, vlane, V);
    const int nx = it + kWaves;
    Item I;
    I.i8 = true;
    I.blk = it;
    I.n_valid = min(kTile, n8 - it * kTile);
    I.tok0 = it * kTile;
    I.mass0 = it * kTile;
    I.held = false;
    float unused[2][4];
    compute_item<D, BF16, MODE, FP8>(
        I, kb, V, q, scale8, scale16, head_ok, wa, sk, nx < nb8 ? rs.k8 : rs.k16,
        nx < nitems ? (uint32_t)(nx < nb8 ? nx : nx - nb8) * ib : kNoItem, klane, unused);
  }
  // the INT8 value scale, once, between the INT8 and the window items (O is still 0
  // for a wavefront without INT8 items)
  apply_vscale<D>(wa, sv);
  for (; it < nitems; it += kWaves) {  // window halves
    const int j = it - nb8;
    load_run_rs<D, 256>(rs.v16, (uint32_t)j * ib, vlane, V);
    const int nx = it + kWaves;
    Item I;
    I.i8 = false;
    I.blk = j;
    I.n_valid = min(32, nw - 32 * j);
    I.tok0 = n8 + 32 * j;
    I.mass0 = cap8 + 32 * j;
    I.held = NK > 0 && hold;
    float hs[2][4];
    compute_item<D, BF16, MODE, FP8>(I, kb, V, q, scale8, scale16, head_ok, wa, sk, rs.k16,
                                     nx < nitems ? (uint32_t)(nx - nb8) * ib : kNoItem, klane,
                                     hs);
    if (NK > 0 && hold) {  // newest first
#pragma unroll
      for (int m = (NK > 0 ? NK : 1) - 1; m > 0; --m)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) held.s[m][r][i] = held.s[m - 1][r][i];
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) held.s[0][r][i] = hs[r][i];
      ++held.n;
    }
  }
}

// First unit token whose item keeps its scores in the workspace rather than in
// LDS rows of `cap` tokens: INT8 block i ends at 64(i+1) and window half j at
// n8 + 32(j+1), and an item stays in LDS when it ends at or before `cap`.  Every
// item from that one on spills, so the LDS holds tokens [0, jsp) and the
// workspace rows the rest.
__host__ __device__ inline int spill_start(int n8, int cap) {
  const int c64 = cap & ~63;
  return n8 > c64 ? c64 : n8 + ((cap - n8) & ~31);
}

// One workgroup per unit.  The unit of KV head 0 also records the (layer,
// sequence)'s sizes before this step in `snap` [L][B][3] = (n8, n16, t) for the
// EMA kernel, which must not read the counters it advances.
template <int D, bool BF16, bool FP8>
__global__ __launch_bounds__(kAttnThreads, attn_min_blocks(D)) void attn_kernel(
    conf_cache c, Dims dm, int layer0, const uint16_t* __restrict__ q_all,
    const uint16_t* __restrict__ knew_all, const uint16_t* __restrict__ vnew_all,
    float* __restrict__ out_all, float* __restrict__ massp_all, int32_t* __restrict__ snap,
    float* __restrict__ spill_all, int score_cap) {
  // Dynamic LDS: the query operands, then a region of score_cap | 1 rows for the
  // scores [G][stride], stride = the unit's LDS-held tokens | 1.  The O merge
  // buffer [4][G][D] follows the unit's rows when the region has room for both;
  // otherwise it takes the rows' space once the mass phase has read them.
  // Scores beyond the LDS rows go to spill_all [L][B][Hkv][G][capt].
  extern __shared__ float dyn_lds[];
  u4* s_qops = (u4*)dyn_lds;
  float* smem = dyn_lds + 4 * qops_u4<D>(dm.G);
  __shared__ float s_qscale[kMaxGroup];    // power-of-two scale of the INT8 query
  __shared__ float s_snew[kMaxGroup];      // score of this step's token
  __shared__ float s_m[kWaves][kMaxGroup], s_l[kWaves][kMaxGroup];
  __shared__ float s_lse[kMaxGroup], s_pnew[kMaxGroup], s_f[kWaves][kMaxGroup];
  __shared__ float s_sv[D];
  __shared__ float s_vn[D];                 // this step's value as fp32

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, hl = lane & 15;
  const int unit_local = blockIdx.x;
  const int hk = unit_local % dm.Hkv;
  const int lbl = unit_local / dm.Hkv;
  const int lb = layer0 * dm.B + lbl;
  const size_t u = (size_t)lb * dm.Hkv + hk;
  const int G = dm.G;
  const int8_t* k8 = c.k8 + u * (size_t)dm.cap8 * D;
  const int8_t* v8 = c.v8 + u * (size_t)dm.cap8 * D;
  uint16_t* k16 = (uint16_t*)c.k16 + u * (size_t)dm.cap16 * D;
  uint16_t* v16 = (uint16_t*)c.v16 + u * (size_t)dm.cap16 * D;
  const uint16_t* knew = knew_all + (size_t)unit_local * D;
  const uint16_t* vnew = vnew_all + (size_t)unit_local * D;
  const uint16_t* qsrc = q_all + ((size_t)lbl * dm.Hq + (size_t)hk * G) * D;
  float* massp = massp_all + u * dm.capt;
  const float rs = 1.0f / sqrtf((float)D);
  const bool head_ok = hl < G;


  // ---- set-up.  Every global load is issued before the first wait.  The query
  // group is read as 16-byte chunks (8 channels of one head); the thread holding
  // chunk k of head h also reads the same 8 channels of the key absmax row and of
  // the new key.  The last D/4 threads read the value absmax row and the new
  // value.  Then the keys of INT8 block `wave` start loading speculatively (they
  // need no counter), and only then are the counters used.
  const int nq = G * D / 8;                 // query chunks (<= 256)
  const int qh_ = tid / (D / 8), qk = tid % (D / 8);
  const int vt = tid - (kAttnThreads - D / 4);
  const u4 z4 = {0u, 0u, 0u, 0u};
  u4 rq = z4, rka0 = z4, rka1 = z4, rkn = z4, rva = z4, rvn = z4;
  if (tid < nq) {
    rq = ld16(qsrc + 8 * tid);
    rka0 = ld16(c.k_amax + u * D + 8 * qk);
    rka1 = ld16(c.k_amax + u * D + 8 * qk + 4);
    rkn = ld16(knew + 8 * qk);
  }
  if (vt >= 0) {
    rva = ld16(c.v_amax + u * D + 4 * vt);
    if (vt < D / 8) rvn = ld16(vnew + 8 * vt);
  }
  const UnitRs urs{make_rsrc(k8, (uint32_t)dm.cap8 * D), make_rsrc(v8, (uint32_t)dm.cap8 * D),
                   make_rsrc(k16, (uint32_t)dm.cap16 * D * 2),
                   make_rsrc(v16, (uint32_t)dm.cap16 * D * 2)};
  const uint32_t ib = (uint32_t)kTile * D;  // bytes per item in every region
  Buf<D> cur;
  // (a block past the region reads as zeros: the descriptor's range check)
  load_run_rs<D>(urs.k8, (uint32_t)wave * ib, 16 * lane, cur);
  const int n8 = c.n8[lb], nw = c.n16[lb], t = c.t[lb];
  const int appended = nw < dm.cap16;
  const int n = n8 + nw + appended;
  const int nb8 = (n8 + kTile - 1) / kTile;
  const int nitems = nb8 + (nw + 31) / 32;
  // CONF-KV and ARKV rank on each token's attention mass; the baselines do not
  const bool mass = dm.policy == CONF_POLICY_CONFKV || dm.policy == CONF_POLICY_ARKV;
  const int nc = n8 + nw;  // cached tokens (this step's token is handled apart)
  // When the cache's scores would not all fit the LDS rows and its window halves
  // fit the wavefronts' registers, the LDS rows and the workspace keep the INT8
  // tokens' scores only: ns tokens are kept there.
  constexpr int NK = held_halves(D);
  const bool hold = mass && nw <= kWaves * NK * 32 && spill_start(n8, score_cap) < nc;
  const int ns = hold ? n8 : nc;
  const int jsp = min(spill_start(n8, score_cap), ns);
  const int stride = jsp | 1;  // odd, so that the 16 heads of a store spread over banks
  const int region = max(G * (score_cap | 1), kWaves * G * D);
  const bool ob_apart = G * stride + kWaves * G * D <= region;  // uniform over the workgroup
  float* ob = ob_apart ? smem + G * stride : smem;
  const ScoreSink sink{smem, stride,
                       make_rsrc(spill_all + u * (size_t)G * dm.capt,
                                 mass && spill_all ? (uint32_t)(G * dm.capt * 4) : 0u),
                       dm.capt, jsp};
  // the speculative keys are this wavefront's first item unless the INT8 part is short
  if (wave < nitems && wave >= nb8)
    load_run_rs<D>(urs.k16, (uint32_t)(wave - nb8) * ib, 16 * lane, cur);

  if (hk == 0 && tid == 0) {
    snap[3 * lb] = n8;
    snap[3 * lb + 1] = nw;
    snap[3 * lb + 2] = t;
  }
  if (!appended && tid == 0 && hk == 0) atomicOr(c.status, (int)CONF_ST_WINDOW_FULL);
  // this step's row into window slot nw; the new value and the value scale into LDS
  if (appended && qh_ == 0 && tid < nq)
    *(u4*)(k16 + k16_off(nw, 8 * qk, D)) = rkn;  // 8 channels are contiguous in a key tile
  if (vt >= 0) {
    const uint32_t wa4[4] = {rva.x, rva.y, rva.z, rva.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) s_sv[4 * vt + e] = code_scale<FP8>(__uint_as_float(wa4[e]));
    if (vt < D / 8) {
      const uint32_t w[4] = {rvn.x, rvn.y, rvn.z, rvn.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t b16 = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        s_vn[8 * vt + e] = h16_to_f32(b16, dm.bf16);
        if (appended) v16[v16_off(nw, 8 * vt + e, D)] = b16;
      }
    }
  }
  // Per head, from its D/8 chunk threads (consecutive lanes of one wavefront):
  // the power-of-two scale that puts max |q * amax_K / 127| in [2^14, 2^15), the
  // new token's score, and the query operands (each thread writes its own chunks).
  {
    float qv[8], x8[8];
    float mx = 0.f, sc = 0.f;
    const uint32_t wq[4] = {rq.x, rq.y, rq.z, rq.w}, wn[4] = {rkn.x, rkn.y, rkn.z, rkn.w};
    const uint32_t wk[8] = {rka0.x, rka0.y, rka0.z, rka0.w, rka1.x, rka1.y, rka1.z, rka1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qv[e] = h16_to_f32((uint16_t)(wq[e >> 1] >> (16 * (e & 1))), dm.bf16);
      const float kn = h16_to_f32((uint16_t)(wn[e >> 1] >> (16 * (e & 1))), dm.bf16);
      x8[e] = qv[e] * code_scale<FP8>(__uint_as_float(wk[e]));
      mx = fmaxf(mx, fabsf(x8[e]));
      sc = fmaf(qv[e], kn, sc);
    }
#pragma unroll
    for (int off = 1; off < D / 8; off <<= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, off));
      sc += __shfl_xor(sc, off);
    }
    const float al = mx > 0.f ? ldexpf(1.0f, 14 - ilogbf(mx)) : 1.0f;
    if (tid < nq) {
      if (qk == 0) {
        s_snew[qh_] = sc * rs;
        s_qscale[qh_] = al;
      }
      // INT8-key operands: channels 8k .. 8k+7 = 64*(s/2) + 16*g + 8*(s%2) + e
      const int s8 = 2 * (qk / 8) + (qk & 1), g8 = (qk % 8) / 2;
      h8 hi8, lo8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = x8[e] * al;
        const _Float16 hi = (_Float16)y;
        hi8[e] = hi;
        lo8[e] = (_Float16)(y - (float)hi);
      }
      u4* d8 = s_qops + (qh_ * 4 + g8) * (D / 32) * 3 + 3 * s8;
      d8[1] = __builtin_bit_cast(u4, hi8);
      d8[2] = __builtin_bit_cast(u4, lo8);
      // window-key operands: the 16-bit query as stored, channels 32*s + 8*g + e
      s_qops[(qh_ * 4 + qk % 4) * (D / 32) * 3 + 3 * (qk / 4)] = rq;
    }
    // the all-zero operands that padding heads point at
    if (tid < (D / 32) * 3) s_qops[4 * G * (D / 32) * 3 + tid] = z4;
  }
  __syncthreads();  // operands, scales and the new token's values complete
  const QOps<D, BF16> q{(const lds_u4*)(head_ok ? s_qops + (hl * 4 + g) * (D / 32) * 3
                                                : s_qops + 4 * G * (D / 32) * 3)};
  const float scale8 = head_ok ? rs / s_qscale[hl] : 0.f;
  const float scale16 = head_ok ? rs : 0.f;

  WaveAcc<D> wa;
  wa.m = -INFINITY;
  wa.l = 0.f;
#pragma unroll
  for (int cb = 0; cb < D / 16; ++cb) wa.o[cb] = (f4){0.f, 0.f, 0.f, 0.f};

  Held<NK> held;
  held.n = 0;
  if (!mass)
    wave_pass<D, BF16, MODE_PLAIN, FP8, NK>(nitems, nb8, n8, nw, dm.cap8, urs, q, scale8,
                                            scale16, head_ok, wa, s_sv, sink, cur, false, held);
  else if (jsp >= ns)
    wave_pass<D, BF16, MODE_ONLINE, FP8, NK>(nitems, nb8, n8, nw, dm.cap8, urs, q, scale8,
                                             scale16, head_ok, wa, s_sv, sink, cur, hold, held);
  else
    wave_pass<D, BF16, MODE_SPILL, FP8, NK>(nitems, nb8, n8, nw, dm.cap8, urs, q, scale8,
                                            scale16, head_ok, wa, s_sv, sink, cur, hold, held);
  // ---- merge the waves' running (max, sum) and add this step's token.  Each
  // wavefront's O (value scale applied, not yet normalised) goes to LDS before
  // the barrier, and the O merge shares a phase with the mass; when its buffer
  // reuses the scores' space, O waits in registers until the mass phase is done.
  if (lane < 16) {
    s_m[wave][lane] = wa.m;
    s_l[wave][lane] = wa.l;
  }
  if (ob_apart) store_o<D>(wa, ob, G);
  __syncthreads();  // also orders the spilled scores before their reads below
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
    for (int w = 0; w < kWaves; ++w)
      s_f[w][tid] = s_m[w][tid] > -INFINITY ? expf(s_m[w][tid] - lse) : 0.f;
  }
  __syncthreads();

  float* out = out_all + ((size_t)lbl * dm.Hq + (size_t)hk * G) * D;
  if (mass) {
    // Per-token mass of this query group from the stored scores, summed over the
    // heads in order: four tokens per thread, the scores of four heads read
    // together (an index past the end reads the last token and is not stored).
    // Tokens [0, jsp) from the LDS rows, the rest of the first ns from the
    // workspace rows, and the window halves held in registers by their wavefronts
    // (the heads' terms gathered lane by lane, added in the same order).
    if (hold) {
      // this wavefront's first window half; held.s[m] is its (held.n-1-m)-th
      const int jf = (wave >= nb8 ? wave : wave + kWaves * ((nb8 - wave + kWaves - 1) / kWaves)) -
                     nb8;
      const float l = head_ok ? s_lse[hl] : 0.f;
#pragma unroll
      for (int m = 0; m < NK; ++m) {
        if (m < held.n) {
          const int j = jf + kWaves * (held.n - 1 - m);
          const int nv = min(32, nw - 32 * j);
          float e[2][4], sum[2][4];
#pragma unroll
          for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              e[r][i] = head_ok ? __expf(held.s[m][r][i] - l) : 0.f;
              sum[r][i] = 0.f;
            }
          add_heads_in_order(e, sum, G);
#pragma unroll
          for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int tk = 16 * r + 4 * g + i;
              if (hl == i && tk < nv) massp[dm.cap8 + 32 * j + tk] = sum[r][i];
            }
        }
      }
    }
    const int nl = jsp;
    for (int j0 = tid; j0 < nl; j0 += 4 * kAttnThreads) {
      float s[4] = {0.f, 0.f, 0.f, 0.f};
      int jj[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) jj[k] = min(j0 + k * kAttnThreads, nl - 1);
      int h = 0;
      for (; h + 4 <= G; h += 4) {
        float x[4][4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int k = 0; k < 4; ++k) x[e][k] = smem[(h + e) * stride + jj[k]];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float l = s_lse[h + e];
#pragma unroll
          for (int k = 0; k < 4; ++k) s[k] += __expf(x[e][k] - l);
        }
      }
      for (; h < G; ++h) {
        const float l = s_lse[h];
        const float* row = smem + h * stride;
#pragma unroll
        for (int k = 0; k < 4; ++k) s[k] += __expf(row[jj[k]] - l);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = j0 + k * kAttnThreads;
        if (j < nl) massp[j < n8 ? j : dm.cap8 + (j - n8)] = s[k];
      }
    }
    const float* sp = spill_all + u * (size_t)G * dm.capt;
    for (int j0 = nl + tid; j0 < ns; j0 += 4 * kAttnThreads) {
      float s[4] = {0.f, 0.f, 0.f, 0.f};
      int sl[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = min(j0 + k * kAttnThreads, ns - 1);
        sl[k] = j < n8 ? j : dm.cap8 + (j - n8);
      }
      int h = 0;
      for (; h + 4 <= G; h += 4) {
        float x[4][4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int k = 0; k < 4; ++k) x[e][k] = sp[(size_t)(h + e) * dm.capt + sl[k]];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float l = s_lse[h + e];
#pragma unroll
          for (int k = 0; k < 4; ++k) s[k] += __expf(x[e][k] - l);
        }
      }
      for (; h < G; ++h) {
        const float l = s_lse[h];
        const float* row = sp + (size_t)h * dm.capt;
#pragma unroll
        for (int k = 0; k < 4; ++k) s[k] += __expf(row[sl[k]] - l);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (j0 + k * kAttnThreads < ns) massp[sl[k]] = s[k];
    }
    // this step's token, from its score in registers (same sums, same order)
    if (appended && tid == kAttnThreads - 1) {
      float s = 0.f;
      for (int h = 0; h < G; ++h) s += __expf(s_snew[h] - s_lse[h]);
      massp[dm.cap8 + nw] = s;
    }
  }
  if (!ob_apart) {
    __syncthreads();  // every score read: their space takes the O merge buffer
    store_o<D>(wa, ob, G);
    __syncthreads();
  }
  // O = sum over wavefronts of O_w * exp(m_w - lse), plus this step's token
  for (int i = tid; i < G * D; i += kAttnThreads) {
    const int hh = i / D, ch = i % D;
    float s = 0.f;
    for (int w = 0; w < kWaves; ++w) s += ob[(w * G + hh) * D + ch] * s_f[w][hh];
    out[i] = fmaf(s_pnew[hh], s_vn[ch], s);
  }
}

// EMA of every token once all KV heads' mass rows exist (kernel boundary).  Each
// (layer, sequence) is spread over gridDim.y workgroups that read the sizes from
// the attention kernel's snapshot; workgroup y = 0 then advances n16 and t.
constexpr int kEmaThreads = 256;

__global__ __launch_bounds__(kEmaThreads) void ema_kernel(conf_cache c, Dims dm, int layer0,
                                                          const float* __restrict__ massp_all,
                                                          const int32_t* __restrict__ snap) {
  const int lb = layer0 * dm.B + blockIdx.x;
  const int n8 = snap[3 * lb], nw = snap[3 * lb + 1], t = snap[3 * lb + 2];
  ema_tokens(c, dm, lb, massp_all, n8, nw, t, blockIdx.y * kEmaThreads + threadIdx.x,
             gridDim.y * kEmaThreads);
  if (blockIdx.y == 0 && threadIdx.x == 0) {
    c.n16[lb] = nw + (nw < dm.cap16);
    c.t[lb] = t + 1;
  }
}

// The EMA launch that follows an attention launch whose EMA is pending.
void launch_ema(const Dims& dm, const conf_cache& c, int layer0, int nl, const float* massp,
                const int32_t* snap, hipStream_t st) {
  // token chunks per (layer, sequence): enough for the largest budget plus the
  // window growth of one phase (a head-wise head typically holds up to twice the
  // per-head budget); larger caches loop inside the workgroups
  const int typical = (dm.n_low > dm.n_high ? dm.n_low : dm.n_high) * (dm.headwise ? 2 : 1) +
                      dm.W + 1;
  const int cap = dm.capt < typical ? dm.capt : typical;
  const int chunks = (cap + kEmaThreads - 1) / kEmaThreads;
  hipLaunchKernelGGL(ema_kernel, dim3(nl * dm.B, chunks), dim3(kEmaThreads), 0, st, c, dm, layer0,
                     massp, snap);
}

// Scores one workgroup keeps in LDS (G rows of stride cap | 1, odd so that the
// 16 heads of a store spread over banks), after the query operands; the O merge
// buffer reuses their space after the mass phase.
static int qops_bytes(const Dims& dm) {
  return 16 * (dm.D == 64 ? qops_u4<64>(dm.G) : qops_u4<128>(dm.G));
}

int attn_score_cap(const Dims& dm) {
  int cap = (lds_dyn_bytes(dm.D) - qops_bytes(dm)) / (4 * dm.G) - 1;
  cap &= ~1;
  return cap < dm.capt + 2 ? cap : dm.capt + 2;
}

// Workspace rows for the scores a unit cannot keep in LDS: [U][G][capt] fp32, needed
// by the policies that rank on attention mass once a cache may outgrow the LDS rows
// (a cache of at most score_cap tokens never spills).
size_t attn_spill_bytes(const Dims& dm) {
  const bool mass = dm.policy == CONF_POLICY_CONFKV || dm.policy == CONF_POLICY_ARKV;
  if (!mass || attn_score_cap(dm) >= dm.capt) return 0;
  return (size_t)dm.L * dm.B * dm.Hkv * dm.G * dm.capt * sizeof(float);
}

size_t attn_dyn_lds(const Dims& dm) {
  const size_t sc = (size_t)dm.G * (attn_score_cap(dm) | 1);
  const size_t ob = (size_t)kWaves * dm.G * dm.D;  // shares the scores' space
  return (size_t)qops_bytes(dm) + 4 * (sc > ob ? sc : ob);
}

template <int D, bool BF16, bool FP8>
static void launch_t(const Dims& dm, const conf_cache& c, int layer0, int nl, const void* q,
                     const void* k_new, const void* v_new, float* out, float* massp,
                     int32_t* snap, float* spill, bool with_ema, hipStream_t st) {
  // the dynamic-LDS limit is a per-device attribute of the function: set it once per device
  static std::atomic<bool> attr_set[kMaxDevices];
  const int slot = current_device_slot();
  if (slot < 0 || !attr_set[slot].load(std::memory_order_acquire)) {
    (void)hipFuncSetAttribute((const void*)attn_kernel<D, BF16, FP8>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds_dyn_bytes(D));
    if (slot >= 0) attr_set[slot].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL((attn_kernel<D, BF16, FP8>), dim3(nl * dm.B * dm.Hkv), dim3(kAttnThreads),
                     attn_dyn_lds(dm), st, c, dm, layer0, (const uint16_t*)q,
                     (const uint16_t*)k_new, (const uint16_t*)v_new, out, massp, snap, spill,
                     attn_score_cap(dm));
  if (with_ema) launch_ema(dm, c, layer0, nl, massp, snap, st);
  // otherwise a launch that applies the EMA itself follows
}

template <int D_, bool BF16_, bool FP8_>
struct Variant {
  static constexpr int D = D_;
  static constexpr bool BF16 = BF16_;
  static constexpr bool FP8 = FP8_;
};

void launch_attn(const Dims& dm, const conf_cache& c, int layer0, int nl, const void* q,
                 const void* k_new, const void* v_new, float* out, float* massp, int32_t* snap,
                 float* spill, bool with_ema, hipStream_t st) {
  auto go = [&](auto kernel_tag) {
    constexpr int D = decltype(kernel_tag)::D;
    constexpr bool BF16 = decltype(kernel_tag)::BF16;
    constexpr bool FP8 = decltype(kernel_tag)::FP8;
    launch_t<D, BF16, FP8>(dm, c, layer0, nl, q, k_new, v_new, out, massp, snap, spill, with_ema,
                           st);
  };
  // the 8-bit region holds e4m3 codes under ARKV, INT8 codes otherwise
  const bool fp8 = dm.policy == CONF_POLICY_ARKV;
  if (dm.D == 64) {
    if (dm.bf16) {
      if (fp8) go(Variant<64, true, true>{}); else go(Variant<64, true, false>{});
    } else {
      if (fp8) go(Variant<64, false, true>{}); else go(Variant<64, false, false>{});
    }
  } else {
    if (dm.bf16) {
      if (fp8) go(Variant<128, true, true>{}); else go(Variant<128, true, false>{});
    } else {
      if (fp8) go(Variant<128, false, true>{}); else go(Variant<128, false, false>{});
    }
  }
}

}  // namespace confkv
