// Internal definitions shared by the HIP kernels and the host entry points of
// the CONF-KV decode-step library.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "confkv.h"

namespace confkv {

constexpr int kTile = 64;        // tokens per value tile
constexpr int kMaxGroup = 16;    // query heads per KV head handled by one unit

// Shapes derived once on the host and passed by value to every kernel.
struct Dims {
  int L, B, Hq, Hkv, G, D, V;
  int W, P, n_high, n_low, cap8, cap16, capt;  // capt = cap8 + cap16
  int bf16;                                    // 1: bfloat16, 0: IEEE half
  int pyramid;
  int policy;                                  // CONF_POLICY_*
  // Head-wise keep sets view each KV head of a sequence as a cache of its own:
  // then B counts (sequence, KV head) pairs, Hkv = 1 and Hq = G, while nseq is
  // the number of sequences and hw = KV heads per sequence.  Otherwise nseq = B
  // and hw = 1.
  int headwise, nseq, hw;
  float tau, w_H, w_m, w_p, decay, one_minus_decay, s_ema, s_rec;
};

// Byte offsets of the workspace regions (all 256-byte aligned).
struct WsMap {
  size_t conf_part;   // float [B][n_vchunks][8]
  size_t massp;       // float [L][B][Hkv][capt]  per-KV-head attention mass
  size_t keep;        // uint8 [L][B][capt]       keep flags of conf_step
  size_t plan;        // int32 [L][B][16]         compaction plan
  size_t mv8;         // int32 [L][B][cap8]       (src, dst) pairs, INT8 region
  size_t mv16;        // int32 [L][B][cap16]      (src, dst) pairs, window
  size_t wkeep;       // uint8 [L][B][cap16]      window keep flags minus the demotee
  size_t snap;        // int32 [L][B][3]          (n8, n16, t) before the step's append
  size_t spill;       // float [L][B][Hkv][G][capt] scores beyond the attention's LDS rows
  size_t arkv_part;   // float [L][B][Hkv]        ARKV prefill statistics per KV head
  size_t total;
  int n_vchunks;      // vocab chunks per sequence in the confidence reduction
};

// Tiled layouts of one unit (layer, sequence, KV head).  Every region is cut
// into 64-token tiles of 64*d elements; inside a tile the order is chosen so that
// each 16-byte-per-lane load of a wavefront lands in the lane that feeds it to
// the matrix cores and reads whole cache lines: a key load reads one contiguous
// 1 KB run, a value load four contiguous 256-byte pieces.  The values are grouped
// by g first so that one token's values (as compaction, demotion and the append
// touch them) sit inside one 16*d-byte stretch, 16 bytes per channel, instead of
// being spread over the whole tile.  Write a slot as
// j = 64*tile + 32u + 16a + 4g + b = 64*tile + 16r + row  (u, a in {0,1}; g, b, r in 0..3).
//
//   k8  (INT8 keys):    [r][c / 64][(c / 16) % 4][row][c % 16]
//   v8  (INT8 values):  [g][c][8u + 4a + b]
//   k16 (16-bit keys):  [u][r % 2][c / 32][(c / 8) % 4][row][c % 8]
//   v16 (16-bit values):[u][g][c][4a + b]
__host__ __device__ inline size_t k8_off(int slot, int c, int D) {
  const int jj = slot & 63, r = jj >> 4, row = jj & 15;
  return (size_t)(slot >> 6) * (size_t)(D * kTile) +
         (size_t)((((r * (D >> 6) + (c >> 6)) * 4 + ((c >> 4) & 3)) * 16 + row) * 16 + (c & 15));
}
__host__ __device__ inline size_t k16_off(int slot, int c, int D) {
  const int jj = slot & 31, rr = jj >> 4, row = jj & 15;
  return (size_t)(slot >> 5) * (size_t)(D * 32) +
         (size_t)((((rr * (D >> 5) + (c >> 5)) * 4 + ((c >> 3) & 3)) * 16 + row) * 8 + (c & 7));
}
__host__ __device__ inline size_t v8_off(int slot, int c, int D) {
  const int s = slot & 63;
  const int b = s & 3, g = (s >> 2) & 3, a = (s >> 4) & 1, u = (s >> 5) & 1;
  return (size_t)(slot >> 6) * (size_t)(D * kTile) + (size_t)(g * D + c) * 16 +
         (size_t)((u << 3) | (a << 2) | b);
}
__host__ __device__ inline size_t v16_off(int slot, int c, int D) {
  const int s = slot & 31;
  const int b = s & 3, g = (s >> 2) & 3, a = (s >> 4) & 1;
  return (size_t)(slot >> 5) * (size_t)(D * 32) + (size_t)(g * D + c) * 8 + (size_t)((a << 2) | b);
}

// Buffer descriptors over one region.  A load whose offset lies past the range
// returns zeros without touching memory (and a store there is dropped), so a
// lane with nothing to access uses kNoItem instead of a branch around the access:
// a branch around a load makes the compiler's wait counts wait for every load in
// flight.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kNoItem = 0x7fff0000u;  // beyond every region (all are < 2 GiB)

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ inline float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ inline float h16_to_f32(uint16_t h, int bf16) {
  return bf16 ? bf16_to_f32(h) : f16_to_f32(h);
}

// Pyramid (CONF-KV-L) layer budget, integer floor; identical to the host form.
__host__ __device__ inline int layer_budget(int N, int l, int L, int pyramid) {
  if (!pyramid || L <= 1) return N;
  const long long Dn = 2LL * (L - 1);
  return (int)(((long long)N * (Dn - l)) / Dn);
}

// Symmetric INT8 code, round half to even, clamp to [-127, 127]; s == 0 -> 0.
__device__ inline int8_t quant_code(float x, float s) {
#pragma clang fp contract(off)
  if (!(s > 0.0f)) return 0;
  float r = __builtin_rintf(x / s);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int8_t)(int)r;
}

// The device a host call runs on, for per-device one-time set-up (function
// attributes are set per device); devices beyond kMaxDevices share slot 0's answer
// and set their attributes on every call.
constexpr int kMaxDevices = 64;
inline int current_device_slot() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  return dev;
}

// e4m3 code (OCP "fn" form: sign, four exponent bits with bias 7, three mantissa
// bits, largest finite 448) of y, |y| <= 448, by round-to-nearest-even; the sign
// bit follows y.  ARKV's Quantized state [the ARKV page, Methodology: three-state
// assignment].
__device__ inline int8_t fp8_code(float y) {
  const uint32_t b = __float_as_uint(y);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7FFFFFFFu;  // |y|
  uint32_t code;
  if (a < 0x3C800000u) {  // |y| < 2^-6: subnormal codes, steps of 2^-9
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);  // 0 .. 8 (8: 2^-6)
  } else {
    const int e = (int)(a >> 23) - 127;  // -6 .. 8
    uint32_t m = (a >> 20) & 7u;         // the three mantissa bits kept
    const uint32_t rest = a & 0xFFFFFu;  // the twenty below them
    if (rest > 0x80000u || (rest == 0x80000u && (m & 1u))) ++m;
    code = ((uint32_t)(e + 7) << 3) + m;  // a carry out of m raises the exponent
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return (int8_t)(sign | code);
}

// Value of an e4m3 code (exact in fp32).
__device__ inline float fp8_value(int8_t code) {
  const uint32_t b = (uint8_t)code;
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float v = e == 0 ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (b & 0x80u) ? -v : v;
}

// The 8-bit quantiser of a cache: INT8 (CONF-KV) or e4m3 (ARKV), both with
// scale = absmax / code_max and a zero scale giving code 0.
__host__ __device__ inline float code_max(bool fp8) { return fp8 ? 448.0f : 127.0f; }

__device__ inline int8_t quant8(float x, float s, bool fp8) {
#pragma clang fp contract(off)
  if (!fp8) return quant_code(x, s);
  if (!(s > 0.0f)) return 0;
  const float r = fminf(fmaxf(x / s, -448.0f), 448.0f);
  return fp8_code(r);
}

__device__ inline float code_value(int8_t c, bool fp8) { return fp8 ? fp8_value(c) : (float)c; }

}  // namespace confkv
