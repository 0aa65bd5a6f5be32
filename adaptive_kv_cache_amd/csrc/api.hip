// Host side of the C ABI declared in include/confkv.h: argument validation,
// workspace layout and kernel launches.  No call allocates device memory or
// synchronises the device.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "common.hpp"

namespace confkv {
// kernel launchers (one translation unit per step)
int conf_vchunks(int V);
void launch_confidence(const Dims&, const float*, float*, float*, int32_t*, hipStream_t);
void launch_reset(const Dims&, const conf_cache&, hipStream_t);
void launch_attn(const Dims&, const conf_cache&, int, int, const void*, const void*, const void*,
                 float*, float*, int32_t*, float*, bool, hipStream_t);
size_t attn_spill_bytes(const Dims&);
void launch_ingest(const Dims&, const conf_cache&, int, int, int, const void*, const void*,
                   hipStream_t);
void launch_select(const Dims&, const conf_cache&, int, int, const int32_t*, uint8_t*, hipStream_t);
void launch_joint_select(const Dims&, const conf_cache&, int, int, const int32_t*, uint8_t*,
                         const float*, const int32_t*, bool, hipStream_t);
void launch_compact(const Dims&, const conf_cache&, int, int, const uint8_t*, int32_t*, int32_t*,
                    int32_t*, uint8_t*, hipStream_t);
void launch_evict(const Dims&, const conf_cache&, int, int, const int32_t*, uint8_t*, int32_t*,
                  int32_t*, int32_t*, uint8_t*, const float*, const int32_t*, const float*, bool,
                  hipStream_t);
void launch_arkv(const Dims&, const conf_cache&, int, int, const int32_t*, const int32_t*,
                 uint8_t*, int32_t*, int32_t*, int32_t*, uint8_t*, const float*, const int32_t*,
                 bool, hipStream_t);
void launch_set_retention(const Dims&, const conf_cache&, int, int, const float*, int, hipStream_t);
void launch_export(const Dims&, const conf_cache&, int, int8_t*, int8_t*, void*, void*, hipStream_t);
void launch_arkv_stats(const Dims&, int, int, int, const void*, const void*, float*, float*,
                       hipStream_t);
void launch_arkv_budgets(const Dims&, const float*, int32_t*, hipStream_t);
}  // namespace confkv

using namespace confkv;

namespace {

thread_local char g_err[512] = "";

int fail_hip(hipError_t e, const char* where) {
  snprintf(g_err, sizeof g_err, "%s: %s", where, hipGetErrorString(e));
  return CONF_E_HIP;
}

int check_launch(const char* where) {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? CONF_OK : fail_hip(e, where);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int make_dims(const conf_params* p, Dims* d) {
  if (!p || !d) return CONF_E_INVALID;
  if (p->n_layers <= 0 || p->batch <= 0 || p->n_q_heads <= 0 || p->n_kv_heads <= 0 ||
      p->vocab < 2)
    return CONF_E_INVALID;
  if (p->n_q_heads % p->n_kv_heads) return CONF_E_INVALID;
  if (p->head_dim != 64 && p->head_dim != 128) return CONF_E_UNSUPPORTED;
  if (p->dtype16 != CONF_F16 && p->dtype16 != CONF_BF16) return CONF_E_UNSUPPORTED;
  const int G = p->n_q_heads / p->n_kv_heads;
  if (G > kMaxGroup) return CONF_E_UNSUPPORTED;
  // the demotion spreads (K|V, KV head, channel) over 512 threads, eight each
  if (p->n_kv_heads * p->head_dim > 2048) return CONF_E_UNSUPPORTED;
  if (p->window < 1 || p->protect < 1 || p->protect > p->window) return CONF_E_INVALID;
  if (p->n_high < 1 || p->n_low < p->n_high) return CONF_E_INVALID;
  const int min_budget = layer_budget(p->n_high, p->n_layers - 1, p->n_layers, p->pyramid);
  if (p->protect > min_budget) return CONF_E_INVALID;
  if (p->cap8 < 64 || p->cap8 % 64) return CONF_E_INVALID;
  if (p->cap8 <= p->n_low) return CONF_E_CAPACITY;
  // a unit's INT8 region (cap8 * head_dim bytes) is addressed through a 32-bit
  // buffer range: keep it at or below 1 GiB
  if ((int64_t)p->cap8 * p->head_dim > ((int64_t)1 << 30)) return CONF_E_INVALID;
  if (!(p->ema_decay >= 0.f && p->ema_decay <= 1.f)) return CONF_E_INVALID;
  if (!(p->s_ema >= 0.f && p->s_rec >= 0.f)) return CONF_E_INVALID;
  if (p->pyramid != 0 && p->pyramid != 1) return CONF_E_INVALID;
  if (p->policy < CONF_POLICY_CONFKV || p->policy > CONF_POLICY_ARKV) return CONF_E_INVALID;
  if (p->headwise != 0 && p->headwise != 1) return CONF_E_INVALID;
  if (p->headwise) {
    // the baselines keep every head's tokens alike: head-wise sets are CONF-KV's
    if (p->policy != CONF_POLICY_CONFKV) return CONF_E_INVALID;
    // one head may hold every pair the others leave it
    if ((int64_t)p->cap8 <= (int64_t)p->n_kv_heads * p->n_low) return CONF_E_CAPACITY;
    if ((int64_t)p->batch * p->n_kv_heads > (1 << 30)) return CONF_E_INVALID;
  }
  d->L = p->n_layers;
  d->headwise = p->headwise;
  d->nseq = p->batch;
  d->hw = p->headwise ? p->n_kv_heads : 1;
  d->B = p->batch * d->hw;
  d->Hq = p->headwise ? G : p->n_q_heads;
  d->Hkv = p->headwise ? 1 : p->n_kv_heads;
  d->G = G;
  d->D = p->head_dim;
  d->V = p->vocab;
  d->W = p->window;
  d->P = p->protect;
  d->n_high = p->n_high;
  d->n_low = p->n_low;
  d->cap8 = p->cap8;
  d->cap16 = (p->window + 1 + kTile - 1) / kTile * kTile;
  d->capt = d->cap8 + d->cap16;
  d->bf16 = p->dtype16 == CONF_BF16;
  d->pyramid = p->pyramid;
  d->policy = p->policy;
  d->tau = p->tau;
  d->w_H = p->w_H;
  d->w_m = p->w_m;
  d->w_p = p->w_p;
  d->decay = p->ema_decay;
  d->one_minus_decay = 1.0f - p->ema_decay;
  d->s_ema = p->s_ema;
  d->s_rec = p->s_rec;
  return CONF_OK;
}

WsMap make_ws(const Dims& d) {
  WsMap w{};
  size_t off = 0;
  const size_t LB = (size_t)d.L * d.B;
  w.n_vchunks = conf_vchunks(d.V);
  w.conf_part = off;
  off = align256(off + (size_t)d.B * w.n_vchunks * 8 * sizeof(float));
  w.massp = off;
  off = align256(off + LB * d.Hkv * d.capt * sizeof(float));
  w.keep = off;
  off = align256(off + LB * d.capt);
  w.plan = off;
  off = align256(off + LB * 16 * sizeof(int32_t));
  w.mv8 = off;
  off = align256(off + LB * d.cap8 * sizeof(int32_t));
  w.mv16 = off;
  off = align256(off + LB * d.cap16 * sizeof(int32_t));
  w.wkeep = off;
  off = align256(off + LB * d.cap16);
  w.snap = off;
  off = align256(off + LB * 3 * sizeof(int32_t));
  const size_t spill = attn_spill_bytes(d);
  w.spill = spill ? off : 0;
  off = align256(off + spill);
  w.arkv_part = off;
  off = align256(off + (d.policy == CONF_POLICY_ARKV ? LB * d.Hkv * sizeof(float) : 0));
  w.total = off;
  return w;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

// The attention's score rows beyond LDS, or null where no cache can need them.
float* spill_rows(void* ws, const WsMap& w) { return w.spill ? at<float>(ws, w.spill) : nullptr; }

// The per-sequence dimensions (logits, confidence and budgets are per sequence
// also when the cache is kept per KV head).
Dims seq_dims(const Dims& d) {
  Dims s = d;
  s.B = d.nseq;
  return s;
}

// Rank + select (+ compaction) of a head-wise cache: the joint selection per
// (layer, sequence), with the pending EMA update first when with_ema, writes
// every head's keep flags to the workspace, then each head is compacted on its
// own.
void headwise_evict(const Dims& d, const conf_cache& c, int l0, int nl, const int32_t* budget,
                    void* ws, const WsMap& w, bool with_ema, hipStream_t st) {
  launch_joint_select(d, c, l0, nl, budget, at<uint8_t>(ws, w.keep), at<float>(ws, w.massp),
                      at<int32_t>(ws, w.snap), with_ema, st);
  launch_compact(d, c, l0, nl, at<uint8_t>(ws, w.keep), at<int32_t>(ws, w.plan),
                 at<int32_t>(ws, w.mv8), at<int32_t>(ws, w.mv16), at<uint8_t>(ws, w.wkeep), st);
}

// non-null and 16-byte aligned (the kernels read these with 16-byte loads)
bool a16(const void* x) { return x && ((uintptr_t)x & 15u) == 0; }

bool cache_ok(const conf_cache* c) {
  return c && a16(c->k8) && a16(c->v8) && a16(c->k16) && a16(c->v16) && a16(c->k_amax) &&
         a16(c->v_amax) && c->pos8 && c->ema8 && c->pos16 && c->ema16 && c->n8 && c->n16 && c->t &&
         c->status;
}

// layer selector -> (first layer, layer count)
bool layer_range(const Dims& d, int32_t layer, int* l0, int* nl) {
  if (layer == -1) {
    *l0 = 0;
    *nl = d.L;
    return true;
  }
  if (layer < 0 || layer >= d.L) return false;
  *l0 = layer;
  *nl = 1;
  return true;
}

}  // namespace

extern "C" {

int conf_cache_layout(const conf_params* p, conf_cache_bytes_t* o) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  if (!o) return CONF_E_INVALID;
  const size_t U = (size_t)d.L * d.B * d.Hkv, LB = (size_t)d.L * d.B;
  o->k8 = U * d.cap8 * d.D;
  o->v8 = o->k8;
  o->k16 = U * d.cap16 * d.D * 2;
  o->v16 = o->k16;
  o->k_amax = U * d.D * sizeof(float);
  o->v_amax = o->k_amax;
  o->pos8 = LB * d.cap8 * sizeof(int32_t);
  o->ema8 = LB * d.cap8 * sizeof(float);
  o->pos16 = LB * d.cap16 * sizeof(int32_t);
  o->ema16 = LB * d.cap16 * sizeof(float);
  o->n8 = LB * sizeof(int32_t);
  o->n16 = o->n8;
  o->t = o->n8;
  o->status = sizeof(int32_t);
  o->cap16 = d.cap16;
  return CONF_OK;
}

int conf_workspace_bytes(const conf_params* p, size_t* bytes) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  if (!bytes) return CONF_E_INVALID;
  *bytes = make_ws(d).total;
  return CONF_OK;
}

int conf_cache_reset(const conf_params* p, conf_cache* c, conf_stream_t stream) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  if (!cache_ok(c)) return CONF_E_INVALID;
  launch_reset(d, *c, (hipStream_t)stream);
  return check_launch("conf_cache_reset");
}

int conf_cache_ingest(const conf_params* p, conf_cache* c, int32_t layer, const void* k_pre,
                      const void* v_pre, int32_t prefill_len, void* ws, conf_stream_t stream) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  int l0, nl;
  if (!cache_ok(c) || !k_pre || !v_pre || prefill_len < 0 || !layer_range(d, layer, &l0, &nl))
    return CONF_E_INVALID;
  (void)ws;
  if (d.policy != CONF_POLICY_WINDOW && prefill_len - d.W > d.cap8) return CONF_E_CAPACITY;
  if ((d.policy == CONF_POLICY_FULL || d.policy == CONF_POLICY_TRIM) && prefill_len > d.W)
    return CONF_E_CAPACITY;
  if (prefill_len == 0) return CONF_OK;
  launch_ingest(d, *c, l0, nl, prefill_len, k_pre, v_pre, (hipStream_t)stream);
  return check_launch("conf_cache_ingest");
}

int conf_confidence(const conf_params* p, const float* logits, float* c, int32_t* budget, void* ws,
                    conf_stream_t stream) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  if (!logits || !c || !budget || !ws) return CONF_E_INVALID;
  const WsMap w = make_ws(d);
  launch_confidence(seq_dims(d), logits, at<float>(ws, w.conf_part), c, budget,
                    (hipStream_t)stream);
  return check_launch("conf_confidence");
}

static int decode_attn(const conf_params* p, conf_cache* c, int32_t layer, const void* q,
                       const void* k_new, const void* v_new, float* out, void* ws,
                       conf_stream_t stream, bool with_ema, const char* name) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  int l0, nl;
  if (!cache_ok(c) || !a16(q) || !a16(k_new) || !a16(v_new) || !out || !ws ||
      !layer_range(d, layer, &l0, &nl))
    return CONF_E_INVALID;
  const WsMap w = make_ws(d);
  launch_attn(d, *c, l0, nl, q, k_new, v_new, out, at<float>(ws, w.massp), at<int32_t>(ws, w.snap),
              spill_rows(ws, w), with_ema, (hipStream_t)stream);
  return check_launch(name);
}

int conf_decode_attn(const conf_params* p, conf_cache* c, int32_t layer, const void* q,
                     const void* k_new, const void* v_new, float* out, void* ws,
                     conf_stream_t stream) {
  // retention eviction keeps no EMA: its step is conf_attend + conf_trim_evict_compact
  if (p && p->policy == CONF_POLICY_TRIM) return CONF_E_INVALID;
  return decode_attn(p, c, layer, q, k_new, v_new, out, ws, stream, true, "conf_decode_attn");
}

int conf_attend(const conf_params* p, conf_cache* c, int32_t layer, const void* q,
                const void* k_new, const void* v_new, float* out, void* ws, conf_stream_t stream) {
  return decode_attn(p, c, layer, q, k_new, v_new, out, ws, stream, false, "conf_attend");
}

int conf_rank_evict(const conf_params* p, conf_cache* c, int32_t layer, const int32_t* budget,
                    uint8_t* keep, void* ws, conf_stream_t stream) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  int l0, nl;
  if (!cache_ok(c) || !budget || !keep || !layer_range(d, layer, &l0, &nl)) return CONF_E_INVALID;
  (void)ws;
  if (d.headwise)
    launch_joint_select(d, *c, l0, nl, budget, keep, nullptr, nullptr, false,
                        (hipStream_t)stream);
  else
    launch_select(d, *c, l0, nl, budget, keep, (hipStream_t)stream);
  return check_launch("conf_rank_evict");
}

int conf_compact_demote(const conf_params* p, conf_cache* c, int32_t layer, const uint8_t* keep,
                        void* ws, conf_stream_t stream) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  int l0, nl;
  if (!cache_ok(c) || !keep || !ws || !layer_range(d, layer, &l0, &nl)) return CONF_E_INVALID;
  if (d.policy == CONF_POLICY_ARKV) return CONF_E_INVALID;  // ARKV demotes by rank, not position
  const WsMap w = make_ws(d);
  launch_compact(d, *c, l0, nl, keep, at<int32_t>(ws, w.plan), at<int32_t>(ws, w.mv8),
                 at<int32_t>(ws, w.mv16), at<uint8_t>(ws, w.wkeep), (hipStream_t)stream);
  return check_launch("conf_compact_demote");
}

static int evict(const conf_params* p, conf_cache* c, int32_t layer, const int32_t* budget,
                 const float* log_beta, void* ws, conf_stream_t stream, bool with_ema,
                 const char* name) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  int l0, nl;
  if (!cache_ok(c) || !budget || !ws || !layer_range(d, layer, &l0, &nl)) return CONF_E_INVALID;
  // the retention policy's appended token needs its ln(beta); nothing else takes one
  if (with_ema && (d.policy == CONF_POLICY_TRIM) != (log_beta != nullptr)) return CONF_E_INVALID;
  if (d.policy == CONF_POLICY_ARKV) return CONF_E_INVALID;  // conf_arkv_evict_compact
  const WsMap w = make_ws(d);
  if (d.headwise) {
    headwise_evict(d, *c, l0, nl, budget, ws, w, with_ema, (hipStream_t)stream);
    return check_launch(name);
  }
  launch_evict(d, *c, l0, nl, budget, at<uint8_t>(ws, w.keep), at<int32_t>(ws, w.plan),
               at<int32_t>(ws, w.mv8), at<int32_t>(ws, w.mv16), at<uint8_t>(ws, w.wkeep),
               at<float>(ws, w.massp), at<int32_t>(ws, w.snap), log_beta, with_ema,
               (hipStream_t)stream);
  return check_launch(name);
}

int conf_evict_compact(const conf_params* p, conf_cache* c, int32_t layer, const int32_t* budget,
                       void* ws, conf_stream_t stream) {
  return evict(p, c, layer, budget, nullptr, ws, stream, false, "conf_evict_compact");
}

int conf_ema_evict_compact(const conf_params* p, conf_cache* c, int32_t layer,
                           const int32_t* budget, void* ws, conf_stream_t stream) {
  return evict(p, c, layer, budget, nullptr, ws, stream, true, "conf_ema_evict_compact");
}

int conf_trim_evict_compact(const conf_params* p, conf_cache* c, int32_t layer,
                            const int32_t* budget, const float* log_beta, void* ws,
                            conf_stream_t stream) {
  if (!log_beta) return CONF_E_INVALID;
  return evict(p, c, layer, budget, log_beta, ws, stream, true, "conf_trim_evict_compact");
}

static int arkv(const conf_params* p, conf_cache* c, int32_t layer, const int32_t* budget,
                const int32_t* n_orig, void* ws, conf_stream_t stream, bool with_ema,
                const char* name) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  int l0, nl;
  if (!cache_ok(c) || !budget || !n_orig || !ws || d.policy != CONF_POLICY_ARKV ||
      !layer_range(d, layer, &l0, &nl))
    return CONF_E_INVALID;
  const WsMap w = make_ws(d);
  launch_arkv(d, *c, l0, nl, budget, n_orig, at<uint8_t>(ws, w.keep), at<int32_t>(ws, w.plan),
              at<int32_t>(ws, w.mv8), at<int32_t>(ws, w.mv16), at<uint8_t>(ws, w.wkeep),
              at<float>(ws, w.massp), at<int32_t>(ws, w.snap), with_ema, (hipStream_t)stream);
  return check_launch(name);
}

int conf_arkv_evict_compact(const conf_params* p, conf_cache* c, int32_t layer,
                            const int32_t* budget, const int32_t* n_orig, void* ws,
                            conf_stream_t stream) {
  return arkv(p, c, layer, budget, n_orig, ws, stream, false, "conf_arkv_evict_compact");
}

int conf_arkv_ema_evict_compact(const conf_params* p, conf_cache* c, int32_t layer,
                                const int32_t* budget, const int32_t* n_orig, void* ws,
                                conf_stream_t stream) {
  return arkv(p, c, layer, budget, n_orig, ws, stream, true, "conf_arkv_ema_evict_compact");
}

int conf_cache_set_retention(const conf_params* p, conf_cache* c, int32_t layer,
                             const float* log_beta, int32_t prefill_len, conf_stream_t stream) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  int l0, nl;
  if (!cache_ok(c) || !log_beta || prefill_len < 0 || prefill_len > d.W ||
      d.policy != CONF_POLICY_TRIM || !layer_range(d, layer, &l0, &nl))
    return CONF_E_INVALID;
  if (prefill_len == 0) return CONF_OK;
  launch_set_retention(d, *c, l0, nl, log_beta, prefill_len, (hipStream_t)stream);
  return check_launch("conf_cache_set_retention");
}

}  // extern "C"

// ---------------------------------------------------------------- conf_step_static
// The workspace of conf_step_static: a device array of the library's own, one copy
// per GPU, held until the process ends.  Host code never passes `scratch` itself to
// a kernel (on the host it is only a stand-in for the symbol); it uses the device
// address that hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kStaticScratchBytes = CONF_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (set up on the first call per device).
int static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "conf_step_static: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(g_err, sizeof g_err, "conf_step_static: device %d beyond the %d supported", dev,
             kMaxDevices);
    return CONF_E_UNSUPPORTED;
  }
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return fail_hip(e, "conf_step_static: hipGetSymbolAddress");
      if (!ptr) {
        snprintf(g_err, sizeof g_err, "conf_step_static: no device address for the scratch array");
        return CONF_E_HIP;
      }
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return CONF_OK;
}
}  // namespace

extern "C" {

int conf_step_static(const conf_params* p, conf_cache* c, const float* logits, const void* q,
                     const void* k_new, const void* v_new, float* out, float* conf,
                     int32_t* budget, conf_stream_t stream) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  const size_t need = make_ws(d).total;
  if (need > kStaticScratchBytes) {  // before any device call
    snprintf(g_err, sizeof g_err,
             "conf_step_static: this shape needs %zu bytes of workspace; the static scratch holds "
             "%zu (use conf_step with a workspace of conf_workspace_bytes())",
             need, kStaticScratchBytes);
    return CONF_E_CAPACITY;
  }
  void* ws = nullptr;
  rc = static_scratch(&ws);
  if (rc) return rc;
  return conf_step(p, c, logits, q, k_new, v_new, out, conf, budget, ws, stream);
}

int conf_step(const conf_params* p, conf_cache* c, const float* logits, const void* q,
              const void* k_new, const void* v_new, float* out, float* conf, int32_t* budget,
              void* ws, conf_stream_t stream) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  if (!cache_ok(c) || !logits || !a16(q) || !a16(k_new) || !a16(v_new) || !out || !conf ||
      !budget || !ws || d.policy == CONF_POLICY_TRIM || d.policy == CONF_POLICY_ARKV)
    return CONF_E_INVALID;
  const WsMap w = make_ws(d);
  hipStream_t st = (hipStream_t)stream;
  if (d.headwise) {
    launch_attn(d, *c, 0, d.L, q, k_new, v_new, out, at<float>(ws, w.massp),
                at<int32_t>(ws, w.snap), spill_rows(ws, w), true, st);
    launch_confidence(seq_dims(d), logits, at<float>(ws, w.conf_part), conf, budget, st);
    headwise_evict(d, *c, 0, d.L, budget, ws, w, false, st);
    return check_launch("conf_step");
  }
  launch_attn(d, *c, 0, d.L, q, k_new, v_new, out, at<float>(ws, w.massp), at<int32_t>(ws, w.snap),
              spill_rows(ws, w), false, st);
  launch_confidence(d, logits, at<float>(ws, w.conf_part), conf, budget, st);
  launch_evict(d, *c, 0, d.L, budget, at<uint8_t>(ws, w.keep), at<int32_t>(ws, w.plan),
               at<int32_t>(ws, w.mv8), at<int32_t>(ws, w.mv16), at<uint8_t>(ws, w.wkeep),
               at<float>(ws, w.massp), at<int32_t>(ws, w.snap), nullptr, true, st);
  return check_launch("conf_step");
}

int conf_arkv_prefill_stats(const conf_params* p, int32_t layer, const void* q,
                            const void* k_pre, int32_t prefill_len, float* conc, void* ws,
                            conf_stream_t stream) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  int l0, nl;
  if (d.policy != CONF_POLICY_ARKV || !a16(q) || !a16(k_pre) || !conc || !ws ||
      prefill_len < 2 || !layer_range(d, layer, &l0, &nl))
    return CONF_E_INVALID;
  const WsMap w = make_ws(d);
  launch_arkv_stats(d, l0, nl, prefill_len, q, k_pre, at<float>(ws, w.arkv_part), conc,
                    (hipStream_t)stream);
  return check_launch("conf_arkv_prefill_stats");
}

int conf_arkv_orig_budgets(const conf_params* p, const float* conc, int32_t* n_orig,
                           conf_stream_t stream) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  if (d.policy != CONF_POLICY_ARKV || !conc || !n_orig) return CONF_E_INVALID;
  launch_arkv_budgets(d, conc, n_orig, (hipStream_t)stream);
  return check_launch("conf_arkv_orig_budgets");
}

int conf_cache_export(const conf_params* p, const conf_cache* c, int32_t layer, int32_t seq,
                      int8_t* k8, int8_t* v8, void* k16, void* v16, conf_stream_t stream) {
  Dims d;
  int rc = make_dims(p, &d);
  if (rc) return rc;
  if (!cache_ok(c) || !k8 || !v8 || !k16 || !v16 || layer < 0 || layer >= d.L || seq < 0 ||
      seq >= d.B)
    return CONF_E_INVALID;
  launch_export(d, *c, layer * d.B + seq, k8, v8, k16, v16, (hipStream_t)stream);
  return check_launch("conf_cache_export");
}

const char* conf_last_error(void) { return g_err; }

const char* conf_status_string(int status) {
  switch (status) {
    case CONF_OK: return "ok";
    case CONF_E_INVALID: return "invalid argument";
    case CONF_E_UNSUPPORTED: return "unsupported shape or dtype";
    case CONF_E_CAPACITY: return "capacity too small";
    case CONF_E_HIP: return "HIP error";
    default: return "unknown status";
  }
}

}  // extern "C"
