/*
 * confkv.h - C ABI of the MI355X (gfx950) CONF-KV decode-step library.
 *
 * CONF-KV keeps a budgeted, dense, mixed-precision KV cache and changes the
 * budget at every decode step from the model's confidence in its next token.
 * Citations name sections of the CONF-KV explainer pages (gist.science
 * technical summary of "CONF-KV: Confidence-Aware KV Cache Eviction with
 * Mixed-Precision Storage for Long-Horizon LLM"; the Dutch, Italian and Korean
 * renderings agree):
 *   [confidence]  Methodology, confidence estimation
 *   [budget]      Methodology, adaptive budget selection
 *   [ranking]     Methodology, token ranking and eviction
 *   [storage]     Methodology, system integration, mixed-precision storage
 *   [pyramid]     Methodology, system integration, pyramidal budgets (CONF-KV-L)
 *   [impl]        Methodology, system integration, implementation
 *   [online]      Key contributions, system design (block-wise online softmax)
 *   [problem]     Problem statement (sliding-window eviction as a prior policy)
 *   [results]     Experimental results (full-KV latency and throughput comparison)
 *   [trim]        the TRIM-KV page, Methodology: retention gate; inference and
 *                 eviction (a related method in the same bundle)
 *   [heads]       Significance and claims (the method composes with head-wise
 *                 allocation)
 *   [arkv]        the ARKV page, Methodology: three-state assignment;
 *                 decoding-phase token ranking (a related method in the bundle)
 *   [arkv-prefill] the ARKV page, Methodology: 1. prefill phase (layer-wise
 *                 budget assignment from entropy, variance and kurtosis)
 *
 * Conventions shared by every call
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except
 *     the `const conf_params*` / `conf_cache*` structs themselves, which are
 *     host memory read during the call only.  The library allocates no device
 *     memory; scratch lives in the caller's workspace `ws` of
 *     conf_workspace_bytes() bytes (256-byte aligned).  Its process-wide
 *     state: one flag per (device, attention kernel variant) recording that
 *     the kernel's dynamic-LDS limit has been raised (an idempotent, thread-
 *     safe one-time set-up; nothing that holds data), and, for
 *     conf_step_static only, that call's fixed scratch array on each GPU and
 *     its looked-up device address (see conf_step_static).
 *   - A call validates its arguments on the host, enqueues kernels on `stream`
 *     (a hipStream_t; NULL is the null stream) and returns without waiting for
 *     the device.  Results are valid once the stream has been synchronised.
 *   - q, k_new, v_new and the cache's k8, v8, k16, v16, k_amax, v_amax must be
 *     16-byte aligned (CONF_E_INVALID otherwise); PyTorch allocations are.
 *   - Return value: CONF_OK (0) or a negative CONF_E_* code; nothing is
 *     enqueued when validation fails.  No C++ exception crosses the ABI.
 *   - `layer` = -1 processes every layer in one launch per kernel; then per-
 *     layer tensors carry a leading [L] dimension.  `layer` = l >= 0 processes
 *     layer l only; then q/k_new/v_new/out/k_pre/v_pre have no [L] dimension.
 *     `budget` and `keep` always cover every layer.
 *   - Calls on the same cache must not overlap (use one stream per cache).
 *   - Data-dependent sizes (tokens per layer and sequence) stay on the device;
 *     no call reads them back, so a step can be captured in a HIP graph.
 */
#ifndef CONFKV_H
#define CONFKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* conf_stream_t; /* hipStream_t */

enum {
  CONF_OK = 0,
  CONF_E_INVALID = -1,     /* null pointer, inconsistent sizes, P > W, P > budget, ... */
  CONF_E_UNSUPPORTED = -2, /* head_dim not 64/128, group > 16, n_kv_heads * head_dim > 2048,
                              unknown dtype */
  CONF_E_CAPACITY = -3,    /* cap8 too small for the budgets or the prefill */
  CONF_E_HIP = -4          /* a HIP launch failed; see conf_last_error() */
};

enum { CONF_F16 = 1, CONF_BF16 = 2 };

/* Cache policy (conf_params.policy).  CONF-KV itself, and two baselines that the
 * pages compare it with, run on the same kernels and layout:
 *   CONF_POLICY_CONFKV  the method: confidence-chosen budgets, EMA ranking,
 *                       INT8 demotion of tokens older than the window.
 *   CONF_POLICY_FULL    full KV [results]: every token stays, in 16 bits.  The
 *                       window W must hold the prefill and every decoded token
 *                       (conf_cache_ingest returns CONF_E_CAPACITY for a longer
 *                       prefill; an append that finds it full sets
 *                       CONF_ST_WINDOW_FULL).  Budgets do not evict, nothing is
 *                       demoted.
 *   CONF_POLICY_WINDOW  sliding window [problem]: after each step only positions
 *                       (t-W, t] stay, in 16 bits; older prefill tokens leave at
 *                       the first step.  Budgets and ranking play no part.
 *   CONF_POLICY_TRIM    retention eviction [trim]: each token carries ln(beta),
 *                       beta in [0, 1], fixed at its creation and supplied by the
 *                       caller; its current score is (t - pos) * ln(beta), the
 *                       logarithm of beta^(t - pos) (0 for the newest token),
 *                       one float32 product.  After each step the budget's best
 *                       tokens stay (ties: newer first), all in 16 bits; nothing
 *                       is demoted and only the newest token is protected.  The
 *                       ema arrays hold ln(beta).  A step is conf_attend, then
 *                       conf_trim_evict_compact; the prefill's ln(beta) is set
 *                       by conf_cache_set_retention after conf_cache_ingest.
 *   CONF_POLICY_ARKV    ARKV's three-state cache [arkv]: Original tokens in 16
 *                       bits (the window arrays), Quantized ones as e4m3 codes
 *                       (the 8-bit arrays: sign, 4 exponent bits with bias 7, 3
 *                       mantissa bits, largest 448; scale = absmax / 448 per (KV
 *                       head, channel), round to nearest even, requantised on a
 *                       new maximum), Evicted ones gone.  The ema arrays hold the
 *                       EMA of the heavy-hitter score mean_k m_k + var_k m_k over
 *                       the KV heads k (m_k: the token's attention averaged over
 *                       head k's query heads; population variance).  A step is
 *                       conf_attend, then conf_arkv_ema_evict_compact; W only sizes
 *                       the 16-bit arrays (at least the largest N_O), and the
 *                       prefill's positions < prefill_len - W are Quantized.
 * The baselines and TRIM need no per-token attention mass: their attention is a
 * single online pass whatever the cache length, and they keep no EMA (it stays
 * 0 for FULL and WINDOW). */
enum { CONF_POLICY_CONFKV = 0, CONF_POLICY_FULL = 1, CONF_POLICY_WINDOW = 2,
       CONF_POLICY_TRIM = 3, CONF_POLICY_ARKV = 4 };

/* Device status word bits (conf_cache.status), set by kernels, never cleared
 * except by conf_cache_reset().  CONF_ST_INT8_FULL cannot arise with parameters
 * the library accepts (cap8 > n_low >= n_high bounds the INT8 part, and eviction
 * runs before demotion); it guards a cache whose counters were changed outside
 * the library. */
enum {
  CONF_ST_WINDOW_FULL = 1, /* append found the 16-bit window full: token dropped */
  CONF_ST_INT8_FULL = 2    /* a demotion found the INT8 region full: token dropped */
};

typedef struct conf_params {
  int32_t n_layers, batch, n_q_heads, n_kv_heads, head_dim, vocab;
  int32_t dtype16;          /* CONF_F16 | CONF_BF16: q, k_new, v_new, k_pre, v_pre, window */
  int32_t window;           /* W: positions (t-W, t] stay 16-bit [storage] */
  int32_t protect;          /* P: positions (t-P, t] are never evicted [ranking]; P <= W */
  int32_t n_high, n_low;    /* budgets for c >= tau and c < tau [budget]; P <= n_high <= n_low */
  int32_t cap8;             /* INT8 slots per (layer, sequence): multiple of 64, > n_low,
                               cap8 * head_dim <= 2^30 */
  int32_t pyramid;          /* 1: N_l = floor(N (2(L-1)-l) / (2(L-1))) [pyramid]; 0: N_l = N */
  float tau;                /* confidence threshold [budget] */
  float w_H, w_m, w_p;      /* confidence weights; the pages use 0.4, 0.3, 0.3 [confidence] */
  float ema_decay;          /* e <- decay*e + (1-decay)*mass [ranking] */
  float s_ema, s_rec;       /* score = s_ema*(e/e_max) + s_rec*(pos/t) [ranking] */
  int32_t policy;           /* CONF_POLICY_*; 0 is CONF-KV */
  int32_t headwise;         /* 1: head-wise keep sets (CONF_POLICY_CONFKV only), below */
} conf_params;

/*
 * Head-wise keep sets [heads] (conf_params.headwise = 1).  Each KV head h of
 * sequence b is a cache of its own, sub-sequence s = b*Hkv + h, with its own
 * tokens, window and INT8 split:
 *   - pos8, ema8, pos16, ema16, n8, n16 and t are [L][B*Hkv][...] in place of
 *     [L][B][...]; conf_cache_layout() reports those sizes; conf_cache_export's
 *     `seq` is s and its outputs have one KV head;
 *   - q, k_new, v_new, out, k_pre, v_pre, logits, c and budget keep their shapes;
 *   - a token's mass in head h is the mean over h's Hq/Hkv query heads;
 *   - the selection of (layer l, sequence b) spends Hkv * budget[b][l]
 *     (token, head) pairs jointly: each head's positions (t-P, t] stay, the
 *     other pairs are ranked by the composite score with e_max over every head
 *     of the layer, ties by position desc, then head desc; each head then
 *     demotes its own position t-W;
 *   - the steps that apply the EMA and select run as separate launches (EMA,
 *     joint selection, per-head compaction).
 * CONF_E_CAPACITY unless cap8 > Hkv * n_low (one head may hold all the pairs
 * the others leave it).  Positions must stay below 2^32 / Hkv.
 */

/*
 * The dense mixed-precision cache [storage][impl].  All arrays are caller-
 * allocated device memory of the sizes conf_cache_layout() reports.  With
 * cap16 = W+1 rounded up to 64 and U = L*B*Hkv units:
 *   k8     int8  [L][B][Hkv][cap8/64][64*d]       INT8 key codes, 64-token tiles
 *   v8     int8  [L][B][Hkv][cap8/64][64*d]       INT8 value codes, 64-token tiles
 *   k16    16-bit[L][B][Hkv][cap16/64][64*d]      window keys, 64-token tiles
 *   v16    16-bit[L][B][Hkv][cap16/64][64*d]      window values, 64-token tiles
 *   k_amax, v_amax fp32 [L][B][Hkv][d]            running absmax; scale = amax/127
 *   pos8, ema8     [L][B][cap8]  int32 / fp32     position and EMA of INT8 slots
 *   pos16, ema16   [L][B][cap16] int32 / fp32     position and EMA of window slots
 *   n8, n16        int32 [L][B]                   occupied slots (dense prefix)
 *   t              int32 [L][B]                   newest position (-1 = empty)
 *   status         int32 [1]                      CONF_ST_* bits
 * Inside a tile, write a slot's index j (mod 64) as j = 32u + 16a + 4g + b =
 * 16r + row (u, a in {0,1}; g, b, r in 0..3; row in 0..15) and a channel c.
 * The element order of a tile is
 *   k8:  [r][c/64][(c/16)%4][row][c%16]         v8:  [g][c][8u + 4a + b]
 *   k16: [u][r%2][c/32][(c/8)%4][row][c%8]      v16: [u][g][c][4a + b]
 * so that every wavefront load of the attention kernel reads whole cache lines
 * (keys: one 1 KB run; values: four 256-byte pieces) and lands in the lane that
 * feeds it to the matrix cores, while one token's values stay inside a 16*d-byte
 * stretch of the tile.
 * conf_cache_export() returns plain row-major copies.
 * Slot order inside a region is arbitrary: compaction fills holes, so a token's
 * identity is its stored position.
 */
typedef struct conf_cache {
  int8_t* k8;
  int8_t* v8;
  void* k16;
  void* v16;
  float* k_amax;
  float* v_amax;
  int32_t* pos8;
  float* ema8;
  int32_t* pos16;
  float* ema16;
  int32_t* n8;
  int32_t* n16;
  int32_t* t;
  int32_t* status;
} conf_cache;

typedef struct conf_cache_bytes_t {
  size_t k8, v8, k16, v16, k_amax, v_amax, pos8, ema8, pos16, ema16, n8, n16, t, status;
  int32_t cap16;
} conf_cache_bytes_t;

/* Byte size of every cache array for `p`.  Returns CONF_E_* if p is invalid. */
int conf_cache_layout(const conf_params* p, conf_cache_bytes_t* out);

/* Workspace bytes every call below may use for `p`. */
int conf_workspace_bytes(const conf_params* p, size_t* bytes);

/* Empty every (layer, sequence): n8 = n16 = 0, t = -1, absmax = 0, status = 0,
 * and every element of k16 and v16 = 0.  The attention reads whole 32-token
 * window halves and gives the free slots past n16 probability 0, which cancels
 * only a finite value (0 * NaN is NaN), so the window's free slots must hold
 * finite bits: the reset establishes that, and the library keeps it as long as
 * k_new, v_new, k_pre and v_pre are finite.  Fills with kernels (no memset
 * nodes), so it may be graph-captured. */
int conf_cache_reset(const conf_params* p, conf_cache* c, conf_stream_t stream);

/*
 * Load a prefilled context of `prefill_len` tokens, positions 0..prefill_len-1.
 * k_pre, v_pre: 16-bit [L][B][Hkv][prefill_len][d] (layer = -1) or
 * [B][Hkv][prefill_len][d] (layer = l).  Positions < prefill_len - W become
 * INT8 with absmax over exactly those tokens (CONF_POLICY_WINDOW drops them
 * instead); the rest fill the window; every EMA is 0 and t = prefill_len - 1
 * [storage].  The layer must be empty.  CONF_E_CAPACITY if prefill_len - W >
 * cap8 (CONF-KV), or prefill_len > W (CONF_POLICY_FULL, CONF_POLICY_TRIM).
 */
int conf_cache_ingest(const conf_params* p, conf_cache* c, int32_t layer, const void* k_pre,
                      const void* v_pre, int32_t prefill_len, void* ws, conf_stream_t stream);

/*
 * (a) Confidence and budget [confidence][budget][pyramid].
 * logits: fp32 [B][vocab], row-contiguous.  Per sequence:
 *   p = softmax(z), H^ = -sum p ln p / ln V, m = z(1) - z(2) (top two logits,
 *   duplicates counted), p1 = max p, c = w_H (1-H^) + w_m / (1+e^-m) + w_p p1.
 * c: fp32 [B] (NaN when any logit is non-finite).  budget: int32 [B][L],
 * budget[b][l] = layer budget of (c >= tau ? n_high : n_low).
 */
int conf_confidence(const conf_params* p, const float* logits, float* c, int32_t* budget,
                    void* ws, conf_stream_t stream);

/*
 * (b)+(c) Append, decode attention and EMA update [online][impl][ranking].
 * Appends this step's key/value (k_new, v_new: 16-bit [L][B][Hkv][d]) at
 * position t+1 in the window, then for every query head h (q: 16-bit
 * [L][B][Hq][d]) computes o_h = sum_j softmax_j(q_h . k_j / sqrt(d)) v_j over all
 * cached tokens of KV head h / (Hq/Hkv), INT8 tokens dequantised as code*amax/127
 * inside the block reads.  out: fp32 [L][B][Hq][d].  Then every token's EMA
 * becomes decay*e + (1-decay)*mass_j, mass_j = mean over the Hq heads of its
 * softmax probability; the new token starts from e = 0.  K and V are read once
 * whatever the cache length: the raw scores wait for the final softmax
 * normaliser in LDS, and those of a cache longer than the LDS rows in ws (at
 * d = 128 with a window of at most 512 tokens, its window's in registers, so
 * that only INT8 tokens past the rows go to ws).
 * Under CONF_POLICY_ARKV
 * the EMA is that of ARKV's heavy-hitter score (see the policy).
 * CONF_E_INVALID under CONF_POLICY_TRIM, whose step is conf_attend followed by
 * conf_trim_evict_compact.  Policy limits of the calls below: conf_step and
 * conf_ema_evict_compact return CONF_E_INVALID under CONF_POLICY_TRIM and
 * CONF_POLICY_ARKV; conf_evict_compact and conf_compact_demote under
 * CONF_POLICY_ARKV, which demotes by rank, not by position (its calls are
 * conf_arkv_*).
 */
int conf_decode_attn(const conf_params* p, conf_cache* c, int32_t layer, const void* q,
                     const void* k_new, const void* v_new, float* out, void* ws,
                     conf_stream_t stream);

/*
 * (b) alone: conf_decode_attn without its EMA update.  The new row is stored in
 * the window and `out` is written, but each token's attention mass stays in ws
 * and n16 and t do not advance yet: conf_ema_evict_compact (under
 * CONF_POLICY_TRIM, conf_trim_evict_compact) on the same layer selector and ws
 * must follow before any other call touches those layers.
 * Together the two calls give exactly the results of conf_decode_attn followed
 * by conf_evict_compact, with one launch fewer.
 */
int conf_attend(const conf_params* p, conf_cache* c, int32_t layer, const void* q,
                const void* k_new, const void* v_new, float* out, void* ws, conf_stream_t stream);

/*
 * (d) Rank and select [ranking].  budget: int32 [B][L] (conf_confidence).
 * keep: uint8 [L][B][cap8 + cap16]; entry i < cap8 flags INT8 slot i, entry
 * cap8 + w flags window slot w; only occupied slots are written.  If a
 * (layer, sequence) holds n <= N tokens every slot is kept (no-op).  Otherwise
 * keep the positions (t-P, t] and the N - |protected| best other tokens in the
 * order (score desc, position desc), score = s_ema*(e/e_max) + s_rec*(pos/t),
 * evaluated in fp32 one rounding per operation (e/e_max = 0 if e_max = 0;
 * pos/t = 1 if t = 0).  Under the other policies the policy's own rule decides
 * (see the policies above): full KV keeps every token, the sliding window the
 * positions (t-W, t], retention eviction ranks by (t - pos) * ln(beta), ARKV by
 * its score EMA.
 * Head-wise, the keep flags are those of the joint selection over the heads of
 * each (layer, sequence), keep [L][B*Hkv][cap8 + cap16].
 */
int conf_rank_evict(const conf_params* p, conf_cache* c, int32_t layer, const int32_t* budget,
                    uint8_t* keep, void* ws, conf_stream_t stream);

/*
 * (e) Compact and demote [impl][storage].  Drops the tokens whose keep flag is
 * 0 by moving survivors from the tail of each region into its holes (the layout
 * stays dense with no indirection table), then moves the token at position
 * t - W, if it survived, from the window to INT8: per (KV head, channel)
 * a = |x|; if a > absmax the channel's stored codes become
 * clamp(rne((code*s_old)/s_new)) and absmax = a; then code = clamp(rne(x/s)),
 * s = absmax/127 (s = 0 gives code 0).  Full KV and retention eviction demote
 * nothing; under ARKV (which demotes by rank) the call returns CONF_E_INVALID.
 */
int conf_compact_demote(const conf_params* p, conf_cache* c, int32_t layer, const uint8_t* keep,
                        void* ws, conf_stream_t stream);

/*
 * (d)+(e) in one launch [ranking][impl][storage]: the same result as
 * conf_rank_evict followed by conf_compact_demote on the same layer selector,
 * without a keep array (the flags stay on chip; those of caches larger than the
 * on-chip flag cache go to ws).  budget: int32 [B][L].
 */
int conf_evict_compact(const conf_params* p, conf_cache* c, int32_t layer, const int32_t* budget,
                       void* ws, conf_stream_t stream);

/*
 * (c)+(d)+(e) in one launch, after conf_attend: the pending EMA update (as in
 * conf_decode_attn), then conf_evict_compact.  budget: int32 [B][L].
 */
int conf_ema_evict_compact(const conf_params* p, conf_cache* c, int32_t layer,
                           const int32_t* budget, void* ws, conf_stream_t stream);

/*
 * Retention eviction after conf_attend (CONF_POLICY_TRIM only) [trim]: this
 * step's token takes log_beta (fp32 [L][B] for layer = -1, [B] otherwise; each
 * <= 0, -INFINITY for beta = 0, no NaN), n16 and t advance, and each (layer,
 * sequence) keeps its budget[b][l] best tokens by (t - pos) * ln(beta), then
 * compacts.  CONF_E_INVALID under any other policy.
 */
int conf_trim_evict_compact(const conf_params* p, conf_cache* c, int32_t layer,
                            const int32_t* budget, const float* log_beta, void* ws,
                            conf_stream_t stream);

/*
 * ARKV's eviction and quantisation (CONF_POLICY_ARKV only) [arkv], after
 * conf_decode_attn (which applied the heavy-hitter score EMA, the new token's
 * from 0): each (layer, sequence) keeps its newest P positions and its
 * budget[b][l] - |P| best other tokens by (EMA desc, position desc); then, while
 * more than n_orig[b][l] kept tokens are Original, the lowest-ranked unprotected
 * Original token is quantised to e4m3 (lowest first; one per step in the steady
 * state).  budget, n_orig: int32 [B][L].  CONF_E_INVALID under any other policy.
 */
int conf_arkv_evict_compact(const conf_params* p, conf_cache* c, int32_t layer,
                            const int32_t* budget, const int32_t* n_orig, void* ws,
                            conf_stream_t stream);

/*
 * The same after conf_attend: the pending score EMA first (n16 and t advance),
 * in the same launch.  conf_attend + conf_arkv_ema_evict_compact give exactly
 * the results of conf_decode_attn + conf_arkv_evict_compact.
 */
int conf_arkv_ema_evict_compact(const conf_params* p, conf_cache* c, int32_t layer,
                                const int32_t* budget, const int32_t* n_orig, void* ws,
                                conf_stream_t stream);

/*
 * ARKV's prefill phase [arkv-prefill] (CONF_POLICY_ARKV only): the statistics
 * from which each layer's Original budget follows.  For every (layer, sequence)
 * of the layer selector and each query head h: the softmax, scale 1/sqrt(d), of
 * the probe query q_h over the prefill keys of KV head h / (Hq/Hkv) gives
 * weights p over prefill_len = L0 tokens; with d_j = p_j - 1/L0,
 *   H^ = -sum p ln p / ln L0,   v^ = L0 sum d^2 / (L0 - 1),
 *   k^ = ln(max(L0 sum d^4 / (sum d^2)^2, 1)) / ln L0  (0 when every d is 0),
 *   concentration = ((1 - H^) + v^ + k^) / 3,
 * and conc[l][b] is its mean over the Hq heads (float32; two passes over the
 * keys, the heads of a KV head summed in order, then the KV heads in order).
 * q: 16-bit [L][B][Hq][d] (layer = -1) or [B][Hq][d] (layer = l): the first query
 * that attends to the whole prefill (the first decode step's); k_pre: 16-bit
 * [L][B][Hkv][L0][d] or [B][Hkv][L0][d], as given to conf_cache_ingest.  conc:
 * fp32 [L][B]; only the selected layers' rows are written.  CONF_E_INVALID
 * under any other policy, for L0 < 2, or on a null or misaligned pointer.
 */
int conf_arkv_prefill_stats(const conf_params* p, int32_t layer, const void* q,
                            const void* k_pre, int32_t prefill_len, float* conc, void* ws,
                            conf_stream_t stream);

/*
 * ARKV's layer-wise Original budgets [arkv-prefill] (CONF_POLICY_ARKV only) from
 * conc (fp32 [L][B], conf_arkv_prefill_stats): per sequence b, with lo and hi
 * the least and largest concentration over its layers, the OQ ratio of layer l
 * is r = 0.75 + (0.95 - 0.75) (conc - lo) / (hi - lo) (r = (0.75 + 0.95) / 2
 * when hi = lo): the more concentrated a layer's prefill attention, the more of
 * its budget stays Original.  n_orig[b][l] = max(P, ceil(r * n_high)), int32
 * [B][L], computed in float32 one rounding at a time.  n_orig is the n_orig of
 * conf_arkv_evict_compact / conf_arkv_ema_evict_compact.
 */
int conf_arkv_orig_budgets(const conf_params* p, const float* conc, int32_t* n_orig,
                           conf_stream_t stream);

/*
 * The prefill's retention (CONF_POLICY_TRIM only), right after
 * conf_cache_ingest of `prefill_len` tokens: log_beta fp32 [L][B][prefill_len]
 * (layer = -1) or [B][prefill_len] gives ln(beta) of positions 0 ..
 * prefill_len-1.
 */
int conf_cache_set_retention(const conf_params* p, conf_cache* c, int32_t layer,
                             const float* log_beta, int32_t prefill_len, conf_stream_t stream);

/*
 * One full decode step of every layer and sequence: conf_attend(-1),
 * conf_confidence and conf_ema_evict_compact(-1), the same results as
 * conf_decode_attn(-1), conf_confidence, conf_rank_evict(-1) and
 * conf_compact_demote(-1).  c: fp32 [B] and budget: int32 [B][L] receive (a)'s
 * results.
 */
int conf_step(const conf_params* p, conf_cache* c, const float* logits, const void* q,
              const void* k_new, const void* v_new, float* out, float* conf, int32_t* budget,
              void* ws, conf_stream_t stream);

/*
 * conf_step without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The step's scratch (conf_workspace_bytes() of it) is a
 * static device array inside the library, CONF_STATIC_SCRATCH_BYTES (32 MiB) per
 * GPU, which each GPU holds from the library's first use on it until the process
 * ends; the call allocates nothing.  Shapes whose workspace exceeds that return
 * CONF_E_CAPACITY before any device work (conf_last_error() says how much they
 * need).  Every call on one GPU shares that GPU's array and leaves its contents
 * behind (nothing in it needs to start at zero): calls that overlap on one GPU
 * race, so a process must order them (one stream, or events).  The first call
 * on a device looks up the array's device address (hipGetSymbolAddress) and
 * keeps it; CONF_E_HIP if that fails.  Results are identical to conf_step's.
 */
#define CONF_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
int conf_step_static(const conf_params* p, conf_cache* c, const float* logits, const void* q,
                     const void* k_new, const void* v_new, float* out, float* conf,
                     int32_t* budget, conf_stream_t stream);

/*
 * Copy one (layer, sequence) into plain row-major arrays in slot order, for
 * inspection: k8, v8: int8 [cap8][Hkv][d]; k16, v16: 16-bit [cap16][Hkv][d].
 * Slots beyond n8 / n16 hold whatever the cache held.
 */
int conf_cache_export(const conf_params* p, const conf_cache* c, int32_t layer, int32_t seq,
                      int8_t* k8, int8_t* v8, void* k16, void* v16, conf_stream_t stream);

/* Text of the last CONF_E_HIP error on this thread (and of conf_step_static's
 * CONF_E_CAPACITY), or of a status code. */
const char* conf_last_error(void);
const char* conf_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* CONFKV_H */
