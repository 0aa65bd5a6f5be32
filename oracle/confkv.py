"""Plain CPU oracle of the CONF-KV decode step (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this module.  It shares no code with the HIP library or its binding and
imports nothing from them.

What it follows.  Every citation below names a section of the CONF-KV explainer
pages: the gist.science technical summary of "CONF-KV: Confidence-Aware KV Cache
Eviction with Mixed-Precision Storage for Long-Horizon LLM" (Yubo Li, Yidi Miao),
whose Dutch, Italian and Korean renderings agree on every formula and number.
  [Method/confidence]  Methodology, confidence estimation: the scalar
                       c = w_H(1 - H^) + w_m sigma(m) + w_p p(1), weights (0.4, 0.3, 0.3).
  [Method/budget]      Methodology, adaptive budget selection: c >= tau gives the
                       tight budget N_high, c < tau the loose N_low; sawtooth memory.
  [Method/ranking]     Methodology, token ranking and eviction: a composite of EMA
                       attention mass and recency; a hard protected window P.
  [Method/storage]     Methodology, system integration, mixed-precision storage:
                       newest W tokens in 16 bits, older kept tokens INT8 per head
                       and channel.
  [Method/pyramid]     Methodology, system integration, pyramidal budgets
                       (CONF-KV-L): deeper layers get smaller budgets.
  [Method/impl]        Methodology, system integration, implementation: contiguous
                       compaction to a dense layout, dequantisation fused into
                       block-wise attention reads.
  [Contrib/system]     Key contributions, system design: block-wise online-softmax
                       attention.
  [Significance]       Significance and claims: a no-op on contexts that never pass
                       the eviction threshold.

Precision.  Attention, token mass and confidence are computed in float64 from
their definitions.  The composite score and the INT8 quantiser are integer-
deciding steps and are written out in float32, one correctly rounded operation
at a time (numpy float32 element-wise arithmetic never fuses a multiply-add).

Readings where the pages leave a step open (each is stated again at its
function):
  * normalised entropy H^ = H / ln V; margin m = z(1) - z(2) in nats (a tie gives
    m = 0); sigma is the logistic function; softmax at temperature 1.
  * any non-finite logit makes c NaN, and NaN >= tau is false, so N_low applies.
  * N counts every kept token of a (layer, sequence), both precisions, protected
    ones included; one keep set per (layer, sequence), shared by all KV heads.
  * token mass = mean over the layer's query heads of this step's softmax
    probability; EMA e <- decay*e + (1-decay)*mass, new tokens start at 0 and are
    updated at their first step.
  * score s = s_ema * (e / e_max) + s_rec * (pos / t), fp32; ties broken by the
    newer position; protected = positions in (t - P, t].
  * window = positions in (t - W, t]; after eviction the token at position t - W,
    if it survived, is demoted.  INT8 is symmetric, codes in [-127, 127], round
    half to even, one fp32 scale = running absmax / 127 per (KV head, channel);
    a new maximum requantises that channel's existing codes.
  * pyramid: N_l = floor(N * (2(L-1) - l) / (2(L-1))), i.e. 1.0x at layer 0 and
    0.5x at the last layer; applies to both budgets.
  * attention scale 1/sqrt(d); the new token attends to itself; no mask.
  * ARKV's prefill phase: each layer's statistics are those of the softmax
    attention of the first query that attends to the whole prefill (the first
    decode step's query) over the 16-bit prefill keys; entropy, variance and
    kurtosis of the weights are each normalised to [0, 1], their mean (with the
    entropy as 1 - H^) is the layer's concentration, averaged over its query
    heads; more concentrated counts as more sensitive to precision loss, and the
    OQ ratio runs linearly from 0.75 (least concentrated layer of the sequence)
    to 0.95 (most concentrated).

Baseline policies the pages compare CONF-KV with ([Problem] sliding windows,
[Results] full KV) are the same step under other parameters:
  * full KV: no token is ever evicted or demoted, i.e. step_layer with a budget
    no cache reaches and a window no position leaves (W > t);
  * sliding window: P = W = N, so the protected newest W positions are exactly
    what stays, all 16-bit; a window cache never holds an older token, so its
    ingest drops the prefill before position L0 - W (`ingest(..., drop_old=True)`).
The baselines need no EMA; the oracle still computes one, which tests ignore.

Retention eviction (the TRIM-KV page, Methodology: retention gate, inference and
eviction): each token carries a retention score beta in [0, 1] fixed when it is
created; its current score at step t is beta^(t - i); once the cache is at its
limit M the lowest current score leaves.  Readings:
  * beta is supplied per token and (layer, sequence), as its logarithm
    l = ln beta <= 0 in float32 (the gate that predicts it is training, not part
    of the decode step); tokens are ranked by ln(beta^(t-i)) = (t - i) * l, one
    float32 product, 0 for the newest token (beta^0 = 1) -- the same order as
    beta^(t-i) in exact arithmetic;
  * ties go to the newer position, as in CONF-KV's ranking; one keep set per
    (layer, sequence); the cache holds at most M tokens after each step, all
    16-bit (the page names no quantisation), and no window is protected beyond
    the newest token.

Head-wise budgets (the CONF-KV page, Significance and claims: the method composes
with head-wise allocation).  Readings:
  * each KV head of a (layer, sequence) keeps its own tokens, so the heads'
    caches have their own lengths, windows and INT8 splits;
  * the layer's budget for the sequence is Hkv * N_l (token, head) pairs, spent
    jointly: a head's own newest P positions are protected, and the other pairs
    compete on the composite score with e_max over every head of the layer;
  * a token's mass in head h is the mean over that head's G query heads;
  * ties: score desc, then position desc, then head index desc.

ARKV (the ARKV page, Methodology: three-state assignment, decoding-phase token
ranking, prefill-phase layer-wise budgets).  Readings:
  * states: Original (16-bit), Quantized (FP8 e4m3, the OCP "fn" form: bias 7,
    three mantissa bits, largest finite 448, subnormals down to 2^-9), Evicted;
    per (KV head, channel) a running absmax, scale = absmax / 448, codes by
    round-to-nearest-even of x / scale clamped to +-448, requantised on a new
    maximum as for INT8;
  * heavy-hitter score of a token this step: over the KV heads, the mean plus
    the population variance of m_k = its attention averaged over head k's query
    heads; ranked on its EMA (decay as for CONF-KV), ties to the newer position;
  * budgets per (layer, sequence): N kept tokens and N_O Original ones (the
    layer's OQ ratio, computed at prefill, is an input); the newest P positions
    are protected and stay Original;
  * a step appends the token as Original, evicts below the top N, then while more
    than N_O tokens are Original, quantises the lowest-ranked unprotected one.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

F32 = np.float32
F64 = np.float64

__all__ = [
    "OracleParams", "LayerSeqState", "decode16", "encode16", "confidence", "budget",
    "layer_budget", "dequantize", "attention", "attention_online", "token_mass",
    "ema_update", "composite_scores", "select_keep", "quant_codes", "requant_codes",
    "demote_token", "ingest", "step_layer", "decode_step",
    "retention_scores", "trim_step", "joint_keep", "headwise_step",
    "FP8_MAX", "fp8_decode", "fp8_encode", "quant_codes_fp8", "requant_codes_fp8",
    "arkv_stat", "Fp8State", "ingest_fp8", "arkv_step",
    "ARKV_R_LO", "ARKV_R_HI", "attention_weights_stats", "arkv_prefill_concentration",
    "arkv_orig_budgets",
]


@dataclass
class OracleParams:
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype16: str            # "f16" | "bf16"
    window: int             # W
    protect: int            # P
    n_high: int
    n_low: int
    pyramid: bool = False
    tau: float = 0.5
    w_H: float = 0.4
    w_m: float = 0.3
    w_p: float = 0.3
    ema_decay: float = 0.9
    s_ema: float = 0.7
    s_rec: float = 0.3

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


# --------------------------------------------------------------------------
# 16-bit storage values
# --------------------------------------------------------------------------
def decode16(bits, dtype16: str) -> np.ndarray:
    """Raw 16-bit patterns -> exact float32 values (IEEE half or bfloat16)."""
    b = np.asarray(bits).astype(np.uint16)
    if dtype16 == "f16":
        return b.view(np.float16).astype(F32)
    if dtype16 == "bf16":
        return (b.astype(np.uint32) << 16).view(F32)
    raise ValueError(dtype16)


def encode16(x, dtype16: str) -> np.ndarray:
    """float -> 16-bit patterns, round to nearest even (test-input helper)."""
    x = np.asarray(x, dtype=F32)
    if dtype16 == "f16":
        return x.astype(np.float16).view(np.uint16)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


# --------------------------------------------------------------------------
# (a) confidence and budget                                [Method/confidence]
# --------------------------------------------------------------------------
def confidence(z, w_H=0.4, w_m=0.3, w_p=0.3) -> dict:
    """Scalar confidence of one step's next-token logits, from the definition.

    p = softmax(z); H = -sum p ln p (0 ln 0 = 0); H^ = H / ln V; m = z(1) - z(2),
    the two largest logits with duplicates counted; p(1) = max p;
    c = w_H (1 - H^) + w_m / (1 + e^-m) + w_p p(1).   [Method/confidence]
    Any non-finite logit gives c = NaN (the budget rule then picks N_low).
    """
    z = np.asarray(z, dtype=F64).ravel()
    V = z.size
    if V < 2:
        raise ValueError("vocabulary of at least two tokens required")
    if not np.all(np.isfinite(z)):
        nan = float("nan")
        return dict(c=nan, H_hat=nan, m=nan, p1=nan)
    zmax = z.max()
    e = np.exp(z - zmax)
    p = e / e.sum()
    pos = p[p > 0]
    H = -np.sum(pos * np.log(pos))
    H_hat = H / math.log(V)
    top = np.sort(z)
    m = top[-1] - top[-2]
    p1 = p.max()
    sig = 1.0 / (1.0 + math.exp(-m))
    c = w_H * (1.0 - H_hat) + w_m * sig + w_p * p1
    return dict(c=float(c), H_hat=float(H_hat), m=float(m), p1=float(p1))


def budget(c: float, tau: float, n_high: int, n_low: int) -> int:
    """c >= tau -> N_high (tight); otherwise (NaN included) N_low.  [Method/budget]"""
    return n_high if c >= tau else n_low


def layer_budget(N: int, layer: int, n_layers: int, pyramid: bool) -> int:
    """Per-layer budget; CONF-KV-L shrinks it linearly to half at the last layer
    (integer floor).  [Method/pyramid]"""
    if not pyramid or n_layers <= 1:
        return N
    D = 2 * (n_layers - 1)
    return (N * (D - layer)) // D


# --------------------------------------------------------------------------
# (b) attention over the mixed-precision cache    [Method/storage] [Contrib/system]
# --------------------------------------------------------------------------
def dequantize(codes, amax) -> np.ndarray:
    """INT8 code * scale in float64, scale = fp32(amax / 127) per (head, channel)."""
    s = (np.asarray(amax, F32) / F32(127.0)).astype(F32)
    return np.asarray(codes).astype(F64) * s.astype(F64)


def attention(q, K, V, group: int):
    """Softmax attention of one decode query, two-pass, float64.

    q [Hq, d]; K, V [n, Hkv, d] (already dequantised); query head h reads KV head
    h // group.  Returns o [Hq, d] and probabilities p [Hq, n].
    """
    q = np.asarray(q, F64)
    Hq, d = q.shape
    n, Hkv, _ = K.shape
    o = np.zeros((Hq, d), F64)
    p = np.zeros((Hq, n), F64)
    for hk in range(Hkv):
        hs = slice(hk * group, (hk + 1) * group)
        sig = (q[hs] @ K[:, hk, :].T) / math.sqrt(d)            # [g, n]
        mx = sig.max(axis=1, keepdims=True)
        e = np.exp(sig - mx)
        ph = e / e.sum(axis=1, keepdims=True)
        p[hs] = ph
        o[hs] = ph @ V[:, hk, :]
    return o, p


def attention_online(q, K, V, group: int, block: int = 64):
    """Block-wise online-softmax form of `attention` (float64).  [Contrib/system]

    Running (max, sum, accumulator) per head, rescaled by exp(m_old - m_new)
    whenever a block raises the maximum; the result is divided by the sum at the
    end.  Reaches the two-pass result up to rounding.
    """
    q = np.asarray(q, F64)
    Hq, d = q.shape
    n = K.shape[0]
    o = np.zeros((Hq, d), F64)
    for h in range(Hq):
        hk = h // group
        m, l = -np.inf, 0.0
        acc = np.zeros(d, F64)
        for s0 in range(0, n, block):
            sig = (K[s0:s0 + block, hk, :] @ q[h]) / math.sqrt(d)
            m_new = max(m, sig.max())
            corr = math.exp(m - m_new) if np.isfinite(m) else 0.0
            w = np.exp(sig - m_new)
            l = l * corr + w.sum()
            acc = acc * corr + w @ V[s0:s0 + block, hk, :]
            m = m_new
        o[h] = acc / l
    return o


# --------------------------------------------------------------------------
# (c) token mass and EMA                                       [Method/ranking]
# --------------------------------------------------------------------------
def token_mass(p) -> np.ndarray:
    """Attention mass of each token this step: mean over the query heads."""
    return np.asarray(p, F64).mean(axis=0)


def ema_update(e, mass, decay: float) -> np.ndarray:
    return decay * np.asarray(e, F64) + (1.0 - decay) * np.asarray(mass, F64)


# --------------------------------------------------------------------------
# (d) composite score and top-N selection                      [Method/ranking]
# --------------------------------------------------------------------------
def composite_scores(e32, pos, t: int, s_ema: float, s_rec: float) -> np.ndarray:
    """s = s_ema * (e / e_max) + s_rec * (pos / t), each op one fp32 rounding.

    e_max is over every cached token of the (layer, sequence); e / e_max is 0 when
    e_max is 0; pos / t is 1 when t is 0.
    """
    e32 = np.asarray(e32, F32)
    pos = np.asarray(pos)
    emax = e32.max() if e32.size else F32(0)
    if emax > 0:
        ehat = (e32 / emax).astype(F32)
    else:
        ehat = np.zeros_like(e32)
    if t > 0:
        r = (pos.astype(F32) / F32(t)).astype(F32)
    else:
        r = np.ones(pos.shape, F32)
    a = (F32(s_ema) * ehat).astype(F32)
    b = (F32(s_rec) * r).astype(F32)
    return (a + b).astype(F32)


def select_keep(scores, pos, t: int, P: int, N: int) -> np.ndarray:
    """Keep mask of one (layer, sequence).  [Method/ranking] [Significance]

    n <= N keeps everything (the method is a no-op below its budget).
    Otherwise the protected positions (t - P, t] are kept, plus the best
    K = N - |protected| other tokens in the order (score desc, position desc).
    """
    scores = np.asarray(scores, F32)
    pos = np.asarray(pos, np.int64)
    n = pos.size
    keep = np.ones(n, bool)
    if n <= N:
        return keep
    prot = pos > (t - P)
    K = N - int(prot.sum())
    if K < 0:
        raise ValueError("protected window larger than the budget")
    cand = np.flatnonzero(~prot)
    order = np.lexsort((-pos[cand], -scores[cand]))
    keep[:] = prot
    keep[cand[order[:K]]] = True
    return keep


def retention_scores(log_beta32, pos, t: int) -> np.ndarray:
    """Current retention log-score (t - i) * ln(beta_i) of each token, float32,
    one rounding; 0 for the newest token.  [TRIM-KV: inference and eviction]"""
    lb = np.asarray(log_beta32, F32)
    age = (t - np.asarray(pos, np.int64)).astype(F32)
    with np.errstate(invalid="ignore"):
        s = (age * lb).astype(F32)
    s[age == 0] = F32(0)
    return s


# --------------------------------------------------------------------------
# (e) INT8 quantiser, per (KV head, channel)                    [Method/storage]
# --------------------------------------------------------------------------
def quant_codes(x32, s32) -> np.ndarray:
    """code = clamp(rne(x / s), -127, 127) in fp32; a zero scale gives code 0."""
    x32 = np.asarray(x32, F32)
    s32 = np.broadcast_to(np.asarray(s32, F32), x32.shape)
    r = np.zeros(x32.shape, F32)
    nz = s32 > 0
    r[nz] = x32[nz] / s32[nz]
    return np.clip(np.rint(r), -127, 127).astype(np.int8)


def requant_codes(codes, s_old, s_new) -> np.ndarray:
    """Re-express codes under a larger scale: clamp(rne((q * s_old) / s_new))."""
    q = np.asarray(codes).astype(F32)
    prod = (q * np.asarray(s_old, F32)).astype(F32)
    return quant_codes(prod, s_new)


def demote_token(x32, amax, codes_all):
    """Quantise one token row x [Hkv, d] into INT8 under the running absmax.

    Channels where |x| exceeds the running absmax first requantise the codes
    already stored (codes_all [n8, Hkv, d], updated in place) and take |x| as the
    new absmax.  Returns (codes [Hkv, d], new amax).
    """
    x32 = np.asarray(x32, F32)
    amax = np.asarray(amax, F32).copy()
    a = np.abs(x32)
    grow = a > amax
    if grow.any() and codes_all.shape[0] > 0:
        s_old = (amax / F32(127.0)).astype(F32)
        s_new = (np.where(grow, a, amax) / F32(127.0)).astype(F32)
        sub = codes_all[:, grow]
        codes_all[:, grow] = requant_codes(sub, s_old[grow], s_new[grow])
    amax = np.where(grow, a, amax).astype(F32)
    s = (amax / F32(127.0)).astype(F32)
    return quant_codes(x32, s), amax


# --------------------------------------------------------------------------
# cache state of one (layer, sequence)
# --------------------------------------------------------------------------
class LayerSeqState:
    """Cache of one (layer, sequence), tokens in position order.

    For each token: position, precision (16-bit window or INT8), its 16-bit bits
    (window tokens) or INT8 codes (older tokens), and its EMA mass.  Per (KV
    head, channel): running absmax of K and of V.  t is the newest position
    (-1 for an empty cache).
    """

    def __init__(self, n_kv_heads: int, head_dim: int, dtype16: str):
        H, d = n_kv_heads, head_dim
        self.dtype16 = dtype16
        self.pos = np.zeros(0, np.int64)
        self.is8 = np.zeros(0, bool)
        self.k16 = np.zeros((0, H, d), np.uint16)
        self.v16 = np.zeros((0, H, d), np.uint16)
        self.k8 = np.zeros((0, H, d), np.int8)
        self.v8 = np.zeros((0, H, d), np.int8)
        self.ema = np.zeros(0, F64)
        self.amax_k = np.zeros((H, d), F32)
        self.amax_v = np.zeros((H, d), F32)
        self.t = -1

    @property
    def n(self) -> int:
        return int(self.pos.size)

    def copy(self) -> "LayerSeqState":
        c = LayerSeqState(self.k16.shape[1], self.k16.shape[2], self.dtype16)
        for f in ("pos", "is8", "k16", "v16", "k8", "v8", "ema", "amax_k", "amax_v"):
            setattr(c, f, getattr(self, f).copy())
        c.t = self.t
        return c

    def kv_values(self):
        """Dequantised K, V [n, Hkv, d] float64: exact 16-bit values or code*scale."""
        K = np.where(self.is8[:, None, None], dequantize(self.k8, self.amax_k),
                     decode16(self.k16, self.dtype16).astype(F64))
        V = np.where(self.is8[:, None, None], dequantize(self.v8, self.amax_v),
                     decode16(self.v16, self.dtype16).astype(F64))
        return K, V

    def append(self, k_bits, v_bits):
        """The decoded token joins the 16-bit window at position t+1, EMA 0."""
        self.t += 1
        H, d = self.k16.shape[1:]
        self.pos = np.append(self.pos, self.t)
        self.is8 = np.append(self.is8, False)
        self.k16 = np.concatenate([self.k16, np.asarray(k_bits, np.uint16).reshape(1, H, d)])
        self.v16 = np.concatenate([self.v16, np.asarray(v_bits, np.uint16).reshape(1, H, d)])
        self.k8 = np.concatenate([self.k8, np.zeros((1, H, d), np.int8)])
        self.v8 = np.concatenate([self.v8, np.zeros((1, H, d), np.int8)])
        self.ema = np.append(self.ema, 0.0)

    def evict(self, keep):
        keep = np.asarray(keep, bool)
        for f in ("pos", "is8", "k16", "v16", "k8", "v8", "ema"):
            setattr(self, f, getattr(self, f)[keep])

    def demote(self, W: int):
        """Move the token at position t - W (if still cached) out of the window.

        [Method/storage]: the window holds the newest W positions; a token that
        leaves it is quantised into INT8 with its (KV head, channel) scales.
        """
        target = self.t - W
        if target < 0:
            return
        idx = np.flatnonzero(self.pos == target)
        if idx.size == 0:
            return
        j = int(idx[0])
        assert not self.is8[j]
        old8 = np.flatnonzero(self.is8)
        xk = decode16(self.k16[j], self.dtype16)
        xv = decode16(self.v16[j], self.dtype16)
        ck = self.k8[old8]
        cv = self.v8[old8]
        code_k, self.amax_k = demote_token(xk, self.amax_k, ck)
        code_v, self.amax_v = demote_token(xv, self.amax_v, cv)
        self.k8[old8] = ck
        self.v8[old8] = cv
        self.k8[j] = code_k
        self.v8[j] = code_v
        self.k16[j] = 0
        self.v16[j] = 0
        self.is8[j] = True


def ingest(k_bits, v_bits, W: int, dtype16: str, drop_old: bool = False) -> LayerSeqState:
    """Prefilled context [Hkv, L0, d] (16-bit patterns) -> cache state.

    Positions 0 .. L0-W-1 go to INT8 with the absmax taken over exactly those
    tokens (with drop_old, the sliding-window baseline, they are not kept at
    all); positions L0-W .. L0-1 stay 16-bit; every EMA is 0; t = L0 - 1.
    """
    k_bits = np.asarray(k_bits, np.uint16)
    v_bits = np.asarray(v_bits, np.uint16)
    H, L0, d = k_bits.shape
    if drop_old and L0 > W:
        st = ingest(k_bits[:, L0 - W:], v_bits[:, L0 - W:], W, dtype16)
        st.pos = st.pos + (L0 - W)
        st.t = L0 - 1
        return st
    st = LayerSeqState(H, d, dtype16)
    st.pos = np.arange(L0, dtype=np.int64)
    st.is8 = st.pos < (L0 - W)
    st.k16 = np.ascontiguousarray(k_bits.transpose(1, 0, 2))
    st.v16 = np.ascontiguousarray(v_bits.transpose(1, 0, 2))
    st.k8 = np.zeros((L0, H, d), np.int8)
    st.v8 = np.zeros((L0, H, d), np.int8)
    st.ema = np.zeros(L0, F64)
    st.t = L0 - 1
    old = st.is8
    if old.any():
        for name, src, dst in (("amax_k", st.k16, st.k8), ("amax_v", st.v16, st.v8)):
            x = decode16(src[old], dtype16)                       # [n8, H, d]
            amax = np.abs(x).max(axis=0).astype(F32)
            s = (amax / F32(127.0)).astype(F32)
            dst[old] = quant_codes(x, s)
            setattr(st, name, amax)
        st.k16[old] = 0
        st.v16[old] = 0
    return st


# --------------------------------------------------------------------------
# one decode step
# --------------------------------------------------------------------------
def step_layer(st: LayerSeqState, q_bits, k_bits, v_bits, N: int, prm: OracleParams,
               ema32_override=None) -> dict:
    """One decode step of one (layer, sequence); `st` is updated in place.

    Order: append, attention (float64, two-pass), mass + EMA, score + select
    against budget N, evict, demote position t - W.  The selection reads the
    float32 rounding of the EMA, or `ema32_override` (the same length as the
    cache after append) when the caller wants to feed a given score input.
    """
    st.append(k_bits, v_bits)
    q = decode16(q_bits, prm.dtype16).astype(F64)
    K, V = st.kv_values()
    o, p = attention(q, K, V, prm.group)
    mass = token_mass(p)
    st.ema = ema_update(st.ema, mass, prm.ema_decay)
    ema64 = st.ema.copy()
    e32 = st.ema.astype(F32) if ema32_override is None else np.asarray(ema32_override, F32)
    scores = composite_scores(e32, st.pos, st.t, prm.s_ema, prm.s_rec)
    keep = select_keep(scores, st.pos, st.t, prm.protect, N)
    pos_before = st.pos.copy()
    if ema32_override is not None:
        st.ema = np.asarray(ema32_override, F64)
    st.evict(keep)
    st.demote(prm.window)
    return dict(o=o, p=p, mass=mass, ema=ema64, scores=scores, keep=keep, pos_before=pos_before)


def trim_step(st: LayerSeqState, q_bits, k_bits, v_bits, log_beta_new: float, M: int,
              prm: OracleParams) -> dict:
    """One step of retention eviction for one (layer, sequence); `st.ema` holds
    each token's ln(beta) (float32 values).  Append (with this step's ln beta),
    attention over the cache (float64), then keep the M tokens with the highest
    current retention score (ties: newer first).  No token is quantised.
    [TRIM-KV: retention gate; inference and eviction]"""
    st.append(k_bits, v_bits)
    st.ema[-1] = float(np.float32(log_beta_new))
    q = decode16(q_bits, prm.dtype16).astype(F64)
    K, V = st.kv_values()
    o, p = attention(q, K, V, prm.group)
    scores = retention_scores(st.ema.astype(F32), st.pos, st.t)
    keep = select_keep(scores, st.pos, st.t, 1, M)
    st.evict(keep)
    return dict(o=o, p=p, scores=scores, keep=keep)


def joint_keep(e32_heads, pos_heads, t: int, P: int, N_total: int, s_ema: float,
               s_rec: float):
    """Keep masks of the KV heads of one (layer, sequence) under a shared budget of
    N_total (token, head) pairs.  [Significance: head-wise allocation]

    Scores are composite_scores over every head's tokens together, so e_max is the
    largest EMA of the layer.  Below the budget everything stays.  Otherwise each
    head's positions (t - P, t] stay, and the best N_total - |protected| other
    pairs in the order (score desc, position desc, head desc).
    """
    H = len(e32_heads)
    sizes = [np.asarray(p).size for p in pos_heads]
    e_all = np.concatenate([np.asarray(e, F32) for e in e32_heads]) if H else np.zeros(0, F32)
    pos_all = np.concatenate([np.asarray(p, np.int64) for p in pos_heads])
    head_all = np.concatenate([np.full(n, h, np.int64) for h, n in enumerate(sizes)])
    keep = np.ones(pos_all.size, bool)
    if pos_all.size > N_total:
        scores = composite_scores(e_all, pos_all, t, s_ema, s_rec)
        prot = pos_all > (t - P)
        K = N_total - int(prot.sum())
        if K < 0:
            raise ValueError("protected windows larger than the budget")
        cand = np.flatnonzero(~prot)
        order = np.lexsort((-head_all[cand], -pos_all[cand], -scores[cand]))
        keep[:] = prot
        keep[cand[order[:K]]] = True
    return np.split(keep, np.cumsum(sizes)[:-1])


def headwise_step(heads, q_bits, k_bits, v_bits, N: int, prm: OracleParams,
                  ema32_override=None) -> dict:
    """One decode step of one (layer, sequence) with head-wise keep sets.

    heads[h] is the LayerSeqState of KV head h alone (one KV head each); q_bits
    [Hq][d], k_bits and v_bits [Hkv][d].  Per head: append, attention of its G
    query heads (float64), mass (mean over those G) and EMA.  Then joint_keep with
    Hkv * N pairs, and per head eviction and the demotion of position t - W.
    The selection reads the float32 rounding of each head's EMA, or
    ema32_override[h] (one value per token after the append), as step_layer does.
    [Method/ranking] [Method/storage] [Significance: head-wise allocation]
    """
    G = prm.group
    H = len(heads)
    q = decode16(q_bits, prm.dtype16).astype(F64)
    outs, emas = [], []
    for h, st in enumerate(heads):
        st.append(np.asarray(k_bits)[h:h + 1], np.asarray(v_bits)[h:h + 1])
        K, V = st.kv_values()
        o, p = attention(q[h * G:(h + 1) * G], K, V, G)
        st.ema = ema_update(st.ema, token_mass(p), prm.ema_decay)
        emas.append(st.ema.copy())
        outs.append(o)
        if ema32_override is not None:
            st.ema = np.asarray(ema32_override[h], F32).astype(F64)
    t = heads[0].t
    keeps = joint_keep([st.ema.astype(F32) for st in heads], [st.pos for st in heads], t,
                       prm.protect, H * N, prm.s_ema, prm.s_rec)
    pos_before = [st.pos.copy() for st in heads]
    for st, kp in zip(heads, keeps):
        st.evict(kp)
        st.demote(prm.window)
    return dict(o=np.concatenate(outs), keeps=keeps, ema=emas, pos_before=pos_before)


# --------------------------------------------------------------------------
# ARKV: FP8 e4m3 codes, heavy-hitter score, three states        [ARKV]
# --------------------------------------------------------------------------
FP8_MAX = 448.0


def fp8_decode(codes) -> np.ndarray:
    """Value of each e4m3 bit pattern (uint8 or int8 bits), float64: sign, four
    exponent bits (bias 7), three mantissa bits; exponent 0 is subnormal
    (m * 2^-9).  0x7f / 0xff (NaN) are never produced here."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(F64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(F64) - 7.0))
    return sign * mag


_FP8_POS = fp8_decode(np.arange(0x7F))          # codes 0x00 .. 0x7e, increasing


def fp8_encode(x32) -> np.ndarray:
    """Nearest e4m3 code (int8 bit pattern) of each value with |x| <= 448, ties to
    the even code; the sign bit follows x (so -0 gives 0x80)."""
    x = np.asarray(x32, F32).astype(F64)
    a = np.abs(x)
    if (a > FP8_MAX).any() or np.isnan(a).any():
        raise ValueError("fp8_encode takes |x| <= 448")
    hi = np.searchsorted(_FP8_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _FP8_POS[lo]
    dhi = _FP8_POS[hi] - a
    pick = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(hi % 2 == 0, hi, lo)))
    code = pick | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8).view(np.int8)


def quant_codes_fp8(x32, s32) -> np.ndarray:
    """code = e4m3(clamp(x / s, -448, 448)) with the division in fp32; a zero
    scale gives code 0."""
    x32 = np.asarray(x32, F32)
    s32 = np.broadcast_to(np.asarray(s32, F32), x32.shape)
    r = np.zeros(x32.shape, F32)
    nz = s32 > 0
    r[nz] = x32[nz] / s32[nz]
    r = np.clip(r, F32(-FP8_MAX), F32(FP8_MAX)).astype(F32)
    return fp8_encode(r)


def requant_codes_fp8(codes, s_old, s_new) -> np.ndarray:
    """Re-express e4m3 codes under a larger scale: e4m3((value * s_old) / s_new),
    fp32 arithmetic (the decoded value is exact in fp32)."""
    v = fp8_decode(codes).astype(F32)
    prod = (v * np.asarray(s_old, F32)).astype(F32)
    return quant_codes_fp8(prod, s_new)


def dequantize_fp8(codes, amax) -> np.ndarray:
    """Code value * scale in float64, scale = fp32(amax / 448)."""
    s = (np.asarray(amax, F32) / F32(FP8_MAX)).astype(F32)
    return fp8_decode(codes) * s.astype(F64)


def arkv_stat(p, group: int) -> np.ndarray:
    """Heavy-hitter score of each token this step (float64) from p [Hq, n]:
    m_k = mean of p over KV head k's query heads; mean_k m_k + var_k m_k
    (population variance over the KV heads).  [ARKV: decoding-phase ranking]"""
    p = np.asarray(p, F64)
    Hq, n = p.shape
    m = p.reshape(Hq // group, group, n).mean(axis=1)
    mu = m.mean(axis=0)
    return mu + ((m - mu) ** 2).mean(axis=0)


class Fp8State(LayerSeqState):
    """A cache whose 8-bit tokens hold e4m3 codes (the ARKV Quantized state)."""

    def copy(self) -> "Fp8State":
        c = Fp8State(self.k16.shape[1], self.k16.shape[2], self.dtype16)
        for f in ("pos", "is8", "k16", "v16", "k8", "v8", "ema", "amax_k", "amax_v"):
            setattr(c, f, getattr(self, f).copy())
        c.t = self.t
        return c

    def kv_values(self):
        K = np.where(self.is8[:, None, None], dequantize_fp8(self.k8, self.amax_k),
                     decode16(self.k16, self.dtype16).astype(F64))
        V = np.where(self.is8[:, None, None], dequantize_fp8(self.v8, self.amax_v),
                     decode16(self.v16, self.dtype16).astype(F64))
        return K, V

    def quantise(self, j: int):
        """Token j (Original) becomes Quantized: per (KV head, channel) a larger |x|
        first requantises the stored codes of that channel and becomes the absmax;
        then code = e4m3(x / (absmax / 448))."""
        assert not self.is8[j]
        old8 = np.flatnonzero(self.is8)
        for key, amax_name, c8 in (("k16", "amax_k", "k8"), ("v16", "amax_v", "v8")):
            x = decode16(getattr(self, key)[j], self.dtype16).astype(F32)
            amax = getattr(self, amax_name).astype(F32)
            a = np.abs(x)
            grow = a > amax
            codes = getattr(self, c8)
            if grow.any() and old8.size:
                s_old = (amax / F32(FP8_MAX)).astype(F32)
                s_new = (np.where(grow, a, amax) / F32(FP8_MAX)).astype(F32)
                hh, cc = np.nonzero(grow)
                rows = old8[:, None]
                codes[rows, hh[None, :], cc[None, :]] = requant_codes_fp8(
                    codes[rows, hh[None, :], cc[None, :]], s_old[hh, cc], s_new[hh, cc])
            amax = np.where(grow, a, amax).astype(F32)
            setattr(self, amax_name, amax)
            codes[j] = quant_codes_fp8(x, (amax / F32(FP8_MAX)).astype(F32))
            getattr(self, key)[j] = 0
        self.is8[j] = True


def ingest_fp8(k_bits, v_bits, W: int, dtype16: str) -> Fp8State:
    """ARKV prefill: positions 0 .. L0-W-1 Quantized (absmax over exactly those
    tokens), the newest W Original, every score 0, t = L0 - 1."""
    k_bits = np.asarray(k_bits, np.uint16)
    v_bits = np.asarray(v_bits, np.uint16)
    H, L0, d = k_bits.shape
    st = Fp8State(H, d, dtype16)
    st.pos = np.arange(L0, dtype=np.int64)
    st.is8 = st.pos < (L0 - W)
    st.k16 = np.ascontiguousarray(k_bits.transpose(1, 0, 2))
    st.v16 = np.ascontiguousarray(v_bits.transpose(1, 0, 2))
    st.k8 = np.zeros((L0, H, d), np.int8)
    st.v8 = np.zeros((L0, H, d), np.int8)
    st.ema = np.zeros(L0, F64)
    st.t = L0 - 1
    old = st.is8
    if old.any():
        for name, src, dst in (("amax_k", st.k16, st.k8), ("amax_v", st.v16, st.v8)):
            x = decode16(src[old], dtype16).astype(F32)
            amax = np.abs(x).max(axis=0).astype(F32)
            dst[old] = quant_codes_fp8(x, (amax / F32(FP8_MAX)).astype(F32))
            setattr(st, name, amax)
        st.k16[old] = 0
        st.v16[old] = 0
    return st


def arkv_step(st: Fp8State, q_bits, k_bits, v_bits, N: int, N_O: int, prm: OracleParams,
              ema32_override=None) -> dict:
    """One ARKV decode step of one (layer, sequence).  [ARKV: three-state
    assignment; decoding-phase ranking]

    Append as Original; attention (float64) over Original values and dequantised
    Quantized ones; heavy-hitter score and its EMA; keep the protected newest P
    and the best N - |protected| others by (EMA desc, position desc); then, while
    more than N_O kept tokens are Original, the lowest-ranked unprotected one is
    quantised (lowest first).  The ranking reads the fp32 rounding of the EMA, or
    `ema32_override` (one value per token after the append).
    """
    st.append(k_bits, v_bits)
    q = decode16(q_bits, prm.dtype16).astype(F64)
    K, V = st.kv_values()
    o, p = attention(q, K, V, prm.group)
    st.ema = ema_update(st.ema, arkv_stat(p, prm.group), prm.ema_decay)
    ema64 = st.ema.copy()
    e32 = st.ema.astype(F32) if ema32_override is None else np.asarray(ema32_override, F32)
    if ema32_override is not None:
        st.ema = e32.astype(F64)
    keep = select_keep(e32, st.pos, st.t, prm.protect, N)
    pos_before = st.pos.copy()
    st.evict(keep)
    e32 = e32[keep]
    demoted = []
    while int((~st.is8).sum()) > N_O:
        cand = np.flatnonzero(~st.is8 & (st.pos <= st.t - prm.protect))
        if cand.size == 0:
            break
        j = cand[np.lexsort((st.pos[cand], e32[cand]))[0]]   # lowest (score, position)
        demoted.append(int(st.pos[j]))
        st.quantise(int(j))
    return dict(o=o, p=p, ema=ema64, keep=keep, pos_before=pos_before, demoted=demoted)


# --------------------------------------------------------------------------
# ARKV prefill phase: layer-wise Original budgets from attention statistics
# [ARKV: Methodology, 1. prefill phase (layer-wise budget assignment)]
# --------------------------------------------------------------------------
ARKV_R_LO, ARKV_R_HI = 0.75, 0.95   # the OQ ratios of the least and most concentrated layer


def attention_weights_stats(p) -> dict:
    """Entropy, variance and kurtosis of one attention distribution p over L0
    tokens (float64), each normalised to [0, 1] so that higher means more
    concentrated.  [ARKV: prefill statistics: entropy (spatial spread), variance
    (difference in token weights), kurtosis (shape of the distribution)]

      H^ = -sum p ln p / ln L0                (1: uniform, 0: one token)
      d  = p - 1/L0                           (deviations from the uniform weight)
      v^ = L0 * sum d^2 / (L0 - 1)            (the weights' variance over its
                                               one-token maximum: 0 uniform, 1 one token)
      k  = L0 * sum d^4 / (sum d^2)^2         (fourth standardised moment of the weights)
      k^ = ln(max(k, 1)) / ln L0              (0 for uniform weights, where k is undefined)
      concentration = ((1 - H^) + v^ + k^) / 3
    Two passes: the deviations are formed from the normalised weights, not from
    power sums, so near-uniform weights keep their precision.
    """
    p = np.asarray(p, F64).ravel()
    L0 = p.size
    if L0 < 2:
        raise ValueError("at least two tokens")
    pos = p[p > 0]
    H_hat = float(-np.sum(pos * np.log(pos)) / math.log(L0))
    d = p - 1.0 / L0
    s2 = float(np.sum(d * d))
    s4 = float(np.sum(d ** 4))
    v_hat = L0 * s2 / (L0 - 1)
    if s2 > 0.0:
        kurt = L0 * s4 / (s2 * s2)
        k_hat = math.log(max(kurt, 1.0)) / math.log(L0)
    else:
        kurt, k_hat = float("nan"), 0.0
    conc = ((1.0 - H_hat) + v_hat + k_hat) / 3.0
    return dict(H_hat=H_hat, v_hat=v_hat, kurtosis=kurt, k_hat=k_hat, conc=conc)


def arkv_prefill_concentration(q, K, group: int) -> np.ndarray:
    """Per query head of one (layer, sequence): the concentration of the softmax
    attention of its probe query q [Hq, d] over the prefill keys K [Hkv, L0, d]
    (float64, scale 1/sqrt(d), KV head h // group), and their mean over the
    heads as the (layer, sequence)'s value.  Returns [Hq + 1]: the heads' values,
    then the mean.  [ARKV: prefill phase]"""
    q = np.asarray(q, F64)
    K = np.asarray(K, F64)
    Hq, d = q.shape
    out = np.zeros(Hq + 1, F64)
    for h in range(Hq):
        z = K[h // group] @ q[h] / math.sqrt(d)
        p = np.exp(z - z.max())
        p /= p.sum()
        out[h] = attention_weights_stats(p)["conc"]
    out[Hq] = out[:Hq].mean()
    return out


def arkv_orig_budgets(conc32, N: int, P: int) -> np.ndarray:
    """Original budget N_O of each layer of one sequence from its layers'
    concentrations (float32, one per layer): the most concentrated layer keeps
    ARKV_R_HI of its N tokens Original, the least ARKV_R_LO, linearly between by
    concentration; all layers alike give the midpoint.  N_O = max(P, ceil(r N)).
    Evaluated in float32 one rounding at a time (it decides an integer).
    [ARKV: prefill phase: layers more sensitive to precision loss get a larger
    full-precision budget]"""
    c = np.asarray(conc32, F32)
    lo, hi = F32(c.min()), F32(c.max())
    span = F32(hi - lo)
    r_lo, r_hi = F32(ARKV_R_LO), F32(ARKV_R_HI)
    width = F32(r_hi - r_lo)
    if span > F32(0):
        t = ((c - lo).astype(F32) / span).astype(F32)
        r = (r_lo + (width * t).astype(F32)).astype(F32)
    else:
        r = np.full(c.shape, F32(F32(r_lo + r_hi) / F32(2)), F32)
    n = np.ceil((r * F32(N)).astype(F32)).astype(np.int64)
    return np.maximum(n, P).astype(np.int32)


def decode_step(states, logits, q_bits, k_bits, v_bits, prm: OracleParams,
                budget_override=None) -> dict:
    """One decode step of the whole batch and every layer.

    states[l][b] are LayerSeqState; logits [B][V]; q_bits [L][B][Hq][d];
    k_bits, v_bits [L][B][Hkv][d].  The budget of sequence b comes from its
    confidence (or from budget_override[b]); the pyramid spreads it over layers.
    """
    L = len(states)
    B = len(states[0])
    conf = [confidence(logits[b], prm.w_H, prm.w_m, prm.w_p) for b in range(B)]
    Ns = []
    for b in range(B):
        N = (budget(conf[b]["c"], prm.tau, prm.n_high, prm.n_low)
             if budget_override is None else int(budget_override[b]))
        Ns.append(N)
    out = np.zeros((L, B) + np.asarray(q_bits).shape[2:], F64)
    for l in range(L):
        for b in range(B):
            Nl = layer_budget(Ns[b], l, prm.n_layers, prm.pyramid)
            r = step_layer(states[l][b], q_bits[l][b], k_bits[l][b], v_bits[l][b], Nl, prm)
            out[l, b] = r["o"]
    return dict(out=out, c=np.array([cf["c"] for cf in conf]), N=np.array(Ns))
