"""Workload shapes and hyper-parameters for the CONF-KV decode-step path.

The CONF-KV explainer pages (gist.science technical summary of "CONF-KV:
Confidence-Aware KV Cache Eviction with Mixed-Precision Storage for
Long-Horizon LLM", Experimental results) evaluate four model families
(GPT-2, Qwen-14B/32B, gpt-oss-20b) but print none of tau, N_high, N_low, P, W,
the EMA decay or the score weights.  The values below are the synthetic
workload definitions this library is measured on; only the confidence
weights (0.4, 0.3, 0.3) come from the pages (Methodology, confidence
estimation).

This module holds shapes and constants only: no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

WORKLOAD_NAMES = (
    "gpt2_1layer_b1",
    "gpt2_12layer_b8_pyramid",
    "qwen14b_gqa_b8_8k",
    "qwen32b_gqa_b8_32k",
    "qwen32b_gqa_b1_32k",
    "gptoss20b_gqa_b32_16k",
    "gptoss20b_gqa_b32_16k_stress",
)

# Confidence threshold of the gpt-oss-20b-shaped stress variant: the median of the
# confidence c over every step and sequence of that workload's own seeded logits
# (seed 0, 512 steps x 32 sequences, T ~ U[1.5, 3], drawn on the GPU as the bench
# draws them), as the CPU checker computes it, rounded to float32.  It is the c of
# one row (step 318, sequence 31), so one step sits at the threshold.  With it
# about half the steps are confident and a sequence's budget changes on about half
# of consecutive steps.  Written by tests/golden/make_tau_stress.py into
# tests/golden/gptoss20b_tau_stress.json.
TAU_STRESS_GPTOSS = 0.2645609676837921


@dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    dtype16: str          # "f16" or "bf16": q, k, v and the 16-bit window
    window: int           # W: newest tokens kept in 16 bits
    protect: int          # P: newest tokens that are never evicted
    n_high: int           # tight budget, used when c >= tau
    n_low: int            # loose budget, used when c < tau
    prefill: int          # tokens ingested before the first decode step (0 = empty)
    steps: int            # decode steps of the full workload
    pyramid: bool = False  # CONF-KV-L: budgets shrink linearly 1.0x -> 0.5x over depth
    tau: float = 0.5
    w_H: float = 0.4
    w_m: float = 0.3
    w_p: float = 0.3
    ema_decay: float = 0.9
    s_ema: float = 0.7
    s_rec: float = 0.3
    temp_schedule: str = "alt"   # "alt": 0.5 / 8 in 64-step runs; "uniform": U[1.5, 3]
    needle: bool = False
    policy: str = "confkv"       # "confkv", or a baseline: "full" (full KV), "window" (sliding),
                                 # "trim" (retention eviction), "arkv" (ARKV's three states)
    headwise: bool = False       # per-KV-head keep sets sharing Hkv * N pairs per layer

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def cap8(self) -> int:
        """INT8-region capacity in tokens per (layer, sequence), a multiple of 64."""
        old = 0 if self.policy == "window" else self.prefill - self.window  # a window drops them
        per_budget = self.n_low * (self.n_kv_heads if self.headwise else 1)
        need = max(old, per_budget + 1, 64)
        return (need + 63) // 64 * 64

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def n_sub(self) -> int:
        """Caches per layer: sequences, or (sequence, KV head) pairs head-wise."""
        return self.batch * (self.n_kv_heads if self.headwise else 1)

    def headwise_variant(self) -> "Workload":
        """The same shape with head-wise keep sets."""
        return replace(self, name=f"{self.name}_hw", headwise=True)

    def baseline(self, policy: str, horizon: int) -> "Workload":
        """The same shape under a baseline policy, for `horizon` decode steps.

        full: the window holds the prefill and every decoded token (rounded up to
        64); budgets and P at their smallest valid values, since nothing is evicted.
        window: a W-token sliding window; P = N_high = N_low = W and no pyramid, so
        the ranking keeps exactly the protected newest W.
        arkv: ARKV's three states with N = N_high kept tokens, up to 95% of them
        Original (W = ceil(0.95 N) sizes the 16-bit arrays), P = 32; the prefill is
        cut to W tokens, all Original, so that after a few steps the cache is in
        ARKV's steady state (N tokens, N_O of them Original) rather than a
        positional split that Original tokens could never win back.
        trim: retention eviction with memory budget M = N_high, held entirely in the
        16-bit window (W = M); P = 1 protects the token being appended; the prefill
        is cut to M tokens, which is the cache that retention eviction holds once it
        has run over a longer one.
        """
        if policy == "confkv":
            return self
        if policy == "full":
            w = (self.prefill + horizon + 1 + 63) // 64 * 64
            return replace(self, name=f"{self.name}_full", policy="full", window=w, protect=1,
                           n_high=64, n_low=64, pyramid=False)
        if policy == "window":
            return replace(self, name=f"{self.name}_window", policy="window", protect=self.window,
                           n_high=self.window, n_low=self.window, pyramid=False)
        if policy == "trim":
            m = self.n_high
            return replace(self, name=f"{self.name}_trim", policy="trim", window=m, protect=1,
                           n_high=m, n_low=m, pyramid=False, prefill=min(self.prefill, m),
                           needle=False)
        if policy == "arkv":
            # N = N_high kept tokens, at most 95% of them Original (the layers' OQ
            # ratios lie in [0.75, 0.95]); the window arrays hold the Original ones;
            # the page's example protects the newest 32
            n = self.n_high
            w = -(-95 * n // 100)
            return replace(self, name=f"{self.name}_arkv", policy="arkv", window=w,
                           protect=min(32, w), n_high=n, n_low=n, pyramid=False,
                           prefill=min(self.prefill, w), needle=False)
        raise ValueError(policy)


def _mk() -> dict:
    gpt2 = dict(n_q_heads=12, n_kv_heads=12, head_dim=64, vocab=50257, dtype16="f16",
                window=128, protect=64, n_high=384, n_low=768, prefill=0, steps=2048)
    qwen = dict(n_q_heads=40, n_kv_heads=8, head_dim=128, vocab=152064, dtype16="bf16")
    w = {}
    w["gpt2_1layer_b1"] = Workload(name="gpt2_1layer_b1", n_layers=1, batch=1, **gpt2)
    w["gpt2_12layer_b8_pyramid"] = Workload(name="gpt2_12layer_b8_pyramid", n_layers=12,
                                            batch=8, pyramid=True, **gpt2)
    w["qwen14b_gqa_b8_8k"] = Workload(name="qwen14b_gqa_b8_8k", n_layers=48, batch=8,
                                      window=256, protect=128, n_high=1024, n_low=2048,
                                      prefill=8192, steps=1024, **qwen)
    q32 = dict(n_layers=64, window=512, protect=256, n_high=2048, n_low=4096,
               prefill=32768, steps=512, needle=True, **qwen)
    w["qwen32b_gqa_b8_32k"] = Workload(name="qwen32b_gqa_b8_32k", batch=8, **q32)
    w["qwen32b_gqa_b1_32k"] = Workload(name="qwen32b_gqa_b1_32k", batch=1, **q32)
    w["gptoss20b_gqa_b32_16k"] = Workload(
        name="gptoss20b_gqa_b32_16k", n_layers=24, batch=32, n_q_heads=64, n_kv_heads=8,
        head_dim=64, vocab=201088, dtype16="bf16", window=256, protect=64, n_high=1024,
        n_low=2048, prefill=16384, steps=512, pyramid=True, temp_schedule="uniform")
    # the same shape with c near tau, so that budgets flip often (the high-temperature
    # regime the pages single out, where the confidence signal is least informative)
    w["gptoss20b_gqa_b32_16k_stress"] = replace(
        w["gptoss20b_gqa_b32_16k"], name="gptoss20b_gqa_b32_16k_stress", tau=TAU_STRESS_GPTOSS)
    return w


WORKLOADS = _mk()


def get(name: str) -> Workload:
    return WORKLOADS[name]
