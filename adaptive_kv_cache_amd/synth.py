"""Seeded synthetic inputs for the CONF-KV decode step.

Every tensor the decode-step path consumes (vocab logits, per-layer q / k / v,
a prefilled context and its planted needle) is drawn here from a counter-style
seed (base seed, stream tag, step), so any single step can be regenerated on its
own.  The same inputs feed the HIP path and the CPU checker.  This module holds
no arithmetic of the method itself: only random draws and the workload's
temperature schedule.

The explainer pages measure on trained models (GPT-2, Qwen-14B/32B,
gpt-oss-20b) with perplexity, needle-in-a-haystack and agent benchmarks; those
are stood in for by N(0,1) tensors of the models' shapes.
"""
from __future__ import annotations

import math

import torch

from .workloads import Workload

(_TAG_LOGITS, _TAG_TEMP, _TAG_Q, _TAG_K, _TAG_V, _TAG_PRE_K, _TAG_PRE_V, _TAG_NEEDLE,
 _TAG_BETA, _TAG_PRE_BETA, _TAG_OQ) = range(11)

TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16}


def _gen(seed: int, tag: int, step: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + tag * 1_009 * 65_537 + step * 7_919) % (2**63 - 1))
    return g


def temperatures(wl: Workload, step: int, seed: int) -> torch.Tensor:
    """Per-sequence logit multiplier T for `step` (float64, CPU).

    "alt": 0.5 for steps [0, 64), 8 for [64, 128), and so on, shared by every
    sequence.  "uniform": independent U[1.5, 3] per step and sequence.
    """
    if wl.temp_schedule == "alt":
        t = 0.5 if (step // 64) % 2 == 0 else 8.0
        return torch.full((wl.batch,), t, dtype=torch.float64)
    g = _gen(seed, _TAG_TEMP, step, "cpu")
    return 1.5 + 1.5 * torch.rand(wl.batch, generator=g, dtype=torch.float64)


def logits(wl: Workload, step: int, seed: int, device="cpu") -> torch.Tensor:
    """Vocab logits [B][V] float32 = N(0,1) * T_t (T multiplies)."""
    g = _gen(seed, _TAG_LOGITS, step, device)
    z = torch.randn(wl.batch, wl.vocab, generator=g, device=device, dtype=torch.float32)
    z *= temperatures(wl, step, seed).to(device=device, dtype=torch.float32)[:, None]
    return z


def q_new(wl: Workload, step: int, seed: int, device="cpu", layers=None) -> torch.Tensor:
    """Queries [L][B][Hq][d] in the workload's 16-bit dtype."""
    nl = wl.n_layers if layers is None else layers
    g = _gen(seed, _TAG_Q, step, device)
    x = torch.randn(nl, wl.batch, wl.n_q_heads, wl.head_dim, generator=g, device=device)
    return x.to(TORCH_DTYPE[wl.dtype16])


def kv_new(wl: Workload, step: int, seed: int, device="cpu", layers=None):
    """New key and value rows [L][B][Hkv][d] in the workload's 16-bit dtype."""
    nl = wl.n_layers if layers is None else layers
    shape = (nl, wl.batch, wl.n_kv_heads, wl.head_dim)
    gk = _gen(seed, _TAG_K, step, device)
    gv = _gen(seed, _TAG_V, step, device)
    k = torch.randn(*shape, generator=gk, device=device).to(TORCH_DTYPE[wl.dtype16])
    v = torch.randn(*shape, generator=gv, device=device).to(TORCH_DTYPE[wl.dtype16])
    return k, v


def needle_site(wl: Workload, seed: int):
    """(position, decode step) of the planted needle, or None."""
    if not wl.needle or wl.prefill <= wl.window:
        return None
    g = _gen(seed, _TAG_NEEDLE, 0, "cpu")
    pos = int(torch.randint(0, wl.prefill - wl.window, (1,), generator=g))
    step = int(torch.randint(0, wl.steps, (1,), generator=g))
    return pos, step


def prefill_kv(wl: Workload, layer: int, seed: int, device="cpu", length=None):
    """Prefilled keys and values of one layer, [B][Hkv][L0][d] 16-bit.

    With a needle, the key at the needle position becomes 4*sqrt(d) times the
    unit query of head (h_kv * g) at the needle's decode step, so that query
    attends to it strongly ("norm x4, aligned to a later query").
    """
    L0 = wl.prefill if length is None else length
    shape = (wl.batch, wl.n_kv_heads, L0, wl.head_dim)
    gk = _gen(seed, _TAG_PRE_K, layer, device)
    gv = _gen(seed, _TAG_PRE_V, layer, device)
    k = torch.randn(*shape, generator=gk, device=device)
    v = torch.randn(*shape, generator=gv, device=device)
    site = needle_site(wl, seed)
    if site is not None and site[0] < L0:
        pos, step = site
        q = q_new(wl, step, seed, device=device)[layer]
        q = q.float()[:, :: wl.group, :]                       # heads h_kv * g
        qhat = q / q.norm(dim=-1, keepdim=True).clamp_min(1e-30)
        k[:, :, pos, :] = 4.0 * math.sqrt(wl.head_dim) * qhat
    dt = TORCH_DTYPE[wl.dtype16]
    return k.to(dt), v.to(dt)


def _log_gate(z: torch.Tensor) -> torch.Tensor:
    # a retention gate's output: beta = sigmoid(z), given as ln(beta) <= 0
    return torch.nn.functional.logsigmoid(z)


def log_beta_new(wl: Workload, step: int, seed: int, device="cpu", layers=None) -> torch.Tensor:
    """ln(beta) of each new token, fp32 [L][B]: beta = sigmoid(z), z ~ N(4, 2),
    so most tokens decay slowly (beta near 0.98) and a tail decays fast.  Stands
    in for a trained retention gate's output."""
    nl = wl.n_layers if layers is None else layers
    g = _gen(seed, _TAG_BETA, step, device)
    z = 4.0 + 2.0 * torch.randn(nl, wl.batch, generator=g, device=device, dtype=torch.float32)
    return _log_gate(z)


def log_beta_prefill(wl: Workload, layer: int, seed: int, device="cpu", length=None):
    """ln(beta) of the prefilled tokens of one layer, fp32 [B][L0], drawn as in
    log_beta_new."""
    L0 = wl.prefill if length is None else length
    g = _gen(seed, _TAG_PRE_BETA, layer, device)
    z = 4.0 + 2.0 * torch.randn(wl.batch, L0, generator=g, device=device, dtype=torch.float32)
    return _log_gate(z)


def arkv_n_orig(wl: Workload, seed: int) -> torch.Tensor:
    """Original-token budget of each layer, int32 [L]: ceil(r_l * N_high) with a
    random OQ ratio r_l ~ U[0.75, 0.95], at least P.  For tests of the three-state
    step that choose their own budgets; ARKV's own budgets follow from the prefill
    attention statistics (conf_arkv_prefill_stats, conf_arkv_orig_budgets)."""
    g = _gen(seed, _TAG_OQ, 0, "cpu")
    r = 0.75 + 0.2 * torch.rand(wl.n_layers, generator=g, dtype=torch.float64)
    n = torch.ceil(r * wl.n_high).to(torch.int32)
    return torch.clamp(n, min=wl.protect)
