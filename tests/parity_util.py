"""Test-side glue between the HIP library (through its binding) and the oracle.

Maps a (layer, sequence) exported from the device into the oracle's
position-ordered state, compares states, and builds small workloads that span
several 64-token tiles with ragged tails.
"""
from __future__ import annotations

import numpy as np
import torch

from adaptive_kv_cache_amd.workloads import Workload
from oracle import LayerSeqState, OracleParams

F32 = np.float32


def oracle_params(wl: Workload) -> OracleParams:
    return OracleParams(n_layers=wl.n_layers, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                        head_dim=wl.head_dim, dtype16=wl.dtype16, window=wl.window,
                        protect=wl.protect, n_high=wl.n_high, n_low=wl.n_low,
                        pyramid=wl.pyramid, tau=wl.tau, w_H=wl.w_H, w_m=wl.w_m, w_p=wl.w_p,
                        ema_decay=wl.ema_decay, s_ema=wl.s_ema, s_rec=wl.s_rec)


def bits16(t: torch.Tensor) -> np.ndarray:
    """16-bit tensor -> numpy uint16 bit patterns (CPU copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def to_oracle_state(ex: dict, dtype16: str) -> LayerSeqState:
    n8, n16 = ex["n8"], ex["n16"]
    H, D = ex["k_amax"].shape
    st = LayerSeqState(H, D, dtype16)
    pos = np.concatenate([ex["pos8"], ex["pos16"]]).astype(np.int64)
    order = np.argsort(pos, kind="stable")
    z8 = np.zeros((n16, H, D), np.int8)
    z16 = np.zeros((n8, H, D), np.uint16)
    st.pos = pos[order]
    st.is8 = np.concatenate([np.ones(n8, bool), np.zeros(n16, bool)])[order]
    st.k8 = np.concatenate([ex["k8"], z8])[order]
    st.v8 = np.concatenate([ex["v8"], z8])[order]
    st.k16 = np.concatenate([z16, ex["k16"]])[order]
    st.v16 = np.concatenate([z16, ex["v16"]])[order]
    st.ema = np.concatenate([ex["ema8"], ex["ema16"]]).astype(np.float64)[order]
    st.amax_k = ex["k_amax"].astype(F32).copy()
    st.amax_v = ex["v_amax"].astype(F32).copy()
    st.t = ex["t"]
    return st


def ema_by_pos(ex: dict) -> dict:
    pos = np.concatenate([ex["pos8"], ex["pos16"]])
    ema = np.concatenate([ex["ema8"], ex["ema16"]])
    return dict(zip(pos.tolist(), ema.tolist()))


def kept_positions(ex_after_attn: dict, keep_row: np.ndarray, cap8: int) -> set:
    n8, n16 = ex_after_attn["n8"], ex_after_attn["n16"]
    k8 = keep_row[:n8].astype(bool)
    k16 = keep_row[cap8:cap8 + n16].astype(bool)
    return set(ex_after_attn["pos8"][k8].tolist()) | set(ex_after_attn["pos16"][k16].tolist())


def assert_same_state(gpu: LayerSeqState, ref: LayerSeqState, ema_rtol=None, what=""):
    """Bit-exact comparison of two position-ordered states (EMA optional, tolerance)."""
    assert gpu.t == ref.t, (what, gpu.t, ref.t)
    assert np.array_equal(gpu.pos, ref.pos), (what, "positions differ")
    assert np.array_equal(gpu.is8, ref.is8), (what, "precision split differs")
    m8 = ref.is8
    assert np.array_equal(gpu.k8[m8], ref.k8[m8]), (what, "INT8 key codes differ")
    assert np.array_equal(gpu.v8[m8], ref.v8[m8]), (what, "INT8 value codes differ")
    assert np.array_equal(gpu.k16[~m8], ref.k16[~m8]), (what, "window keys differ")
    assert np.array_equal(gpu.v16[~m8], ref.v16[~m8]), (what, "window values differ")
    assert np.array_equal(gpu.amax_k.view(np.uint32), ref.amax_k.view(np.uint32)), (what, "K absmax")
    assert np.array_equal(gpu.amax_v.view(np.uint32), ref.amax_v.view(np.uint32)), (what, "V absmax")
    if ema_rtol is not None:
        np.testing.assert_allclose(gpu.ema, ref.ema, rtol=ema_rtol, atol=1e-12, err_msg=what)


def attn_rel_err(o_gpu: np.ndarray, o_ref: np.ndarray) -> float:
    """max over heads of ||o_gpu - o_ref||_inf / ||o_ref||_inf."""
    num = np.max(np.abs(o_gpu - o_ref), axis=-1)
    den = np.maximum(np.max(np.abs(o_ref), axis=-1), 1e-30)
    return float(np.max(num / den))


def tiny_workloads() -> dict:
    """Shapes the oracle finishes in seconds that still span several 64-token tiles,
    ragged tails, every supported head_dim, dtype and query-group width."""
    w = {}
    w["mha_f16_d64"] = Workload(
        name="mha_f16_d64", n_layers=2, batch=2, n_q_heads=4, n_kv_heads=4, head_dim=64,
        vocab=1000, dtype16="f16", window=80, protect=16, n_high=150, n_low=260, prefill=0,
        steps=320, pyramid=True)
    w["gqa5_bf16_d128"] = Workload(
        name="gqa5_bf16_d128", n_layers=2, batch=2, n_q_heads=10, n_kv_heads=2, head_dim=128,
        vocab=3001, dtype16="bf16", window=70, protect=20, n_high=130, n_low=200, prefill=517,
        steps=40)
    w["gqa8_bf16_d64"] = Workload(
        name="gqa8_bf16_d64", n_layers=1, batch=3, n_q_heads=16, n_kv_heads=2, head_dim=64,
        vocab=2048, dtype16="bf16", window=64, protect=8, n_high=100, n_low=180, prefill=300,
        steps=40, pyramid=False)
    w["gqa16_f16_d128"] = Workload(
        name="gqa16_f16_d128", n_layers=1, batch=1, n_q_heads=16, n_kv_heads=1, head_dim=128,
        vocab=777, dtype16="f16", window=33, protect=5, n_high=40, n_low=90, prefill=200,
        steps=30)
    # from empty with 2 x 8 x 128 (K|V, KV head, channel) triples: the early demotions grow
    # more than 512 channels of a non-empty INT8 region (the requantisation list overflows)
    w["mha_bf16_d128_empty"] = Workload(
        name="mha_bf16_d128_empty", n_layers=1, batch=2, n_q_heads=8, n_kv_heads=8, head_dim=128,
        vocab=500, dtype16="bf16", window=24, protect=6, n_high=40, n_low=70, prefill=0,
        steps=150)
    # more scores than the LDS holds at the first step: the items past the LDS rows
    # keep theirs in the workspace
    w["gqa16_bf16_d64_long"] = Workload(
        name="gqa16_bf16_d64_long", n_layers=1, batch=2, n_q_heads=16, n_kv_heads=1, head_dim=64,
        vocab=500, dtype16="bf16", window=64, protect=8, n_high=100, n_low=300, prefill=2500,
        steps=8)
    # 16 KV heads of 128 channels: the largest Hkv * d the library takes (2048), so the
    # demotion uses all eight (K|V, head, channel) triples per compaction thread
    w["mha16_f16_d128"] = Workload(
        name="mha16_f16_d128", n_layers=1, batch=2, n_q_heads=16, n_kv_heads=16, head_dim=128,
        vocab=600, dtype16="f16", window=40, protect=8, n_high=60, n_low=100, prefill=150,
        steps=12)
    # every budget above what the LDS score rows hold, so that every step also keeps
    # scores in the workspace
    w["gqa16_bf16_d64_wide"] = Workload(
        name="gqa16_bf16_d64_wide", n_layers=1, batch=2, n_q_heads=16, n_kv_heads=1,
        head_dim=64, vocab=500, dtype16="bf16", window=64, protect=8, n_high=1300, n_low=1400,
        prefill=2500, steps=6)
    # d = 128 with 16 query heads: the LDS keeps the scores of about 1040 tokens, and
    # the window of 1200 is longer than that, so the items that keep their scores in
    # the workspace start inside the window (the INT8 part fits)
    w["gqa16_f16_d128_winspill"] = Workload(
        name="gqa16_f16_d128_winspill", n_layers=1, batch=2, n_q_heads=16, n_kv_heads=1,
        head_dim=128, vocab=700, dtype16="f16", window=1200, protect=50, n_high=1400,
        n_low=1700, prefill=1600, steps=8)
    # d = 128 with 16 query heads and a window of 250 (eight halves, the last one
    # ragged): every cache holds more tokens than the LDS score rows, so the
    # wavefronts keep their window halves' scores in registers; the first step's
    # INT8 part is longer than the rows as well (its tail goes to the workspace),
    # the later steps' INT8 part fits them
    w["gqa16_bf16_d128_held"] = Workload(
        name="gqa16_bf16_d128_held", n_layers=1, batch=2, n_q_heads=16, n_kv_heads=1,
        head_dim=128, vocab=600, dtype16="bf16", window=250, protect=30, n_high=1100,
        n_low=1250, prefill=2000, steps=8)
    return w
