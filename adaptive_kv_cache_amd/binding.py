"""ctypes binding of libconfkv.so (the C ABI in include/confkv.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity (so no kernel is launched on operands of the wrong size) and their
data pointers are handed to the library together with torch's current stream.
Every step of the decode path runs in the library's HIP kernels; there is no
fallback.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_size_t, c_void_p

import torch

from .workloads import Workload

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libconfkv.so")

CONF_F16, CONF_BF16 = 1, 2
DTYPE16 = {"f16": (CONF_F16, torch.float16), "bf16": (CONF_BF16, torch.bfloat16)}
ST_WINDOW_FULL, ST_INT8_FULL = 1, 2
STATIC_SCRATCH_BYTES = 32 << 20   # CONF_STATIC_SCRATCH_BYTES: conf_step_static's workspace
POLICY = {"confkv": 0, "full": 1, "window": 2, "trim": 3, "arkv": 4}

EXPORTED = ("conf_cache_layout", "conf_workspace_bytes", "conf_cache_reset", "conf_cache_ingest",
            "conf_confidence", "conf_decode_attn", "conf_rank_evict", "conf_compact_demote",
            "conf_evict_compact", "conf_attend", "conf_ema_evict_compact",
            "conf_trim_evict_compact", "conf_cache_set_retention", "conf_arkv_evict_compact",
            "conf_arkv_ema_evict_compact", "conf_arkv_prefill_stats", "conf_arkv_orig_budgets",
            "conf_step", "conf_step_static",
            "conf_cache_export", "conf_last_error", "conf_status_string")


class ConfParams(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in ("n_layers", "batch", "n_q_heads", "n_kv_heads", "head_dim",
                                        "vocab", "dtype16", "window", "protect", "n_high", "n_low",
                                        "cap8", "pyramid")] + \
               [(n, c_float) for n in ("tau", "w_H", "w_m", "w_p", "ema_decay", "s_ema", "s_rec")] + \
               [("policy", c_int32), ("headwise", c_int32)]


_CACHE_FIELDS = ("k8", "v8", "k16", "v16", "k_amax", "v_amax", "pos8", "ema8", "pos16", "ema16",
                 "n8", "n16", "t", "status")


class ConfCache(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in _CACHE_FIELDS]


class ConfCacheBytes(ctypes.Structure):
    _fields_ = [(n, c_size_t) for n in _CACHE_FIELDS] + [("cap16", c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libconfkv.so once; raise if it is missing (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m adaptive_kv_cache_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, C = POINTER(ConfParams), POINTER(ConfCache)
    vp = c_void_p
    sig = {
        "conf_cache_layout": [P, POINTER(ConfCacheBytes)],
        "conf_workspace_bytes": [P, POINTER(c_size_t)],
        "conf_cache_reset": [P, C, vp],
        "conf_cache_ingest": [P, C, c_int32, vp, vp, c_int32, vp, vp],
        "conf_confidence": [P, vp, vp, vp, vp, vp],
        "conf_decode_attn": [P, C, c_int32, vp, vp, vp, vp, vp, vp],
        "conf_rank_evict": [P, C, c_int32, vp, vp, vp, vp],
        "conf_compact_demote": [P, C, c_int32, vp, vp, vp],
        "conf_evict_compact": [P, C, c_int32, vp, vp, vp],
        "conf_attend": [P, C, c_int32, vp, vp, vp, vp, vp, vp],
        "conf_ema_evict_compact": [P, C, c_int32, vp, vp, vp],
        "conf_trim_evict_compact": [P, C, c_int32, vp, vp, vp, vp],
        "conf_cache_set_retention": [P, C, c_int32, vp, c_int32, vp],
        "conf_arkv_evict_compact": [P, C, c_int32, vp, vp, vp, vp],
        "conf_arkv_ema_evict_compact": [P, C, c_int32, vp, vp, vp, vp],
        "conf_arkv_prefill_stats": [P, c_int32, vp, vp, c_int32, vp, vp, vp],
        "conf_arkv_orig_budgets": [P, vp, vp, vp],
        "conf_step": [P, C, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "conf_step_static": [P, C, vp, vp, vp, vp, vp, vp, vp, vp],
        "conf_cache_export": [P, C, c_int32, c_int32, vp, vp, vp, vp, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = c_int
    lib.conf_last_error.argtypes = []
    lib.conf_last_error.restype = c_char_p
    lib.conf_status_string.argtypes = [c_int]
    lib.conf_status_string.restype = c_char_p
    _lib = lib
    return lib


class ConfKVError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != 0:
        lib = load()
        msg = lib.conf_status_string(rc).decode()
        extra = lib.conf_last_error().decode() if rc == -4 else ""
        raise ConfKVError(f"{what} failed: {msg} ({rc}) {extra}".strip())


def params_from_workload(wl: Workload, cap8: int | None = None, **over) -> ConfParams:
    d = dict(n_layers=wl.n_layers, batch=wl.batch, n_q_heads=wl.n_q_heads,
             n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim, vocab=wl.vocab,
             dtype16=DTYPE16[wl.dtype16][0], window=wl.window, protect=wl.protect,
             n_high=wl.n_high, n_low=wl.n_low, cap8=wl.cap8 if cap8 is None else cap8,
             pyramid=int(wl.pyramid), tau=wl.tau, w_H=wl.w_H, w_m=wl.w_m, w_p=wl.w_p,
             ema_decay=wl.ema_decay, s_ema=wl.s_ema, s_rec=wl.s_rec,
             policy=POLICY[wl.policy], headwise=int(wl.headwise))
    d.update(over)
    return ConfParams(**d)


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


class Engine:
    """Device state of one cache plus its workspace; every method is one C-ABI call.

    All tensors live on `device`; calls are enqueued on torch's current stream.
    """

    def __init__(self, wl: Workload, device="cuda", cap8: int | None = None, **over):
        self.lib = load()
        self.wl = wl
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.p = params_from_workload(wl, cap8, **over)
        self.dtype16 = DTYPE16[wl.dtype16][1]
        sizes = ConfCacheBytes()
        _check(self.lib.conf_cache_layout(ctypes.byref(self.p), ctypes.byref(sizes)), "layout")
        self.cap8 = self.p.cap8
        self.cap16 = sizes.cap16
        ws = c_size_t()
        _check(self.lib.conf_workspace_bytes(ctypes.byref(self.p), ctypes.byref(ws)), "workspace")
        L, B, Hkv, D = wl.n_layers, wl.batch, wl.n_kv_heads, wl.head_dim
        dev = self.device
        U = L * B * Hkv
        S = wl.n_sub      # caches per layer: sequences, or (sequence, KV head) head-wise
        self.n_sub = S
        self.t_k8 = torch.zeros(U * self.cap8 * D, dtype=torch.int8, device=dev)
        self.t_v8 = torch.zeros_like(self.t_k8)
        # the reset below zeroes the window arrays itself
        self.t_k16 = torch.empty(U * self.cap16 * D, dtype=torch.int16, device=dev)
        self.t_v16 = torch.empty_like(self.t_k16)
        self.t_k_amax = torch.zeros(L, B, Hkv, D, dtype=torch.float32, device=dev)
        self.t_v_amax = torch.zeros_like(self.t_k_amax)
        self.t_pos8 = torch.zeros(L, S, self.cap8, dtype=torch.int32, device=dev)
        self.t_ema8 = torch.zeros(L, S, self.cap8, dtype=torch.float32, device=dev)
        self.t_pos16 = torch.zeros(L, S, self.cap16, dtype=torch.int32, device=dev)
        self.t_ema16 = torch.zeros(L, S, self.cap16, dtype=torch.float32, device=dev)
        self.t_n8 = torch.zeros(L, S, dtype=torch.int32, device=dev)
        self.t_n16 = torch.zeros_like(self.t_n8)
        self.t_t = torch.zeros_like(self.t_n8)
        self.t_status = torch.zeros(1, dtype=torch.int32, device=dev)
        for f in _CACHE_FIELDS:
            assert getattr(self, "t_" + f).numel() * getattr(self, "t_" + f).element_size() \
                == getattr(sizes, f), f
        self.cache = ConfCache(*[_ptr(getattr(self, "t_" + f)) for f in _CACHE_FIELDS])
        self.ws = torch.zeros(max(ws.value, 256), dtype=torch.uint8, device=dev)
        self.reset()

    def layer_view(self, l0: int, nl: int) -> "Engine":
        """Layers l0 .. l0+nl-1 of this cache as a cache of its own (the arrays are
        layer-major, so the view is pointer offsets into the same memory), with a
        workspace of its own, so that calls on two views may run concurrently on
        two streams.  The view's `layer` arguments count from l0, and its
        per-layer inputs (q, k, v, out, budget columns) cover its nl layers."""
        wl = self.wl
        if not (0 <= l0 and nl >= 1 and l0 + nl <= wl.n_layers):
            raise ValueError(f"layers {l0}..{l0 + nl - 1} outside 0..{wl.n_layers - 1}")
        v = Engine.__new__(Engine)
        v.lib, v.device, v.dtype16 = self.lib, self.device, self.dtype16
        v.wl = wl.scaled(n_layers=nl, name=f"{wl.name}_layers{l0}-{l0 + nl - 1}")
        v.p = ConfParams.from_buffer_copy(self.p)
        v.p.n_layers = nl
        v.cap8, v.cap16, v.n_sub = self.cap8, self.cap16, self.n_sub
        per_layer = lambda t: t.numel() // wl.n_layers  # noqa: E731
        for f in _CACHE_FIELDS:
            t = getattr(self, "t_" + f)
            if f == "status":
                setattr(v, "t_" + f, t)
            elif t.dim() == 1:
                n = per_layer(t)
                setattr(v, "t_" + f, t[l0 * n:(l0 + nl) * n])
            else:
                setattr(v, "t_" + f, t[l0:l0 + nl])
        v.cache = ConfCache(*[_ptr(getattr(v, "t_" + f)) for f in _CACHE_FIELDS])
        ws = c_size_t()
        _check(v.lib.conf_workspace_bytes(ctypes.byref(v.p), ctypes.byref(ws)), "workspace")
        v.ws = torch.zeros(max(ws.value, 256), dtype=torch.uint8, device=v.device)
        return v

    # -- helpers ------------------------------------------------------------
    def _stream(self):
        return c_void_p(torch.cuda.current_stream(self.device).cuda_stream)

    def _expect(self, t: torch.Tensor, shape, dtype, name):
        if t.device != self.device or t.dtype != dtype or tuple(t.shape) != tuple(shape) \
                or not t.is_contiguous():
            raise ValueError(f"{name}: want {dtype} {tuple(shape)} contiguous on {self.device}, "
                             f"got {t.dtype} {tuple(t.shape)} on {t.device}")

    def _layer_shape(self, layer, *tail):
        return tail if layer >= 0 else (self.wl.n_layers, *tail)

    # -- C-ABI calls ---------------------------------------------------------
    def reset(self):
        _check(self.lib.conf_cache_reset(ctypes.byref(self.p), ctypes.byref(self.cache),
                                         self._stream()), "conf_cache_reset")

    def ingest(self, layer: int, k_pre: torch.Tensor, v_pre: torch.Tensor):
        wl = self.wl
        L0 = k_pre.shape[-2]
        shp = self._layer_shape(layer, wl.batch, wl.n_kv_heads, L0, wl.head_dim)
        self._expect(k_pre, shp, self.dtype16, "k_pre")
        self._expect(v_pre, shp, self.dtype16, "v_pre")
        _check(self.lib.conf_cache_ingest(ctypes.byref(self.p), ctypes.byref(self.cache), layer,
                                          _ptr(k_pre), _ptr(v_pre), L0, _ptr(self.ws),
                                          self._stream()), "conf_cache_ingest")

    def confidence(self, logits: torch.Tensor, c=None, budget=None):
        wl = self.wl
        self._expect(logits, (wl.batch, wl.vocab), torch.float32, "logits")
        c = torch.empty(wl.batch, dtype=torch.float32, device=self.device) if c is None else c
        budget = torch.empty(wl.batch, wl.n_layers, dtype=torch.int32, device=self.device) \
            if budget is None else budget
        self._expect(c, (wl.batch,), torch.float32, "c")
        self._expect(budget, (wl.batch, wl.n_layers), torch.int32, "budget")
        _check(self.lib.conf_confidence(ctypes.byref(self.p), _ptr(logits), _ptr(c), _ptr(budget),
                                        _ptr(self.ws), self._stream()), "conf_confidence")
        return c, budget

    def _attention(self, layer, q, k_new, v_new, out, fn, name):
        wl = self.wl
        self._expect(q, self._layer_shape(layer, wl.batch, wl.n_q_heads, wl.head_dim),
                     self.dtype16, "q")
        kv = self._layer_shape(layer, wl.batch, wl.n_kv_heads, wl.head_dim)
        self._expect(k_new, kv, self.dtype16, "k_new")
        self._expect(v_new, kv, self.dtype16, "v_new")
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=self.device)
        self._expect(out, q.shape, torch.float32, "out")
        _check(fn(ctypes.byref(self.p), ctypes.byref(self.cache), layer, _ptr(q), _ptr(k_new),
                  _ptr(v_new), _ptr(out), _ptr(self.ws), self._stream()), name)
        return out

    def decode_attn(self, layer: int, q, k_new, v_new, out=None):
        return self._attention(layer, q, k_new, v_new, out, self.lib.conf_decode_attn,
                               "conf_decode_attn")

    def attend(self, layer: int, q, k_new, v_new, out=None):
        """conf_attend: the attention without its EMA update, which the next
        ema_evict_compact on the same layers applies."""
        return self._attention(layer, q, k_new, v_new, out, self.lib.conf_attend, "conf_attend")

    def ema_evict_compact(self, layer: int, budget):
        wl = self.wl
        self._expect(budget, (wl.batch, wl.n_layers), torch.int32, "budget")
        _check(self.lib.conf_ema_evict_compact(ctypes.byref(self.p), ctypes.byref(self.cache),
                                               layer, _ptr(budget), _ptr(self.ws), self._stream()),
               "conf_ema_evict_compact")

    def trim_evict_compact(self, layer: int, budget, log_beta):
        """conf_trim_evict_compact: after attend, the new token takes ln(beta)
        (fp32 [L][B], or [B] for one layer) and each (layer, sequence) keeps its
        budget[b][l] tokens of largest (t - pos) * ln(beta)."""
        wl = self.wl
        self._expect(budget, (wl.batch, wl.n_layers), torch.int32, "budget")
        self._expect(log_beta, self._layer_shape(layer, wl.batch), torch.float32, "log_beta")
        _check(self.lib.conf_trim_evict_compact(ctypes.byref(self.p), ctypes.byref(self.cache),
                                                layer, _ptr(budget), _ptr(log_beta),
                                                _ptr(self.ws), self._stream()),
               "conf_trim_evict_compact")

    def _arkv(self, fn, name, layer, budget, n_orig):
        wl = self.wl
        self._expect(budget, (wl.batch, wl.n_layers), torch.int32, "budget")
        self._expect(n_orig, (wl.batch, wl.n_layers), torch.int32, "n_orig")
        _check(fn(ctypes.byref(self.p), ctypes.byref(self.cache), layer, _ptr(budget),
                  _ptr(n_orig), _ptr(self.ws), self._stream()), name)

    def arkv_evict_compact(self, layer: int, budget, n_orig):
        """conf_arkv_evict_compact (after decode_attn): keep budget[b][l] tokens by the
        heavy-hitter EMA, then quantise the lowest-ranked Originals beyond n_orig."""
        self._arkv(self.lib.conf_arkv_evict_compact, "conf_arkv_evict_compact", layer, budget,
                   n_orig)

    def arkv_ema_evict_compact(self, layer: int, budget, n_orig):
        """conf_arkv_ema_evict_compact (after attend): the score EMA, then the same."""
        self._arkv(self.lib.conf_arkv_ema_evict_compact, "conf_arkv_ema_evict_compact", layer,
                   budget, n_orig)

    def arkv_prefill_stats(self, layer: int, q_probe, k_pre, conc=None):
        """conf_arkv_prefill_stats: the concentration of each (layer, sequence)'s prefill
        attention (q_probe 16-bit [L][B][Hq][d] or [B][Hq][d], k_pre as for ingest);
        conc fp32 [L][B], the selected layers' rows written."""
        wl = self.wl
        L0 = k_pre.shape[-2]
        self._expect(q_probe, self._layer_shape(layer, wl.batch, wl.n_q_heads, wl.head_dim),
                     self.dtype16, "q_probe")
        self._expect(k_pre, self._layer_shape(layer, wl.batch, wl.n_kv_heads, L0, wl.head_dim),
                     self.dtype16, "k_pre")
        if conc is None:
            conc = torch.zeros(wl.n_layers, wl.batch, dtype=torch.float32, device=self.device)
        self._expect(conc, (wl.n_layers, wl.batch), torch.float32, "conc")
        _check(self.lib.conf_arkv_prefill_stats(ctypes.byref(self.p), layer, _ptr(q_probe),
                                                _ptr(k_pre), L0, _ptr(conc), _ptr(self.ws),
                                                self._stream()), "conf_arkv_prefill_stats")
        return conc

    def arkv_orig_budgets(self, conc, n_orig=None):
        """conf_arkv_orig_budgets: n_orig int32 [B][L] from conc fp32 [L][B]."""
        wl = self.wl
        self._expect(conc, (wl.n_layers, wl.batch), torch.float32, "conc")
        if n_orig is None:
            n_orig = torch.empty(wl.batch, wl.n_layers, dtype=torch.int32, device=self.device)
        self._expect(n_orig, (wl.batch, wl.n_layers), torch.int32, "n_orig")
        _check(self.lib.conf_arkv_orig_budgets(ctypes.byref(self.p), _ptr(conc), _ptr(n_orig),
                                               self._stream()), "conf_arkv_orig_budgets")
        return n_orig

    def set_retention(self, layer: int, log_beta):
        """conf_cache_set_retention: ln(beta) of the prefill, fp32 [L][B][L0] or
        [B][L0] for one layer, right after ingest."""
        wl = self.wl
        L0 = int(log_beta.shape[-1])
        self._expect(log_beta, self._layer_shape(layer, wl.batch, L0), torch.float32, "log_beta")
        _check(self.lib.conf_cache_set_retention(ctypes.byref(self.p), ctypes.byref(self.cache),
                                                 layer, _ptr(log_beta), L0, self._stream()),
               "conf_cache_set_retention")

    def rank_evict(self, layer: int, budget, keep=None):
        wl = self.wl
        self._expect(budget, (wl.batch, wl.n_layers), torch.int32, "budget")
        if keep is None:
            keep = torch.zeros(wl.n_layers, self.n_sub, self.cap8 + self.cap16, dtype=torch.uint8,
                               device=self.device)
        self._expect(keep, (wl.n_layers, self.n_sub, self.cap8 + self.cap16), torch.uint8, "keep")
        _check(self.lib.conf_rank_evict(ctypes.byref(self.p), ctypes.byref(self.cache), layer,
                                        _ptr(budget), _ptr(keep), _ptr(self.ws), self._stream()),
               "conf_rank_evict")
        return keep

    def compact_demote(self, layer: int, keep):
        wl = self.wl
        self._expect(keep, (wl.n_layers, self.n_sub, self.cap8 + self.cap16), torch.uint8, "keep")
        _check(self.lib.conf_compact_demote(ctypes.byref(self.p), ctypes.byref(self.cache), layer,
                                            _ptr(keep), _ptr(self.ws), self._stream()),
               "conf_compact_demote")

    def evict_compact(self, layer: int, budget):
        wl = self.wl
        self._expect(budget, (wl.batch, wl.n_layers), torch.int32, "budget")
        _check(self.lib.conf_evict_compact(ctypes.byref(self.p), ctypes.byref(self.cache), layer,
                                           _ptr(budget), _ptr(self.ws), self._stream()),
               "conf_evict_compact")

    def step(self, logits, q, k_new, v_new, out=None, c=None, budget=None, static=False):
        """conf_step (static=False, this engine's workspace) or conf_step_static (the
        library's own static scratch; shapes beyond it raise ConfKVError)."""
        wl = self.wl
        self._expect(logits, (wl.batch, wl.vocab), torch.float32, "logits")
        self._expect(q, (wl.n_layers, wl.batch, wl.n_q_heads, wl.head_dim), self.dtype16, "q")
        kv = (wl.n_layers, wl.batch, wl.n_kv_heads, wl.head_dim)
        self._expect(k_new, kv, self.dtype16, "k_new")
        self._expect(v_new, kv, self.dtype16, "v_new")
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=self.device)
        if c is None:
            c = torch.empty(wl.batch, dtype=torch.float32, device=self.device)
        if budget is None:
            budget = torch.empty(wl.batch, wl.n_layers, dtype=torch.int32, device=self.device)
        self._expect(out, q.shape, torch.float32, "out")
        self._expect(c, (wl.batch,), torch.float32, "c")
        self._expect(budget, (wl.batch, wl.n_layers), torch.int32, "budget")
        if static:
            _check(self.lib.conf_step_static(ctypes.byref(self.p), ctypes.byref(self.cache),
                                             _ptr(logits), _ptr(q), _ptr(k_new), _ptr(v_new),
                                             _ptr(out), _ptr(c), _ptr(budget), self._stream()),
                   "conf_step_static")
        else:
            _check(self.lib.conf_step(ctypes.byref(self.p), ctypes.byref(self.cache),
                                      _ptr(logits), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out),
                                      _ptr(c), _ptr(budget), _ptr(self.ws), self._stream()),
                   "conf_step")
        return out, c, budget

    def export(self, layer: int, seq: int) -> dict:
        """One (layer, sequence) as host numpy arrays, slot order, occupied slots only.
        Head-wise, `seq` is the (sequence, KV head) pair b * Hkv + h and the
        arrays hold that one head."""
        wl = self.wl
        H, D = (1 if wl.headwise else wl.n_kv_heads), wl.head_dim
        k8 = torch.empty(self.cap8, H, D, dtype=torch.int8, device=self.device)
        v8 = torch.empty_like(k8)
        k16 = torch.empty(self.cap16, H, D, dtype=torch.int16, device=self.device)
        v16 = torch.empty_like(k16)
        _check(self.lib.conf_cache_export(ctypes.byref(self.p), ctypes.byref(self.cache), layer,
                                          seq, _ptr(k8), _ptr(v8), _ptr(k16), _ptr(v16),
                                          self._stream()), "conf_cache_export")
        torch.cuda.synchronize(self.device)
        n8 = int(self.t_n8[layer, seq])
        n16 = int(self.t_n16[layer, seq])
        return dict(
            n8=n8, n16=n16, t=int(self.t_t[layer, seq]),
            k8=k8[:n8].cpu().numpy(), v8=v8[:n8].cpu().numpy(),
            k16=k16[:n16].cpu().numpy().view("uint16"), v16=v16[:n16].cpu().numpy().view("uint16"),
            pos8=self.t_pos8[layer, seq, :n8].cpu().numpy(),
            ema8=self.t_ema8[layer, seq, :n8].cpu().numpy(),
            pos16=self.t_pos16[layer, seq, :n16].cpu().numpy(),
            ema16=self.t_ema16[layer, seq, :n16].cpu().numpy(),
            k_amax=self.t_k_amax.view(wl.n_layers, self.n_sub, H, D)[layer, seq].cpu().numpy(),
            v_amax=self.t_v_amax.view(wl.n_layers, self.n_sub, H, D)[layer, seq].cpu().numpy(),
        )

    def status(self) -> int:
        return int(self.t_status[0])
