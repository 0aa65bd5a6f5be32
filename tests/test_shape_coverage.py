"""The small parity shapes reach each way the attention keeps a unit's raw scores
(CPU check of the shapes against the attention kernel's LDS budget).

The budget is restated here as the library sizes it: dynamic LDS of 38 KB at
d = 64 and 79360 bytes at d = 128; the query operands take 48 bytes per 32
channels for each of the 4G + 1 lane groups; the rest holds G fp32 rows.  A
change of that sizing makes these checks fail, which is the point: the parity
shapes then have to be re-chosen so that every path is still exercised.
"""
from parity_util import tiny_workloads

TINY = tiny_workloads()
LDS_DYN = {64: 38 * 1024, 128: 79360}
HELD_HALVES = {64: 0, 128: 4}  # window halves a wavefront keeps in registers


def score_cap(D, G):
    qops = 16 * (4 * G + 1) * (D // 32) * 3
    return ((LDS_DYN[D] - qops) // (4 * G) - 1) & ~1


def spill_start(n8, cap):
    c64 = cap & ~63
    return c64 if n8 > c64 else n8 + ((cap - n8) & ~31)


def held(D, n8, nw, cap):
    return nw <= 4 * 32 * HELD_HALVES[D] and spill_start(n8, cap) < n8 + nw


def test_held_window_shape():
    """gqa16_bf16_d128_held: the first step's cache (its INT8 part longer than the
    rows, so INT8 items spill) and every later one (INT8 part within the rows) hold
    their window halves' scores in registers."""
    wl = TINY["gqa16_bf16_d128_held"]
    cap = score_cap(wl.head_dim, wl.group)
    assert cap == 1044
    n8, nw = wl.prefill - wl.window, wl.window
    assert held(wl.head_dim, n8, nw, cap) and spill_start(n8, cap) < n8
    assert nw % 32 != 0  # a ragged last half
    for n in (wl.n_high, wl.n_low + 1):  # the smallest and largest later caches
        n8 = n - wl.window
        assert held(wl.head_dim, n8, nw, cap) and n8 <= spill_start(n8, cap)


def test_window_spill_shape():
    """gqa16_f16_d128_winspill: a window longer than the registers take, whose own
    items spill to the workspace."""
    wl = TINY["gqa16_f16_d128_winspill"]
    cap = score_cap(wl.head_dim, wl.group)
    n8, nw = wl.prefill - wl.window, wl.window
    assert not held(wl.head_dim, n8, nw, cap)
    assert n8 < spill_start(n8, cap) < n8 + nw


def test_d64_spill_shapes():
    """The d = 64 shapes that outgrow the rows keep every spilled score in the
    workspace (no held halves at d = 64)."""
    for name in ("gqa16_bf16_d64_long", "gqa16_bf16_d64_wide"):
        wl = TINY[name]
        cap = score_cap(wl.head_dim, wl.group)
        n8, nw = wl.prefill - wl.window, wl.window
        assert not held(wl.head_dim, n8, nw, cap)
        assert spill_start(n8, cap) < n8 + nw, name
