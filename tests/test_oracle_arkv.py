"""ARKV's three-state cache, as the oracle runs it.

The ARKV page, Methodology: Original / Quantized (FP8) / Evicted tokens, ranked
by a heavy-hitter score (mean and variance of attention over heads).  Pins: the
e4m3 codec against the format's closed forms and against PyTorch's own
float8_e4m3fn rounding; the quantiser and its requantisation in closed form;
the score in closed form; and on random runs the invariants that fix the three
states (exactly min(n, N) tokens kept, at most N_O Original unless protected,
protected tokens Original, quantised tokens the lowest-ranked Original ones).
The prefill phase's attention statistics (entropy, variance, kurtosis of the
weights) are pinned to closed forms and to scipy's own routines, and the layer
budgets to their endpoints and monotonicity.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from oracle import (FP8_MAX, OracleParams, arkv_stat, arkv_step, encode16, fp8_decode,
                    fp8_encode, ingest_fp8, quant_codes_fp8, requant_codes_fp8)


def test_fp8_decode_closed_forms():
    c = np.array([0x7E, 0x08, 0x07, 0x01, 0x38, 0x3C, 0xB8, 0x00, 0x77], np.uint8)
    want = [448.0, 2.0 ** -6, 7 * 2.0 ** -9, 2.0 ** -9, 1.0, 1.5, -1.0, 0.0, 240.0]
    assert fp8_decode(c).tolist() == want
    pos = fp8_decode(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)                 # codes 0 .. 0x7e increase strictly
    assert np.signbit(fp8_decode(np.array([0x80], np.uint8)))[0]


def test_fp8_encode_round_trips_every_code():
    codes = np.concatenate([np.arange(0x7F), np.arange(0x80, 0xFF)]).astype(np.uint8)
    back = fp8_encode(fp8_decode(codes).astype(np.float32)).view(np.uint8)
    assert np.array_equal(back, codes)


def test_fp8_encode_matches_torch_float8_e4m3fn():
    rng = np.random.default_rng(21)
    x = np.concatenate([
        rng.uniform(-448, 448, 4000), rng.normal(0, 1, 4000), rng.normal(0, 1e-2, 2000),
        # every midpoint between neighbouring codes (ties go to the even code)
        (fp8_decode(np.arange(0x7E)) + fp8_decode(np.arange(1, 0x7F))) / 2,
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = fp8_encode(x).view(np.uint8)
    assert np.array_equal(got, ref)


def test_fp8_quantiser_closed_forms():
    amax = np.float32(3.5)
    s = np.float32(amax / np.float32(FP8_MAX))
    codes = quant_codes_fp8(np.array([3.5, -3.5, 1.75, 0.0], np.float32), s).view(np.uint8)
    assert codes.tolist() == [0x7E, 0xFE, 0x76, 0x00]      # 448, -448, 224, 0
    assert quant_codes_fp8(np.array([1.0], np.float32), np.float32(0)).tolist() == [0]
    # doubling the scale halves every value that stays representable
    c = np.array([0x7E, 0x76, 0x50], np.uint8).view(np.int8)
    half = requant_codes_fp8(c, s, np.float32(2 * s))
    assert np.array_equal(fp8_decode(half), fp8_decode(c) / 2)


def test_heavy_hitter_score_closed_form():
    p = np.array([[0.2, 0.5], [0.4, 0.5], [0.6, 0.5], [0.8, 0.5]])   # Hq = 4, two KV heads
    s = arkv_stat(p, group=2)
    assert abs(s[0] - (0.5 + 0.04)) < 1e-15                           # m = (0.3, 0.7)
    assert s[1] == 0.5                                                # equal heads: no variance


def _prm(**kw):
    base = dict(n_layers=1, n_q_heads=4, n_kv_heads=2, head_dim=16, dtype16="bf16",
                window=12, protect=3, n_high=16, n_low=16, pyramid=False)
    base.update(kw)
    return OracleParams(**base)


def _run(seed, prm, N, N_O, L0, steps):
    rng = np.random.default_rng(seed)
    H, d = prm.n_kv_heads, prm.head_dim
    k = encode16(rng.standard_normal((H, L0, d)), "bf16")
    v = encode16(rng.standard_normal((H, L0, d)), "bf16")
    st = ingest_fp8(k, v, prm.window, "bf16")
    for _ in range(steps):
        q = encode16(rng.standard_normal((prm.n_q_heads, d)) * 2, "bf16")
        kn = encode16(rng.standard_normal((H, d)), "bf16")
        vn = encode16(rng.standard_normal((H, d)), "bf16")
        n_before = st.n
        orig_before = set(st.pos[~st.is8].tolist()) | {st.t + 1}
        r = arkv_step(st, q, kn, vn, N, N_O, prm)
        yield st, r, n_before, orig_before


def test_three_states_invariants():
    prm = _prm()
    for seed in range(6):
        N, N_O = 16, 9 + seed % 4
        for st, r, n_before, orig_before in _run(seed, prm, N, N_O, 30, 40):
            assert st.n == min(n_before + 1, N)
            prot = st.pos > st.t - prm.protect
            assert not st.is8[prot].any()                     # protected tokens stay Original
            n_orig = int((~st.is8).sum())
            assert n_orig <= N_O or (~st.is8 <= prot).all()
            # the quantised ones were Original and rank below every unprotected Original left
            e32 = st.ema.astype(np.float32)
            left = [(e32[i], st.pos[i]) for i in np.flatnonzero(~st.is8 & ~prot)]
            for p in r["demoted"]:
                assert p in orig_before
                i = int(np.flatnonzero(st.pos == p)[0])
                assert st.is8[i]
                assert all((e32[i], p) < x for x in left)


def test_no_quantisation_when_every_kept_token_fits_original():
    """N_O >= N and a prefill inside the window: ARKV is plain top-N eviction by the
    heavy-hitter EMA, every token 16-bit."""
    prm = _prm(window=40)
    for st, r, _, _ in _run(7, prm, 16, 16, 30, 30):
        assert not st.is8.any() and not r["demoted"]


def test_ingest_quantises_the_old_prefill_to_fp8():
    prm = _prm()
    rng = np.random.default_rng(3)
    k = encode16(rng.standard_normal((2, 30, 16)), "bf16")
    v = encode16(rng.standard_normal((2, 30, 16)), "bf16")
    st = ingest_fp8(k, v, prm.window, "bf16")
    old = st.pos < 30 - prm.window
    assert st.is8.tolist() == old.tolist()
    K, _ = st.kv_values()
    from oracle import decode16
    x = decode16(k, "bf16").transpose(1, 0, 2)
    # FP8 keeps 3 mantissa bits: relative error at most 2^-4 above the subnormal range
    big = np.abs(x[old]) > st.amax_k * 2.0 ** -6
    rel = np.abs(K[old] - x[old])[big] / np.abs(x[old])[big]
    assert rel.max() <= 2.0 ** -4
    assert np.array_equal(K[~old], x[~old])


# ---------------------------------------------------------------- prefill statistics
def test_weight_stats_uniform_and_one_hot_closed_forms():
    for L0 in (2, 7, 1946):
        u = O.attention_weights_stats(np.full(L0, 1.0 / L0))
        assert u["H_hat"] == pytest.approx(1.0, abs=1e-12)
        assert u["v_hat"] == pytest.approx(0.0, abs=1e-15) and u["k_hat"] == 0.0
        assert u["conc"] == pytest.approx(0.0, abs=1e-12)
        e = np.zeros(L0)
        e[L0 // 3] = 1.0
        o = O.attention_weights_stats(e)
        s2 = (L0 - 1) / L0
        s4 = ((L0 - 1) / L0) ** 4 + (L0 - 1) / L0 ** 4
        kurt = L0 * s4 / s2 ** 2
        assert o["H_hat"] == 0.0
        assert o["v_hat"] == pytest.approx(1.0, rel=1e-12)
        assert o["kurtosis"] == pytest.approx(kurt, rel=1e-12)
        assert o["k_hat"] == pytest.approx(math.log(kurt) / math.log(L0), rel=1e-12)


def test_weight_stats_two_level_closed_form():
    L0, k, a = 500, 7, 0.1
    b = (1.0 - k * a) / (L0 - k)
    p = np.full(L0, b)
    p[:k] = a
    H = -(k * a * math.log(a) + (L0 - k) * b * math.log(b))
    da, db = a - 1 / L0, b - 1 / L0
    s2 = k * da ** 2 + (L0 - k) * db ** 2
    s4 = k * da ** 4 + (L0 - k) * db ** 4
    r = O.attention_weights_stats(p)
    assert r["H_hat"] == pytest.approx(H / math.log(L0), rel=1e-12)
    assert r["v_hat"] == pytest.approx(L0 * s2 / (L0 - 1), rel=1e-12)
    assert r["kurtosis"] == pytest.approx(L0 * s4 / s2 ** 2, rel=1e-10)


def test_weight_stats_agree_with_scipy():
    """scipy's own entropy and (Pearson, population) kurtosis of the same weights."""
    import scipy.stats as ss
    rng = np.random.default_rng(3)
    for L0 in (64, 1000, 4096):
        z = rng.standard_normal(L0) * rng.uniform(0.5, 4.0)
        p = np.exp(z - z.max())
        p /= p.sum()
        r = O.attention_weights_stats(p)
        assert r["H_hat"] == pytest.approx(ss.entropy(p) / math.log(L0), rel=1e-12)
        assert r["kurtosis"] == pytest.approx(ss.kurtosis(p, fisher=False, bias=True), rel=1e-9)
        assert r["v_hat"] == pytest.approx(np.var(p) * L0 ** 2 / (L0 - 1), rel=1e-9)


def test_sharper_attention_is_more_concentrated():
    rng = np.random.default_rng(5)
    z = rng.standard_normal(800)
    prev = -1.0
    for beta in (0.0, 0.5, 1.0, 2.0, 4.0, 8.0, 16.0):
        p = np.exp(beta * z - (beta * z).max())
        p /= p.sum()
        c = O.attention_weights_stats(p)["conc"]
        assert c > prev - 1e-12
        prev = c
    assert prev > 0.5


def test_prefill_concentration_heads_and_group_mapping():
    """q = 0 gives uniform attention (0); a query aligned with one key of large norm
    gives nearly one-hot attention; each query head reads KV head h // group."""
    rng = np.random.default_rng(9)
    Hkv, group, L0, d = 2, 3, 300, 64
    K = rng.standard_normal((Hkv, L0, d))
    K[1, 17] = 40.0 * np.ones(d) / math.sqrt(d)          # a sharp key in KV head 1 only
    q = np.zeros((Hkv * group, d))
    q[3:] = np.ones(d) / math.sqrt(d) * 10.0              # heads 3..5 read KV head 1
    r = O.arkv_prefill_concentration(q, K, group)
    assert np.allclose(r[:3], 0.0, atol=1e-12)            # heads 0..2: q = 0, uniform
    assert np.all(r[3:6] > 0.9)
    assert r[6] == pytest.approx(r[:6].mean())
    # the same sharp key in KV head 0 instead: heads 3..5 see no sharp key
    K2 = K.copy()
    K2[0, 17], K2[1, 17] = K[1, 17], K[0, 17]
    r2 = O.arkv_prefill_concentration(q, K2, group)
    assert np.all(r2[3:6] < 0.2)


def test_orig_budgets_endpoints_monotone_and_floor():
    N, P = 2048, 32
    c = np.array([0.02, 0.30, 0.11, 0.30, 0.05, 0.21], np.float32)
    n = O.arkv_orig_budgets(c, N, P)
    assert n[0] == math.ceil(np.float32(0.75) * N)                   # least concentrated
    assert n[1] == n[3] == math.ceil(np.float32(0.95) * np.float32(N))  # most concentrated
    order = np.argsort(c, kind="stable")
    assert np.all(np.diff(n[order]) >= 0)                            # monotone in c
    same = O.arkv_orig_budgets(np.full(4, 0.4, np.float32), N, P)
    assert np.all(same == math.ceil(np.float32(0.85) * N))
    tiny = O.arkv_orig_budgets(c, 20, 32)                            # never below P
    assert np.all(tiny == 32)
