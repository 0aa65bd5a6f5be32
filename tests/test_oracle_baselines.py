"""The baseline policies the pages compare CONF-KV with, as the oracle runs them.

CONF-KV explainer, Problem statement (sliding-window eviction) and Experimental
results (full KV).  Pins: a sliding window holds exactly the positions
(t - W, t], all 16-bit; full KV holds every position, all 16-bit; a window
ingest keeps the newest W prefill tokens bit for bit; full-KV attention is the
textbook softmax attention over every token.
"""
import numpy as np

from oracle import OracleParams, decode16, encode16, ingest, step_layer


def _prm(**kw):
    base = dict(n_layers=1, n_q_heads=4, n_kv_heads=2, head_dim=16, dtype16="f16",
                window=10, protect=10, n_high=10, n_low=10, pyramid=False)
    base.update(kw)
    return OracleParams(**base)


def _kv(rng, prm, n):
    k = encode16(rng.standard_normal((prm.n_kv_heads, n, prm.head_dim)), prm.dtype16)
    v = encode16(rng.standard_normal((prm.n_kv_heads, n, prm.head_dim)), prm.dtype16)
    return k, v


def _step(st, prm, rng, N):
    q = encode16(rng.standard_normal((prm.n_q_heads, prm.head_dim)), prm.dtype16)
    k, v = _kv(rng, prm, 1)
    return step_layer(st, q, k[:, 0], v[:, 0], N, prm)


def test_sliding_window_keeps_exactly_the_newest_w():
    rng = np.random.default_rng(3)
    prm = _prm()
    W = prm.window
    k, v = _kv(rng, prm, 37)
    st = ingest(k, v, W, prm.dtype16, drop_old=True)
    assert st.pos.tolist() == list(range(37 - W, 37)) and not st.is8.any()
    for _ in range(25):
        _step(st, prm, rng, W)
        assert st.pos.tolist() == list(range(st.t - W + 1, st.t + 1))
        assert not st.is8.any()


def test_window_ingest_is_the_newest_w_bits():
    rng = np.random.default_rng(4)
    prm = _prm(dtype16="bf16")
    W = prm.window
    k, v = _kv(rng, prm, 29)
    st = ingest(k, v, W, prm.dtype16, drop_old=True)
    assert np.array_equal(st.k16, k[:, 29 - W:].transpose(1, 0, 2))
    assert np.array_equal(st.v16, v[:, 29 - W:].transpose(1, 0, 2))
    assert st.t == 28 and not st.amax_k.any() and not st.amax_v.any()
    short = ingest(k[:, :7], v[:, :7], W, prm.dtype16, drop_old=True)
    assert short.pos.tolist() == list(range(7))


def test_full_kv_keeps_every_token_in_16_bits():
    rng = np.random.default_rng(5)
    prm = _prm(window=1000, protect=1, n_high=10 ** 9, n_low=10 ** 9)
    k, v = _kv(rng, prm, 23)
    st = ingest(k, v, prm.window, prm.dtype16)
    for _ in range(20):
        _step(st, prm, rng, 10 ** 9)
    assert st.pos.tolist() == list(range(43)) and not st.is8.any()


def test_full_kv_attention_is_plain_softmax_attention():
    rng = np.random.default_rng(6)
    prm = _prm(window=1000, protect=1, n_high=10 ** 9, n_low=10 ** 9)
    k, v = _kv(rng, prm, 31)
    st = ingest(k, v, prm.window, prm.dtype16)
    q = encode16(rng.standard_normal((prm.n_q_heads, prm.head_dim)), prm.dtype16)
    kn, vn = _kv(rng, prm, 1)
    r = step_layer(st, q, kn[:, 0], vn[:, 0], 10 ** 9, prm)
    K = decode16(np.concatenate([k, kn], axis=1), prm.dtype16).astype(np.float64)  # [H, n, d]
    V = decode16(np.concatenate([v, vn], axis=1), prm.dtype16).astype(np.float64)
    Q = decode16(q, prm.dtype16).astype(np.float64)
    g = prm.n_q_heads // prm.n_kv_heads
    for h in range(prm.n_q_heads):
        s = K[h // g] @ Q[h] / np.sqrt(prm.head_dim)
        p = np.exp(s - s.max())
        p /= p.sum()
        np.testing.assert_allclose(r["o"][h], p @ V[h // g], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# Retention eviction (TRIM-KV page, Methodology: retention gate; inference and
# eviction): the current score is beta^(t - i); at the limit M the lowest goes.
# ----------------------------------------------------------------------------
from oracle import retention_scores, trim_step  # noqa: E402


def _trim_run(rng, prm, M, betas, steps):
    """From an empty cache; returns the state and every token's beta by position."""
    from oracle import LayerSeqState
    st = LayerSeqState(prm.n_kv_heads, prm.head_dim, prm.dtype16)
    for i in range(steps):
        q = encode16(rng.standard_normal((prm.n_q_heads, prm.head_dim)), prm.dtype16)
        k, v = _kv(rng, prm, 1)
        trim_step(st, q, k[:, 0], v[:, 0], np.log(np.float32(betas[i])), M, prm)
    return st


def test_retention_keeps_the_m_largest_beta_powers_float64():
    """Brute force: after every step the kept set is the M tokens with the largest
    beta_i^(t-i) computed in float64 (betas spread so that no two are close)."""
    rng = np.random.default_rng(7)
    prm = _prm()
    M, steps = 12, 60
    betas = rng.permutation(np.linspace(0.05, 0.999, steps)).astype(np.float32)
    from oracle import LayerSeqState
    st = LayerSeqState(prm.n_kv_heads, prm.head_dim, prm.dtype16)
    for t in range(steps):
        q = encode16(rng.standard_normal((prm.n_q_heads, prm.head_dim)), prm.dtype16)
        k, v = _kv(rng, prm, 1)
        trim_step(st, q, k[:, 0], v[:, 0], np.log(betas[t]), M, prm)
        if t + 1 <= M:
            assert st.pos.tolist() == list(range(t + 1))
            prev = st.pos.tolist()
            continue
        # the survivors of the previous step plus the new token, best M of them
        cand = set(prev) | {t}
        val = {i: np.float64(betas[i]) ** (t - i) for i in cand}
        want = sorted(cand, key=lambda i: (-val[i], -i))[:M]
        assert sorted(st.pos.tolist()) == sorted(want), t
        prev = st.pos.tolist()
    assert st.n == M and not st.is8.any()


def test_retention_with_beta_one_is_a_sliding_window():
    """beta = 1 for every token: all scores are 0, the newer wins every tie, so the
    cache is the newest M positions."""
    rng = np.random.default_rng(8)
    prm = _prm()
    st = _trim_run(rng, prm, 9, np.ones(40, np.float32), 40)
    assert st.pos.tolist() == list(range(31, 40))


def test_retention_scores_closed_form():
    with np.errstate(divide="ignore"):
        lb = np.log(np.array([0.5, 0.25, 1.0, 0.0], np.float32))   # ln 0 = -inf
    s = retention_scores(lb, np.array([3, 4, 0, 5]), 5)
    assert s[0] == np.float32(2) * np.float32(np.log(np.float32(0.5)))
    assert s[1] == np.float32(np.log(np.float32(0.25)))
    assert s[2] == 0 and s[3] == 0            # beta = 1 never decays; the newest scores 0
