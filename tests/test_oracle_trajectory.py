"""Multi-step invariants of the oracle's decode loop.

CONF-KV explainer, Methodology: adaptive budget selection (the cache grows in
uncertain phases and shrinks in confident ones: a sawtooth), token ranking and
eviction (the protected window P is never evicted), mixed-precision storage
(the newest W positions stay 16-bit); Significance: a no-op on short contexts.
"""
import numpy as np
import pytest

from oracle import (LayerSeqState, OracleParams, budget, confidence, decode_step, encode16,
                    ingest, layer_budget)


def _params(**kw):
    base = dict(n_layers=3, n_q_heads=4, n_kv_heads=2, head_dim=16, dtype16="bf16",
                window=12, protect=6, n_high=20, n_low=32, pyramid=True)
    base.update(kw)
    return OracleParams(**base)


def _inputs(prm, B, step, rng):
    L, Hq, Hkv, d = prm.n_layers, prm.n_q_heads, prm.n_kv_heads, prm.head_dim
    T = 0.5 if (step // 16) % 2 == 0 else 8.0
    logits = rng.standard_normal((B, 500)) * T
    q = encode16(rng.standard_normal((L, B, Hq, d)), prm.dtype16)
    k = encode16(rng.standard_normal((L, B, Hkv, d)), prm.dtype16)
    v = encode16(rng.standard_normal((L, B, Hkv, d)), prm.dtype16)
    return logits, q, k, v


def _check_layout(st, prm):
    t = st.t
    assert len(np.unique(st.pos)) == st.n                     # no duplicates
    assert np.all(np.diff(st.pos) > 0)                        # position order
    window = st.pos > t - prm.window
    assert np.array_equal(~st.is8, window)                    # 16-bit exactly (t-W, t]
    prot = np.arange(max(0, t - prm.protect + 1), t + 1)
    assert np.isin(prot, st.pos).all()                        # protected always present


@pytest.mark.parametrize("prefill", [0, 40])
def test_sawtooth_and_layout_invariants(prefill):
    prm = _params()
    B = 2
    rng = np.random.default_rng(prefill + 1)
    if prefill:
        states = []
        for l in range(prm.n_layers):
            row = []
            for b in range(B):
                k = encode16(rng.standard_normal((prm.n_kv_heads, prefill, prm.head_dim)), "bf16")
                v = encode16(rng.standard_normal((prm.n_kv_heads, prefill, prm.head_dim)), "bf16")
                row.append(ingest(k, v, prm.window, "bf16"))
            states.append(row)
    else:
        states = [[LayerSeqState(prm.n_kv_heads, prm.head_dim, "bf16") for _ in range(B)]
                  for _ in range(prm.n_layers)]
    sizes = np.array([[s.n for s in row] for row in states])
    saw_high = saw_low = False
    for step in range(96):
        logits, q, k, v = _inputs(prm, B, step, rng)
        r = decode_step(states, logits, q, k, v, prm)
        for b in range(B):
            c = confidence(logits[b])["c"]
            assert r["c"][b] == c
            N = budget(c, prm.tau, prm.n_high, prm.n_low)
            saw_high |= N == prm.n_high
            saw_low |= N == prm.n_low
            for l in range(prm.n_layers):
                Nl = layer_budget(N, l, prm.n_layers, True)
                want = min(sizes[l, b] + 1, Nl)               # s_t = min(s_{t-1} + 1, N_t)
                assert states[l][b].n == want
                sizes[l, b] = want
                _check_layout(states[l][b], prm)
    assert saw_high and saw_low                               # budgets flipped


def test_no_op_on_short_context():
    prm = _params(n_layers=1, window=4, protect=2, n_high=50, n_low=60, pyramid=False)
    rng = np.random.default_rng(5)
    states = [[LayerSeqState(2, 16, "bf16")]]
    for step in range(45):
        logits, q, k, v = _inputs(prm, 1, step, rng)
        decode_step(states, logits, q, k, v, prm)
    st = states[0][0]
    assert list(st.pos) == list(range(45))                    # never evicted anything


def test_budget_override_teacher_forcing():
    prm = _params(n_layers=1, pyramid=False)
    rng = np.random.default_rng(6)
    states = [[LayerSeqState(2, 16, "bf16")]]
    for step in range(40):
        logits, q, k, v = _inputs(prm, 1, step, rng)
        decode_step(states, logits, q, k, v, prm, budget_override=[prm.n_high])
    assert states[0][0].n == prm.n_high
