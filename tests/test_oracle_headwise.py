"""Head-wise keep sets, as the oracle runs them.

CONF-KV explainer, Significance and claims: the method composes with head-wise
allocation.  Pins: with one KV head the head-wise step is the per-sequence step;
with identical heads every head keeps what the per-sequence step keeps at budget
N; closed forms fix the shared e_max, the shared budget of Hkv * N pairs, each
head's own protected window and the tie order (score, position, head); and on
random caches the kept pairs are exactly the best ones.
"""
import numpy as np

from oracle import (LayerSeqState, OracleParams, composite_scores, encode16, headwise_step,
                    ingest, joint_keep, step_layer)


def _prm(**kw):
    base = dict(n_layers=1, n_q_heads=6, n_kv_heads=3, head_dim=16, dtype16="bf16",
                window=9, protect=3, n_high=14, n_low=20, pyramid=False)
    base.update(kw)
    return OracleParams(**base)


def _split(st: LayerSeqState, h: int) -> LayerSeqState:
    """KV head h of a cache, as a cache of its own."""
    one = LayerSeqState(1, st.k16.shape[2], st.dtype16)
    for f in ("pos", "is8", "ema"):
        setattr(one, f, getattr(st, f).copy())
    for f in ("k16", "v16", "k8", "v8"):
        setattr(one, f, getattr(st, f)[:, h:h + 1].copy())
    one.amax_k = st.amax_k[h:h + 1].copy()
    one.amax_v = st.amax_v[h:h + 1].copy()
    one.t = st.t
    return one


def _same(a: LayerSeqState, b: LayerSeqState):
    assert a.t == b.t
    assert np.array_equal(a.pos, b.pos) and np.array_equal(a.is8, b.is8)
    for f in ("k16", "v16"):
        assert np.array_equal(getattr(a, f)[~a.is8], getattr(b, f)[~b.is8])
    for f in ("k8", "v8"):
        assert np.array_equal(getattr(a, f)[a.is8], getattr(b, f)[b.is8])
    assert np.array_equal(a.amax_k, b.amax_k) and np.array_equal(a.amax_v, b.amax_v)
    assert np.array_equal(a.ema, b.ema)


def test_one_kv_head_is_the_per_sequence_step():
    rng = np.random.default_rng(11)
    prm = _prm(n_q_heads=4, n_kv_heads=1)
    k = encode16(rng.standard_normal((1, 30, 16)), "bf16")
    v = encode16(rng.standard_normal((1, 30, 16)), "bf16")
    ref = ingest(k, v, prm.window, "bf16")
    heads = [_split(ref, 0)]
    for step in range(40):
        q = encode16(rng.standard_normal((4, 16)), "bf16")
        kn = encode16(rng.standard_normal((1, 16)), "bf16")
        vn = encode16(rng.standard_normal((1, 16)), "bf16")
        N = prm.n_high if step % 9 < 5 else prm.n_low
        r1 = step_layer(ref, q, kn, vn, N, prm)
        r2 = headwise_step(heads, q, kn, vn, N, prm)
        assert np.array_equal(r1["o"], r2["o"])
        _same(heads[0], ref)
    assert ref.is8.any() and ref.n == prm.n_high


def test_identical_heads_keep_what_one_head_keeps():
    """H copies of one head (same keys, values and queries): the joint budget H * N
    splits evenly, each head keeps the per-sequence keep set at budget N."""
    rng = np.random.default_rng(12)
    H, G = 3, 2
    prm = _prm(n_q_heads=H * G, n_kv_heads=H)
    one = _prm(n_q_heads=G, n_kv_heads=1)
    k = encode16(rng.standard_normal((1, 25, 16)), "bf16")
    v = encode16(rng.standard_normal((1, 25, 16)), "bf16")
    ref = ingest(k, v, prm.window, "bf16")
    heads = [_split(ref, 0) for _ in range(H)]
    for step in range(30):
        q1 = encode16(rng.standard_normal((G, 16)), "bf16")
        kn = encode16(rng.standard_normal((1, 16)), "bf16")
        vn = encode16(rng.standard_normal((1, 16)), "bf16")
        N = prm.n_high if step % 7 < 4 else prm.n_low
        step_layer(ref, q1, kn, vn, N, one)
        headwise_step(heads, np.tile(q1, (H, 1)), np.tile(kn, (H, 1)), np.tile(vn, (H, 1)), N,
                      prm)
        for st in heads:
            _same(st, ref)


def test_shared_e_max_and_shared_budget_closed_form():
    """Scores e / e_max with e_max over both heads: head 1's larger EMAs win the
    pairs left after each head's protected newest position (budget 4, two
    protected, two more pairs: head 1 at positions 2 and 1)."""
    e = [np.array([1, 2, 3, 4], np.float32), np.array([10, 20, 30, 40], np.float32)]
    pos = [np.arange(4), np.arange(4)]
    k0, k1 = joint_keep(e, pos, 3, 1, 4, 1.0, 0.0)
    assert k0.tolist() == [False, False, False, True]
    assert k1.tolist() == [False, True, True, True]
    # under the budget nothing is ranked
    assert all(k.all() for k in joint_keep(e, pos, 3, 1, 8, 1.0, 0.0))
    # a budget of the protected pairs alone keeps exactly them
    k0, k1 = joint_keep(e, pos, 3, 2, 4, 1.0, 0.0)
    assert k0.tolist() == k1.tolist() == [False, False, True, True]


def test_ties_go_to_the_newer_position_then_the_higher_head():
    e = [np.full(3, 5, np.float32), np.full(3, 5, np.float32)]
    pos = [np.array([0, 1, 2]), np.array([0, 1, 2])]
    # t = 3 (the newest token sits elsewhere): nothing protected with P = 1, budget 3
    k0, k1 = joint_keep(e, pos, 3, 1, 3, 1.0, 0.0)
    assert k1.tolist() == [False, True, True]
    assert k0.tolist() == [False, False, True]


def test_ragged_heads_keep_the_best_pairs():
    """Random ragged caches: exactly min(n, budget) pairs stay, every protected one
    among them, and no evicted candidate outranks a kept one."""
    rng = np.random.default_rng(13)
    for trial in range(60):
        H = int(rng.integers(1, 6))
        t = int(rng.integers(5, 200))
        P = int(rng.integers(1, 5))
        pos = [np.sort(rng.choice(t + 1, size=int(rng.integers(1, t + 1)), replace=False))
               for _ in range(H)]
        for p in pos:                      # every head holds the newest position
            if p[-1] != t:
                p[-1] = t
        pos = [np.unique(p) for p in pos]
        e = [rng.random(p.size).astype(np.float32) * (h + 1) for h, p in enumerate(pos)]
        if trial % 5 == 0:
            e = [np.round(x * 4) / 4 for x in e]      # many equal scores
        n = sum(p.size for p in pos)
        prot = sum(int((p > t - P).sum()) for p in pos)
        N_total = int(rng.integers(prot, n + 3))
        keeps = joint_keep(e, pos, t, P, N_total, 0.7, 0.3)
        assert sum(int(k.sum()) for k in keeps) == min(n, N_total)
        s = composite_scores(np.concatenate(e), np.concatenate(pos), t, 0.7, 0.3)
        rank = list(zip(s.tolist(), np.concatenate(pos).tolist(),
                        np.concatenate([np.full(p.size, h) for h, p in enumerate(pos)]).tolist()))
        kept = np.concatenate(keeps)
        is_prot = np.concatenate(pos) > t - P
        assert kept[is_prot].all()
        cand = ~is_prot
        if n > N_total and cand.any():
            worst_kept = min((rank[i] for i in np.flatnonzero(kept & cand)), default=None)
            best_gone = max((rank[i] for i in np.flatnonzero(~kept & cand)), default=None)
            if worst_kept is not None and best_gone is not None:
                assert worst_kept > best_gone
