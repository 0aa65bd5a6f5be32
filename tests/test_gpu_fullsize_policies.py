"""Full-size parity of the later rows on the Qwen-32B-shaped batch-8 cache, on
sampled (layer, sequence) pairs, driven as the benchmark drives them.

  * retention eviction (M = 2048, the bench's `--policy trim`): the steps between
    checked ones run conf_attend + conf_trim_evict_compact; a checked step runs
    the same and compares with the oracle's trim_step from a snapshot (its
    arithmetic is exact, so no teacher forcing of scores is needed);
  * ARKV (N = 2048, per-layer N_O, `--policy arkv`): unchecked steps run
    conf_attend + conf_arkv_ema_evict_compact; a checked step runs
    conf_decode_attn (so that the score EMA can be read) and
    conf_arkv_evict_compact.  Step 0 quantises each layer's prefill Original
    tokens beyond its N_O (several rounds), step 150 is the steady state;
  * head-wise keep sets (`--headwise`): unchecked steps run the bench's launches;
    a checked step runs conf_decode_attn, the confidence, and the joint selection
    with the per-head compaction (fused on even steps, separate on odd ones).
    Step 0 cuts 8 x 32769 (token, head) pairs to 8 x N.
Tolerances are those of the small-shape parity tests.
"""
import numpy as np
import pytest
import torch

import oracle as O
from adaptive_kv_cache_amd import synth
from adaptive_kv_cache_amd.binding import Engine
from adaptive_kv_cache_amd.workloads import WORKLOADS
from parity_util import (assert_same_state, attn_rel_err, bits16, ema_by_pos, kept_positions,
                         oracle_params, to_oracle_state)

pytestmark = pytest.mark.gpu

ATTN_TOL = 2e-3
EMA_RTOL = 1e-5
SEED = 0
BASE = "qwen32b_gqa_b8_32k"
SAMPLES = [(0, 0), (37, 5), (63, 7)]


def _say(*a):
    print(*a, flush=True)


def _ingest(eng, wl, dev, check=None):
    for l in range(wl.n_layers):
        k, v = synth.prefill_kv(wl, l, SEED, device=dev)
        eng.ingest(l, k, v)
        if check is not None:
            check(l, k, v)
        del k, v


def test_full_size_retention_eviction():
    wl = WORKLOADS[BASE].baseline("trim", 64)
    prm = oracle_params(wl)
    dev = torch.device("cuda", 0)
    _say("full size trim: ingest", wl.name)
    eng = Engine(wl, dev)

    def set_beta(l, k, v):
        eng.set_retention(l, synth.log_beta_prefill(wl, l, SEED, device=dev))

    _ingest(eng, wl, dev, set_beta)
    budget = torch.full((wl.batch, wl.n_layers), wl.n_high, dtype=torch.int32, device=dev)
    worst = 0.0
    for step in range(41):
        q = synth.q_new(wl, step, SEED, device=dev)
        k, v = synth.kv_new(wl, step, SEED, device=dev)
        lbn = synth.log_beta_new(wl, step, SEED, device=dev)
        check = step in (0, 1, 40)
        S0 = {s: eng.export(*s) for s in SAMPLES} if check else None
        out = eng.attend(-1, q, k, v)
        eng.trim_evict_compact(-1, budget, lbn)
        if not check:
            continue
        _say("  checking step", step)
        S2 = {s: eng.export(*s) for s in SAMPLES}
        out_h, lb_h = out.cpu().numpy(), lbn.cpu().numpy()
        qb, kb, vb = bits16(q), bits16(k), bits16(v)
        for (l, b) in SAMPLES:
            what = ("trim", step, l, b)
            st = to_oracle_state(S0[(l, b)], wl.dtype16)
            r = O.trim_step(st, qb[l, b], kb[l, b], vb[l, b], float(lb_h[l, b]), wl.n_high, prm)
            err = attn_rel_err(out_h[l, b], r["o"])
            worst = max(worst, err)
            assert err <= ATTN_TOL, (what, err)
            got = to_oracle_state(S2[(l, b)], wl.dtype16)
            assert_same_state(got, st, what=what)
            assert np.array_equal(got.ema, st.ema), what
            assert st.n == wl.n_high
    assert eng.status() == 0
    _say("  worst attention rel err", worst)
    del eng
    torch.cuda.empty_cache()


def test_full_size_arkv():
    wl = WORKLOADS[BASE].baseline("arkv", 160)
    prm = oracle_params(wl)
    dev = torch.device("cuda", 0)
    _say("full size arkv: ingest", wl.name, "W", wl.window, "prefill", wl.prefill)
    eng = Engine(wl, dev)
    # ARKV's prefill phase: each layer's Original budget from its prefill attention
    q0 = synth.q_new(wl, 0, SEED, device=dev)
    conc = torch.zeros(wl.n_layers, wl.batch, dtype=torch.float32, device=dev)
    pre = {}

    def stats(l, k, v):
        eng.arkv_prefill_stats(l, q0[l], k, conc)
        for (sl, b) in SAMPLES:
            if sl == l:
                pre[(l, b)] = bits16(k[b])

    _ingest(eng, wl, dev, check=stats)
    budget = torch.full((wl.batch, wl.n_layers), wl.n_high, dtype=torch.int32, device=dev)
    n_orig = eng.arkv_orig_budgets(conc)
    no_h = n_orig.cpu().numpy()
    conc_h = conc.cpu().numpy()
    qb0 = bits16(q0)
    for (l, b) in SAMPLES:
        ref = O.arkv_prefill_concentration(O.decode16(qb0[l, b], wl.dtype16),
                                           O.decode16(pre[(l, b)], wl.dtype16), wl.group)
        assert abs(float(conc_h[l, b]) - ref[-1]) <= 2e-5, ("prefill concentration", l, b)
    for b in range(wl.batch):
        assert no_h[b].tolist() == O.arkv_orig_budgets(conc_h[:, b], wl.n_high,
                                                       wl.protect).tolist(), ("N_O", b)
    _say("  N_O of sequence 0 over the layers:", sorted(set(no_h[0].tolist())))
    worst = 0.0
    quantised = 0
    for step in range(151):
        q = synth.q_new(wl, step, SEED, device=dev)
        k, v = synth.kv_new(wl, step, SEED, device=dev)
        if step not in (0, 1, 150):
            eng.attend(-1, q, k, v)
            eng.arkv_ema_evict_compact(-1, budget, n_orig)
            continue
        _say("  checking step", step)
        S0 = {s: eng.export(*s) for s in SAMPLES}
        out = eng.decode_attn(-1, q, k, v)
        S1 = {s: eng.export(*s) for s in SAMPLES}
        eng.arkv_evict_compact(-1, budget, n_orig)
        S2 = {s: eng.export(*s) for s in SAMPLES}
        out_h = out.cpu().numpy()
        qb, kb, vb = bits16(q), bits16(k), bits16(v)
        for (l, b) in SAMPLES:
            what = ("arkv", step, l, b)
            st0 = to_oracle_state(S0[(l, b)], wl.dtype16)
            st = O.Fp8State(st0.k16.shape[1], st0.k16.shape[2], st0.dtype16)
            for f in ("pos", "is8", "k16", "v16", "k8", "v8", "ema", "amax_k", "amax_v", "t"):
                setattr(st, f, getattr(st0, f))
            e_gpu = ema_by_pos(S1[(l, b)])
            override = np.array([e_gpu[p] for p in np.append(st.pos, st.t + 1).tolist()],
                                np.float32)
            r = O.arkv_step(st, qb[l, b], kb[l, b], vb[l, b], wl.n_high, int(no_h[b, l]), prm,
                            ema32_override=override)
            err = attn_rel_err(out_h[l, b], r["o"])
            worst = max(worst, err)
            assert err <= ATTN_TOL, (what, err)
            np.testing.assert_allclose(override, r["ema"], rtol=EMA_RTOL, atol=1e-12,
                                       err_msg=str(what))
            assert_same_state(to_oracle_state(S2[(l, b)], wl.dtype16), st, ema_rtol=0, what=what)
            quantised += len(r["demoted"])
            _say(f"    {what}: n={st.n} Original={int((~st.is8).sum())} "
                 f"quantised {len(r['demoted'])} attention rel err {err:.2e}")
    assert eng.status() == 0
    assert quantised > 0
    _say("  worst attention rel err", worst)
    del eng
    torch.cuda.empty_cache()


def test_full_size_headwise():
    wl = WORKLOADS[BASE].headwise_variant()
    H = wl.n_kv_heads
    prm = oracle_params(wl)
    dev = torch.device("cuda", 0)
    _say("full size head-wise: ingest", wl.name, "cap8", wl.cap8)
    eng = Engine(wl, dev)
    _ingest(eng, wl, dev)
    worst = 0.0
    for step in range(67):
        z = synth.logits(wl, step, SEED, device=dev)
        q = synth.q_new(wl, step, SEED, device=dev)
        k, v = synth.kv_new(wl, step, SEED, device=dev)
        if step not in (0, 1, 66):
            eng.attend(-1, q, k, v)
            _, budget = eng.confidence(z)
            eng.ema_evict_compact(-1, budget)
            continue
        _say("  checking step", step)
        subs = [(l, b * H + h) for (l, b) in SAMPLES for h in range(H)]
        S0 = {s: eng.export(*s) for s in subs}
        out = eng.decode_attn(-1, q, k, v)
        S1 = {s: eng.export(*s) for s in subs}
        _, budget = eng.confidence(z)
        fused = step % 2 == 0
        if fused:
            eng.evict_compact(-1, budget)
        else:
            keep = eng.rank_evict(-1, budget)
            eng.compact_demote(-1, keep)
        S2 = {s: eng.export(*s) for s in subs}
        out_h, bud_h = out.cpu().numpy(), budget.cpu().numpy()
        keep_h = None if fused else keep.cpu().numpy()
        qb, kb, vb = bits16(q), bits16(k), bits16(v)
        for (l, b) in SAMPLES:
            what = ("headwise", step, l, b)
            heads = [to_oracle_state(S0[(l, b * H + h)], wl.dtype16) for h in range(H)]
            override = []
            for h, st in enumerate(heads):
                e_gpu = ema_by_pos(S1[(l, b * H + h)])
                override.append(np.array([e_gpu[p] for p in np.append(st.pos, st.t + 1).tolist()],
                                         np.float32))
            r = O.headwise_step(heads, qb[l, b], kb[l, b], vb[l, b], int(bud_h[b, l]), prm,
                                ema32_override=override)
            err = attn_rel_err(out_h[l, b], r["o"])
            worst = max(worst, err)
            assert err <= ATTN_TOL, (what, err)
            for h in range(H):
                s = (l, b * H + h)
                np.testing.assert_allclose(override[h], r["ema"][h], rtol=EMA_RTOL, atol=1e-12,
                                           err_msg=str((what, h)))
                want = set(r["pos_before"][h][r["keeps"][h]].tolist())
                if fused:  # the kept set, read off the compacted cache
                    got = set(S2[s]["pos8"].tolist()) | set(S2[s]["pos16"].tolist())
                else:
                    got = kept_positions(S1[s], keep_h[s[0], s[1]], eng.cap8)
                assert got == want, (what, h)
                assert_same_state(to_oracle_state(S2[s], wl.dtype16), heads[h], ema_rtol=0,
                                  what=(what, h))
            _say(f"    {what}: sizes {[heads[h].n for h in range(H)]} attention rel err {err:.2e}")
    assert eng.status() == 0
    _say("  worst attention rel err", worst)
    del eng
    torch.cuda.empty_cache()
