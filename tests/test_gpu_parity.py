"""HIP library vs the oracle, element by element, on identical seeded inputs.

Every call goes through the C ABI (libconfkv.so via the ctypes binding).  The
oracle is run from a snapshot of the device state copied back before each step
(teacher forcing), so every step is compared on identical inputs:
  * confidence c: absolute error <= 1e-5; budgets exact unless |c - tau| <= 1e-5
  * attention output: max over heads of ||o - o_ref||_inf / ||o_ref||_inf <= 2e-3
  * EMA: relative error <= 1e-5 against the oracle's float64 EMA
  * keep sets, INT8 codes, absmax, window bits, positions: bit-exact (the oracle's
    selection is fed the device's fp32 EMA, so both rank identical score arrays)
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from adaptive_kv_cache_amd import synth
from adaptive_kv_cache_amd.binding import Engine
from adaptive_kv_cache_amd.workloads import Workload
from parity_util import (assert_same_state, attn_rel_err, bits16, ema_by_pos, kept_positions,
                         oracle_params, tiny_workloads, to_oracle_state)

pytestmark = pytest.mark.gpu

ATTN_TOL = 2e-3
C_TOL = 1e-5
EMA_RTOL = 1e-5
SEED = 1234
TINY = tiny_workloads()


def _say(*a):
    print(*a, flush=True)


def _ingest(eng, wl, seed):
    pre = {}
    for l in range(wl.n_layers):
        k, v = synth.prefill_kv(wl, l, seed, device="cpu")
        eng.ingest(l, k.cuda(), v.cuda())
        pre[l] = (bits16(k), bits16(v))
    return pre


def _snap(eng, wl):
    return [[eng.export(l, b) for b in range(wl.batch)] for l in range(wl.n_layers)]


def _conf_wl(V, B, L=3, pyramid=True):
    return Workload(name="conf", n_layers=L, batch=B, n_q_heads=2, n_kv_heads=1, head_dim=64,
                    vocab=V, dtype16="f16", window=16, protect=4, n_high=100, n_low=200,
                    prefill=0, steps=1, pyramid=pyramid)


def _check_conf(c_gpu, budget_gpu, z, wl):
    for b in range(z.shape[0]):
        ref = O.confidence(z[b], wl.w_H, wl.w_m, wl.w_p)["c"]
        if np.isnan(ref):
            assert np.isnan(c_gpu[b])
            N = wl.n_low
        else:
            assert abs(float(c_gpu[b]) - ref) <= C_TOL, (b, float(c_gpu[b]), ref)
            N = O.budget(ref, wl.tau, wl.n_high, wl.n_low)
            if abs(ref - wl.tau) <= C_TOL:               # either budget is correct
                N = wl.n_high if c_gpu[b] >= wl.tau else wl.n_low
        want = [O.layer_budget(N, l, wl.n_layers, wl.pyramid) for l in range(wl.n_layers)]
        assert list(budget_gpu[b]) == want


# V = 2, 3, 4 and 5: rows shorter than one thread's loads (the loads past the row
# are clamped into it and discarded), with 16-byte loads at V = 4
@pytest.mark.parametrize("V,B", [(2, 2), (3, 1), (4, 2), (5, 3), (1000, 3), (4097, 1), (50257, 2),
                                 (152064, 8), (201088, 4)])
@pytest.mark.parametrize("T", [0.5, 2.0, 8.0])
def test_confidence(V, B, T):
    _say("confidence", V, B, T)
    wl = _conf_wl(V, B)
    eng = Engine(wl)
    g = torch.Generator().manual_seed(V + B)
    z = torch.randn(B, V, generator=g) * T
    c, budget = eng.confidence(z.cuda())
    _check_conf(c.cpu().numpy(), budget.cpu().numpy(), z.numpy().astype(np.float64), wl)


@pytest.mark.parametrize("V", [50257, 152064], ids=["scalar-loads", "16-byte-loads"])
def test_confidence_special_cases(V):
    B = 5
    wl = _conf_wl(V, B, L=1, pyramid=False)
    eng = Engine(wl)
    z = torch.zeros(B, V)
    z[1, 77] = 100.0                                # one-hot, gap 100: c = 1
    z[2, 5] = z[2, 9] = 3.0                         # tied maximum: margin 0
    z[3, 11] = float("nan")                         # non-finite: NaN, loose budget
    z[4, :] = torch.linspace(-50, 50, V)            # ramp
    c, budget = eng.confidence(z.cuda())
    c = c.cpu().numpy()
    assert abs(c[0] - (0.15 + 0.3 / V)) <= C_TOL     # uniform closed form
    assert abs(c[1] - 1.0) <= C_TOL
    assert np.isnan(c[3]) and int(budget[3, 0]) == wl.n_low
    _check_conf(c, budget.cpu().numpy(), z.numpy().astype(np.float64), wl)


@pytest.mark.parametrize("name", [n for n, w in TINY.items() if w.prefill > 0])
def test_ingest_bit_exact(name):
    wl = TINY[name]
    _say("ingest", name)
    eng = Engine(wl)
    pre = _ingest(eng, wl, SEED)
    for l in range(wl.n_layers):
        for b in range(wl.batch):
            ex = eng.export(l, b)
            ref = O.ingest(pre[l][0][b], pre[l][1][b], wl.window, wl.dtype16)
            assert_same_state(to_oracle_state(ex, wl.dtype16), ref, ema_rtol=0, what=(l, b))
    assert eng.status() == 0


def _teacher_forced(wl, steps, seed=SEED, poison=False):
    prm = oracle_params(wl)
    eng = Engine(wl)
    if poison:
        # NaN bit patterns in every window slot, then a reset: the attention reads
        # whole window halves, so it relies on the reset having zeroed the free slots
        nan = 0x7FC0 if wl.dtype16 == "bf16" else 0x7E00
        eng.t_k16.fill_(nan)
        eng.t_v16.fill_(nan)
        eng.reset()
    if wl.prefill:
        _ingest(eng, wl, seed)
    cap8 = eng.cap8
    worst = 0.0
    for step in range(steps):
        S0 = _snap(eng, wl)
        z = synth.logits(wl, step, seed)
        q = synth.q_new(wl, step, seed)
        k, v = synth.kv_new(wl, step, seed)
        out = eng.decode_attn(-1, q.cuda(), k.cuda(), v.cuda())
        S1 = _snap(eng, wl)
        c, budget = eng.confidence(z.cuda())
        keep = eng.rank_evict(-1, budget)
        eng.compact_demote(-1, keep)
        keep = keep.cpu().numpy()
        S2 = _snap(eng, wl)
        out = out.cpu().numpy()
        budget = budget.cpu().numpy()
        _check_conf(c.cpu().numpy(), budget, z.numpy().astype(np.float64), wl)
        qb, kb, vb = bits16(q), bits16(k), bits16(v)
        for l in range(wl.n_layers):
            for b in range(wl.batch):
                what = (wl.name, step, l, b)
                st = to_oracle_state(S0[l][b], wl.dtype16)
                new_pos = np.append(st.pos, st.t + 1)
                e_gpu = ema_by_pos(S1[l][b])
                override = np.array([e_gpu[p] for p in new_pos.tolist()], np.float32)
                r = O.step_layer(st, qb[l, b], kb[l, b], vb[l, b], int(budget[b, l]), prm,
                                 ema32_override=override)
                err = attn_rel_err(out[l, b], r["o"])
                worst = max(worst, err)
                assert err <= ATTN_TOL, (what, err)
                np.testing.assert_allclose(override, r["ema"], rtol=EMA_RTOL, atol=1e-12,
                                           err_msg=str(what))
                got = kept_positions(S1[l][b], keep[l, b], cap8)
                assert got == set(new_pos[r["keep"]].tolist()), what
                assert_same_state(to_oracle_state(S2[l][b], wl.dtype16), st, ema_rtol=0, what=what)
    assert eng.status() == 0
    return worst


@pytest.mark.parametrize("seed", [SEED, 99])
@pytest.mark.parametrize("name", list(TINY))
def test_teacher_forced_steps(name, seed):
    wl = TINY[name]
    steps = 150 if wl.prefill == 0 else 12
    _say("teacher-forced", name, steps, "seed", seed)
    worst = _teacher_forced(wl, steps, seed)
    _say("  worst attention rel err", worst)


@pytest.mark.parametrize("name", ["mha_bf16_d128_empty", "mha_f16_d64", "gqa16_bf16_d64_long"])
def test_reset_zeroes_the_window(name):
    """Window arrays full of NaN bit patterns before conf_cache_reset: every output,
    EMA and cache state still matches the oracle (the free slots of partial window
    halves meet probability 0, which cancels only the finite values the reset left)."""
    wl = TINY[name]
    steps = 60 if wl.prefill == 0 else 6
    _say("poisoned window before reset", name, steps)
    worst = _teacher_forced(wl, steps, poison=True)
    _say("  worst attention rel err", worst)


@pytest.mark.parametrize("name", list(TINY))
def test_fused_launches_equal_the_separate_ones(name):
    """Three engines on the same inputs: (a) decode_attn, rank_evict, compact_demote;
    (b) decode_attn, evict_compact; (c) attend, ema_evict_compact.  All leave the
    same cache (every exported array, bit for bit) and the same attention output,
    for all layers at once and layer by layer."""
    wl = TINY[name]
    _say("fused launches", name)
    a, b, c = Engine(wl), Engine(wl), Engine(wl)
    if wl.prefill:
        for e in (a, b, c):
            _ingest(e, wl, SEED)
    steps = min(wl.steps, 40) if wl.prefill else 200
    for step in range(steps):
        z = synth.logits(wl, step, SEED).cuda()
        q = synth.q_new(wl, step, SEED).cuda()
        k, v = (x.cuda() for x in synth.kv_new(wl, step, SEED))
        _, bud = a.confidence(z)
        layers = [-1] if step % 2 == 0 else list(range(wl.n_layers))
        outs = []
        for l in layers:
            ql, kl, vl = (x if l < 0 else x[l].contiguous() for x in (q, k, v))
            oa = a.decode_attn(l, ql, kl, vl)
            ob = b.decode_attn(l, ql, kl, vl)
            oc = c.attend(l, ql, kl, vl)
            outs.append((oa, ob, oc))
            a.compact_demote(l, a.rank_evict(l, bud))
            b.evict_compact(l, bud)
            c.ema_evict_compact(l, bud)
        for oa, ob, oc in outs:
            assert torch.equal(oa, ob) and torch.equal(oa, oc), step
        if step % 10 == 9 or step == steps - 1:
            for l in range(wl.n_layers):
                for s_ in range(wl.batch):
                    ea, eb, ec = a.export(l, s_), b.export(l, s_), c.export(l, s_)
                    for key in ea:
                        assert np.array_equal(np.asarray(ea[key]), np.asarray(eb[key])), \
                            ("evict_compact", step, l, s_, key)
                        assert np.array_equal(np.asarray(ea[key]), np.asarray(ec[key])), \
                            ("ema_evict_compact", step, l, s_, key)
    assert a.status() == 0 and b.status() == 0 and c.status() == 0


@pytest.mark.parametrize("name", ["gqa5_bf16_d128", "mha_f16_d64"])
def test_conf_step_equals_the_four_calls(name):
    """conf_step (attention, confidence and the fused selection + compaction) must
    be exactly decode_attn + confidence + rank_evict + compact_demote, which the
    teacher-forced test holds to the oracle."""
    wl = TINY[name]
    _say("conf_step", name)
    a, b = Engine(wl), Engine(wl)
    if wl.prefill:
        _ingest(a, wl, SEED)
        _ingest(b, wl, SEED)
    for step in range(12):
        z = synth.logits(wl, step, SEED).cuda()
        q = synth.q_new(wl, step, SEED).cuda()
        k, v = (x.cuda() for x in synth.kv_new(wl, step, SEED))
        out_a = a.decode_attn(-1, q, k, v)
        c_a, bud_a = a.confidence(z)
        a.compact_demote(-1, a.rank_evict(-1, bud_a))
        out_b, c_b, bud_b = b.step(z, q, k, v)
        assert torch.equal(out_a, out_b) and torch.equal(c_a, c_b) and torch.equal(bud_a, bud_b)
        for l in range(wl.n_layers):
            for s in range(wl.batch):
                ea, eb = a.export(l, s), b.export(l, s)
                for key in ea:
                    assert np.array_equal(np.asarray(ea[key]), np.asarray(eb[key])), (step, l, s, key)


@pytest.mark.parametrize("name", ["gqa5_bf16_d128", "mha_f16_d64"])
def test_rank_evict_budget_sweep(name):
    """Selection alone against the oracle, bit-exact, for budgets that evict 1 .. 40
    tokens (a few evictions take minimum rounds, more take the radix select), for a
    budget of exactly the protected window and one more, and for budgets the cache
    is already within."""
    wl = TINY[name]
    prm = oracle_params(wl)
    eng = Engine(wl)
    if wl.prefill:
        _ingest(eng, wl, SEED)
    for step in range(wl.n_high + 5 if not wl.prefill else 4):
        z, q = synth.logits(wl, step, SEED).cuda(), synth.q_new(wl, step, SEED).cuda()
        k, v = (x.cuda() for x in synth.kv_new(wl, step, SEED))
        eng.step(z, q, k, v)
    S = _snap(eng, wl)
    ntok = (eng.t_n8 + eng.t_n16).cpu().numpy()
    cap8 = eng.cap8
    P = wl.protect
    cases = [ntok - e for e in (1, 2, 3, 5, 8, 9, 17, 40)]
    # the degenerate budgets: only the protected window (K = 0), one more, and
    # budgets the cache is within (a no-op)
    cases += [np.full_like(ntok, P), np.full_like(ntok, P + 1), ntok, ntok + 5]
    for bud in cases:
        budget = np.ascontiguousarray(bud.T).astype(np.int32)
        keep = eng.rank_evict(-1, torch.from_numpy(budget).cuda()).cpu().numpy()
        for l in range(wl.n_layers):
            for b in range(wl.batch):
                st = to_oracle_state(S[l][b], wl.dtype16)
                scores = O.composite_scores(st.ema.astype(np.float32), st.pos, st.t,
                                            prm.s_ema, prm.s_rec)
                kr = O.select_keep(scores, st.pos, st.t, prm.protect, int(budget[b, l]))
                got = kept_positions(S[l][b], keep[l, b], cap8)
                assert got == set(st.pos[kr].tolist()), (int(budget[b, l]), l, b)
                assert len(got) == min(int(budget[b, l]), st.n)


@pytest.mark.parametrize("policy", ["full", "window"])
@pytest.mark.parametrize("name", ["gqa5_bf16_d128", "mha_f16_d64", "gqa16_bf16_d64_long"])
def test_baseline_policies(policy, name):
    """Full KV and the sliding window on the same kernels (conf_step), teacher-
    forced against the oracle run with the same policy's parameters: the ingest
    and every step's cache (positions, 16-bit bits) bit-exact, attention within
    tolerance.  The baselines keep no EMA, so it is not compared."""
    import dataclasses
    base = TINY[name]
    steps = 24 if base.prefill else 120
    wl = base.baseline(policy, steps)
    prm = oracle_params(wl)
    N = wl.window if policy == "window" else 10 ** 9
    if policy == "full":
        prm = dataclasses.replace(prm, n_high=N, n_low=N)
    _say("baseline", policy, name)
    eng = Engine(wl)
    if wl.prefill:
        pre = _ingest(eng, wl, SEED)
        for l in range(wl.n_layers):
            for b in range(wl.batch):
                ref = O.ingest(pre[l][0][b], pre[l][1][b], wl.window, wl.dtype16,
                               drop_old=policy == "window")
                assert_same_state(to_oracle_state(eng.export(l, b), wl.dtype16), ref,
                                  what=("ingest", l, b))
    worst = 0.0
    for step in range(steps):
        S0 = _snap(eng, wl)
        z = synth.logits(wl, step, SEED)
        q = synth.q_new(wl, step, SEED)
        k, v = synth.kv_new(wl, step, SEED)
        out, _, _ = eng.step(z.cuda(), q.cuda(), k.cuda(), v.cuda())
        out = out.cpu().numpy()
        S2 = _snap(eng, wl)
        qb, kb, vb = bits16(q), bits16(k), bits16(v)
        for l in range(wl.n_layers):
            for b in range(wl.batch):
                st = to_oracle_state(S0[l][b], wl.dtype16)
                r = O.step_layer(st, qb[l, b], kb[l, b], vb[l, b], N, prm)
                err = attn_rel_err(out[l, b], r["o"])
                worst = max(worst, err)
                assert err <= ATTN_TOL, (policy, name, step, l, b, err)
                assert_same_state(to_oracle_state(S2[l][b], wl.dtype16), st,
                                  what=(policy, step, l, b))
                assert not st.is8.any()                     # the baselines stay 16-bit
                if policy == "window":
                    assert st.pos.tolist() == list(range(max(0, st.t - wl.window + 1), st.t + 1))
    assert eng.status() == 0
    _say("  worst attention rel err", worst)


@pytest.mark.parametrize("name", ["gqa5_bf16_d128", "mha_f16_d64"])
def test_window_policy_ignores_the_budget(name):
    """The sliding window keeps exactly (t-W, t] in 16 bits even when the budgets
    exceed W: the oracle runs the window's own parameters (N = P = W), the library
    budgets of W + 37 and W + 90 that the window rule must override."""
    import dataclasses
    base = TINY[name]
    steps = 16 if base.prefill else 100
    wl_ref = base.baseline("window", steps)
    W = wl_ref.window
    wl = dataclasses.replace(wl_ref, n_high=W + 37, n_low=W + 90, protect=max(1, W // 4))
    prm = oracle_params(wl_ref)
    _say("window with budgets above W", name)
    eng = Engine(wl)
    if wl.prefill:
        _ingest(eng, wl, SEED)
    for step in range(steps):
        S0 = _snap(eng, wl)
        z = synth.logits(wl, step, SEED)
        q = synth.q_new(wl, step, SEED)
        k, v = synth.kv_new(wl, step, SEED)
        out, _, budget = eng.step(z.cuda(), q.cuda(), k.cuda(), v.cuda())
        assert int(budget.min()) > W
        out = out.cpu().numpy()
        S2 = _snap(eng, wl)
        qb, kb, vb = bits16(q), bits16(k), bits16(v)
        for l in range(wl.n_layers):
            for b in range(wl.batch):
                st = to_oracle_state(S0[l][b], wl.dtype16)
                r = O.step_layer(st, qb[l, b], kb[l, b], vb[l, b], W, prm)
                assert attn_rel_err(out[l, b], r["o"]) <= ATTN_TOL, (name, step, l, b)
                got = to_oracle_state(S2[l][b], wl.dtype16)
                assert_same_state(got, st, what=("window", step, l, b))
                assert not got.is8.any()
                assert got.pos.tolist() == list(range(max(0, got.t - W + 1), got.t + 1))
    assert eng.status() == 0


def test_sawtooth_and_no_op_from_empty():
    wl = TINY["mha_f16_d64"]
    eng = Engine(wl)
    sizes = np.zeros((wl.n_layers, wl.batch), np.int64)
    saw = set()
    for step in range(wl.steps):
        z = synth.logits(wl, step, 7)
        q = synth.q_new(wl, step, 7)
        k, v = synth.kv_new(wl, step, 7)
        _, c, budget = eng.step(z.cuda(), q.cuda(), k.cuda(), v.cuda())
        n = (eng.t_n8 + eng.t_n16).cpu().numpy()
        budget = budget.cpu().numpy()
        for l in range(wl.n_layers):
            for b in range(wl.batch):
                want = min(sizes[l, b] + 1, budget[b, l])
                assert n[l, b] == want, (step, l, b)
                sizes[l, b] = want
        saw |= set(budget[:, 0].tolist())
        if step < min(wl.n_high, wl.n_low) // 2:
            assert int(n.min()) == step + 1                 # no-op under budget
    assert saw == {wl.n_high, wl.n_low}
    assert int((eng.t_n16).max()) <= wl.window
    assert eng.status() == 0


def _trim_cases():
    long = TINY["gqa16_bf16_d64_long"].scaled(name="gqa16_bf16_d64_trim6k", prefill=6100,
                                             n_high=6000, n_low=6000, steps=5)
    return {"mha_f16_d64": (TINY["mha_f16_d64"], 190), "gqa5_bf16_d128": (TINY["gqa5_bf16_d128"], 30),
            "gqa8_bf16_d64": (TINY["gqa8_bf16_d64"], 30), "trim6k": (long, 5)}


def _trim_betas(shape, step, special):
    """ln(beta) of the new tokens: the seeded gate draws, or a small set of values
    (0, -0.5, -1, -2, -inf) that gives tied retention scores."""
    if not special:
        return None
    g = torch.Generator().manual_seed(999 + step)
    vals = torch.tensor([0.0, -0.5, -1.0, -2.0, float("-inf")])
    return vals[torch.randint(0, 5, shape, generator=g)]


@pytest.mark.parametrize("special", [False, True])
@pytest.mark.parametrize("case", ["mha_f16_d64", "gqa5_bf16_d128", "gqa8_bf16_d64", "trim6k"])
def test_retention_eviction(case, special):
    """Retention eviction (conf_attend + conf_trim_evict_compact) teacher-forced
    against the oracle's trim_step: attention within tolerance, kept positions,
    window bits and each token's ln(beta) bit-exact.  Budgets are M, with some
    steps cutting 9 to 40 tokens at once (the radix path) and the cache then
    growing back under its budget (no-op steps)."""
    base, steps = _trim_cases()[case]
    wl = base.baseline("trim", steps)
    M = wl.n_high
    prm = oracle_params(wl)
    _say("trim", case, "special" if special else "gate", "M", M, "prefill", wl.prefill)
    eng = Engine(wl)
    if wl.prefill:
        pre = _ingest(eng, wl, SEED)
        for l in range(wl.n_layers):
            lb_pre = synth.log_beta_prefill(wl, l, SEED)
            if special:
                lb_pre = _trim_betas(lb_pre.shape, -1 - l, True)
            eng.set_retention(l, lb_pre.cuda())
            for b in range(wl.batch):
                ref = O.ingest(pre[l][0][b], pre[l][1][b], wl.window, wl.dtype16)
                ref.ema = lb_pre[b].numpy().astype(np.float32).astype(np.float64)
                got = to_oracle_state(eng.export(l, b), wl.dtype16)
                assert_same_state(got, ref, what=("ingest", l, b))
                assert np.array_equal(got.ema, ref.ema)
    worst = 0.0
    L, B = wl.n_layers, wl.batch
    for step in range(steps):
        S0 = _snap(eng, wl)
        q = synth.q_new(wl, step, SEED)
        k, v = synth.kv_new(wl, step, SEED)
        lbn = _trim_betas((L, B), step, special) if special else synth.log_beta_new(wl, step, SEED)
        budget = torch.full((B, L), M, dtype=torch.int32)
        if step % 7 == 3:
            for b in range(B):
                for l in range(L):
                    budget[b, l] = M - (9 + 11 * b + 5 * l) % 32
        out = eng.attend(-1, q.cuda(), k.cuda(), v.cuda())
        eng.trim_evict_compact(-1, budget.cuda(), lbn.cuda())
        out = out.cpu().numpy()
        S2 = _snap(eng, wl)
        qb, kb, vb = bits16(q), bits16(k), bits16(v)
        for l in range(L):
            for b in range(B):
                st = to_oracle_state(S0[l][b], wl.dtype16)
                n_before = st.n
                r = O.trim_step(st, qb[l, b], kb[l, b], vb[l, b], float(lbn[l, b]),
                                int(budget[b, l]), prm)
                err = attn_rel_err(out[l, b], r["o"])
                worst = max(worst, err)
                assert err <= ATTN_TOL, (case, step, l, b, err)
                got = to_oracle_state(S2[l][b], wl.dtype16)
                assert_same_state(got, st, what=("trim", step, l, b))
                assert np.array_equal(got.ema, st.ema), ("ln(beta)", step, l, b)
                assert not st.is8.any()
                assert st.n == min(n_before + 1, int(budget[b, l]))
    assert eng.status() == 0
    _say("  worst attention rel err", worst)


def _headwise_cases():
    wide = Workload(name="hw_wide_f16_d64", n_layers=1, batch=1, n_q_heads=8, n_kv_heads=8,
                    head_dim=64, vocab=500, dtype16="f16", window=40, protect=6, n_high=700,
                    n_low=760, prefill=1000, steps=6)
    return {"mha_f16_d64": (TINY["mha_f16_d64"], 170), "gqa5_bf16_d128": (TINY["gqa5_bf16_d128"], 14),
            "gqa8_bf16_d64": (TINY["gqa8_bf16_d64"], 14), "mha16_f16_d128": (TINY["mha16_f16_d128"], 10),
            "hw_wide_f16_d64": (wide, 6)}


@pytest.mark.parametrize("case", list(_headwise_cases()))
def test_headwise_teacher_forced(case):
    """Head-wise keep sets through the C ABI (decode_attn, confidence, the joint
    rank_evict, compact_demote), teacher-forced against the oracle's
    headwise_step on every (layer, sequence): attention within tolerance, each
    head's EMA within 1e-5, the joint keep sets and every head's cache bit-exact.
    hw_wide holds 8000 tokens over its 8 heads at the first step, more than the
    selection's LDS key cache, and cuts them to 5600 pairs."""
    base, steps = _headwise_cases()[case]
    wl = base.headwise_variant()
    H, S = wl.n_kv_heads, wl.n_sub
    prm = oracle_params(wl)
    _say("headwise", case, "heads", H, "steps", steps)
    eng = Engine(wl)
    cap8 = eng.cap8
    if wl.prefill:
        pre = _ingest(eng, wl, SEED)
        for l in range(wl.n_layers):
            for b in range(wl.batch):
                for h in range(H):
                    ref = O.ingest(pre[l][0][b][h:h + 1], pre[l][1][b][h:h + 1], wl.window,
                                   wl.dtype16)
                    got = to_oracle_state(eng.export(l, b * H + h), wl.dtype16)
                    assert_same_state(got, ref, ema_rtol=0, what=("ingest", l, b, h))
    worst = 0.0
    sizes_seen = set()
    for step in range(steps):
        S0 = _snap_sub(eng, wl)
        z = synth.logits(wl, step, SEED)
        q = synth.q_new(wl, step, SEED)
        k, v = synth.kv_new(wl, step, SEED)
        out = eng.decode_attn(-1, q.cuda(), k.cuda(), v.cuda())
        S1 = _snap_sub(eng, wl)
        c, budget = eng.confidence(z.cuda())
        keep = eng.rank_evict(-1, budget)
        eng.compact_demote(-1, keep)
        keep = keep.cpu().numpy()
        S2 = _snap_sub(eng, wl)
        out = out.cpu().numpy()
        budget = budget.cpu().numpy()
        _check_conf(c.cpu().numpy(), budget, z.numpy().astype(np.float64), wl)
        qb, kb, vb = bits16(q), bits16(k), bits16(v)
        for l in range(wl.n_layers):
            for b in range(wl.batch):
                subs = [b * H + h for h in range(H)]
                heads = [to_oracle_state(S0[l][s], wl.dtype16) for s in subs]
                override = []
                for s, st in zip(subs, heads):
                    e_gpu = ema_by_pos(S1[l][s])
                    override.append(np.array([e_gpu[p] for p in np.append(st.pos, st.t + 1)],
                                             np.float32))
                n_before = sum(st.n for st in heads)
                r = O.headwise_step(heads, qb[l, b], kb[l, b], vb[l, b], int(budget[b, l]), prm,
                                    ema32_override=override)
                what = (case, step, l, b)
                err = attn_rel_err(out[l, b], r["o"])
                worst = max(worst, err)
                assert err <= ATTN_TOL, (what, err)
                for h, s in enumerate(subs):
                    np.testing.assert_allclose(override[h], r["ema"][h], rtol=EMA_RTOL,
                                               atol=1e-12, err_msg=str((what, h)))
                    got = kept_positions(S1[l][s], keep[l, s], cap8)
                    assert got == set(r["pos_before"][h][r["keeps"][h]].tolist()), (what, h)
                    assert_same_state(to_oracle_state(S2[l][s], wl.dtype16), heads[h],
                                      ema_rtol=0, what=(what, h))
                n_heads = [heads[h].n for h in range(H)]
                sizes_seen.add(tuple(n_heads))
                assert sum(n_heads) == min(n_before + H, H * int(budget[b, l])), what
    assert eng.status() == 0
    # the keep sets are ragged: heads of one (layer, sequence) end with different sizes
    assert any(len(set(sz)) > 1 for sz in sizes_seen) or H == 1
    _say("  worst attention rel err", worst)


def _snap_sub(eng, wl):
    return [[eng.export(l, s) for s in range(wl.n_sub)] for l in range(wl.n_layers)]


@pytest.mark.parametrize("case", ["mha_f16_d64", "gqa5_bf16_d128", "hw_wide_f16_d64"])
def test_headwise_entry_points_agree(case):
    """Head-wise: conf_step, attend + ema_evict_compact, and decode_attn +
    evict_compact leave bit-identical caches and outputs, for all layers at once
    and layer by layer."""
    base, steps = _headwise_cases()[case]
    wl = base.headwise_variant()
    _say("headwise entry points", case)
    a, b, c = Engine(wl), Engine(wl), Engine(wl)
    if wl.prefill:
        for e in (a, b, c):
            _ingest(e, wl, SEED)
    steps = min(steps, 60)
    for step in range(steps):
        z = synth.logits(wl, step, SEED).cuda()
        q = synth.q_new(wl, step, SEED).cuda()
        k, v = (x.cuda() for x in synth.kv_new(wl, step, SEED))
        oa, ca, bud = a.step(z, q, k, v)
        layers = [-1] if step % 2 == 0 else list(range(wl.n_layers))
        for l in layers:
            ql, kl, vl = (x if l < 0 else x[l].contiguous() for x in (q, k, v))
            ob = b.attend(l, ql, kl, vl)
            b.ema_evict_compact(l, bud)
            oc = c.decode_attn(l, ql, kl, vl)
            c.evict_compact(l, bud)
            ref = oa if l < 0 else oa[l]
            assert torch.equal(ref, ob) and torch.equal(ref, oc), (step, l)
        if step % 5 == 4 or step == steps - 1:
            for l in range(wl.n_layers):
                for s_ in range(wl.n_sub):
                    ea, eb, ec = a.export(l, s_), b.export(l, s_), c.export(l, s_)
                    for key in ea:
                        assert np.array_equal(np.asarray(ea[key]), np.asarray(eb[key])), \
                            ("ema_evict_compact", step, l, s_, key)
                        assert np.array_equal(np.asarray(ea[key]), np.asarray(ec[key])), \
                            ("evict_compact", step, l, s_, key)
    assert a.status() == 0 and b.status() == 0 and c.status() == 0


def _arkv_cases():
    return {"mha_f16_d64": (TINY["mha_f16_d64"], 190), "gqa5_bf16_d128": (TINY["gqa5_bf16_d128"], 24),
            "gqa8_bf16_d64": (TINY["gqa8_bf16_d64"], 24), "mha16_f16_d128": (TINY["mha16_f16_d128"], 12),
            "gqa16_bf16_d64_long": (TINY["gqa16_bf16_d64_long"], 8)}


def _arkv_wl(base, steps):
    # the full prefill, so that ingest quantises its older part to e4m3 and the first
    # step after a long one attends past the LDS score rows over FP8 tokens
    return base.baseline("arkv", steps).scaled(prefill=base.prefill)


def _fp8_state(st):
    f = O.Fp8State(st.k16.shape[1], st.k16.shape[2], st.dtype16)
    for k in ("pos", "is8", "k16", "v16", "k8", "v8", "ema", "amax_k", "amax_v", "t"):
        setattr(f, k, getattr(st, k))
    return f


def _arkv_budgets(wl, step, n_orig0):
    """N kept tokens per (sequence, layer), with every seventh step cutting 9 to 40;
    N_O from the layer's OQ ratio, lowered by up to 12 on some steps so that a step
    has several tokens to quantise."""
    B, L = wl.batch, wl.n_layers
    N = torch.full((B, L), wl.n_high, dtype=torch.int32)
    NO = n_orig0[None, :].repeat(B, 1).clone()
    if step % 7 == 3:
        for b in range(B):
            for l in range(L):
                N[b, l] = wl.n_high - (9 + 11 * b + 5 * l) % 32
    if step % 5 == 2:
        for b in range(B):
            NO[b] = torch.clamp(NO[b] - (3 + 4 * b) % 13, min=wl.protect)
    NO = torch.minimum(NO, N)
    return N, NO


@pytest.mark.parametrize("case", list(_arkv_cases()))
def test_arkv_teacher_forced(case):
    """ARKV through the C ABI (decode_attn with the heavy-hitter score EMA, then
    arkv_evict_compact), teacher-forced against the oracle's arkv_step on every
    (layer, sequence): attention within tolerance, the score EMA within 1e-5,
    kept positions, which tokens are Original or FP8, e4m3 codes, absmax and
    window bits bit-exact."""
    base, steps = _arkv_cases()[case]
    wl = _arkv_wl(base, steps)
    prm = oracle_params(wl)
    # Original budgets a little above P, so that the short runs after a prefill
    # (whose kept tokens are mostly FP8 at first) reach them and quantise
    n_orig0 = torch.minimum(synth.arkv_n_orig(wl, SEED),
                            wl.protect + 6 + 3 * torch.arange(wl.n_layers, dtype=torch.int32))
    _say("arkv", case, "N", wl.n_high, "W", wl.window, "N_O", n_orig0.tolist())
    eng = Engine(wl)
    if wl.prefill:
        pre = _ingest(eng, wl, SEED)
        for l in range(wl.n_layers):
            for b in range(wl.batch):
                ref = O.ingest_fp8(pre[l][0][b], pre[l][1][b], wl.window, wl.dtype16)
                assert_same_state(to_oracle_state(eng.export(l, b), wl.dtype16), ref, ema_rtol=0,
                                  what=("ingest", l, b))
    worst = 0.0
    demoted = 0
    for step in range(steps):
        S0 = _snap(eng, wl)
        q = synth.q_new(wl, step, SEED)
        k, v = synth.kv_new(wl, step, SEED)
        N, NO = _arkv_budgets(wl, step, n_orig0)
        out = eng.decode_attn(-1, q.cuda(), k.cuda(), v.cuda())
        S1 = _snap(eng, wl)
        eng.arkv_evict_compact(-1, N.cuda(), NO.cuda())
        S2 = _snap(eng, wl)
        out = out.cpu().numpy()
        qb, kb, vb = bits16(q), bits16(k), bits16(v)
        for l in range(wl.n_layers):
            for b in range(wl.batch):
                what = (case, step, l, b)
                st = _fp8_state(to_oracle_state(S0[l][b], wl.dtype16))
                e_gpu = ema_by_pos(S1[l][b])
                override = np.array([e_gpu[p] for p in np.append(st.pos, st.t + 1).tolist()],
                                    np.float32)
                r = O.arkv_step(st, qb[l, b], kb[l, b], vb[l, b], int(N[b, l]), int(NO[b, l]),
                                prm, ema32_override=override)
                err = attn_rel_err(out[l, b], r["o"])
                worst = max(worst, err)
                assert err <= ATTN_TOL, (what, err)
                np.testing.assert_allclose(override, r["ema"], rtol=EMA_RTOL, atol=1e-12,
                                           err_msg=str(what))
                assert_same_state(to_oracle_state(S2[l][b], wl.dtype16), st, ema_rtol=0, what=what)
                demoted += len(r["demoted"])
    assert eng.status() == 0
    assert demoted > 0
    _say("  worst attention rel err", worst, "tokens quantised", demoted)


@pytest.mark.parametrize("case", ["mha_f16_d64", "gqa5_bf16_d128", "gqa16_bf16_d64_long"])
def test_arkv_fused_equals_split(case):
    """attend + arkv_ema_evict_compact (the score EMA in the eviction launch) leaves
    exactly the cache and output of decode_attn + arkv_evict_compact, for all
    layers at once and layer by layer."""
    base, steps = _arkv_cases()[case]
    wl = _arkv_wl(base, steps)
    n_orig0 = torch.minimum(synth.arkv_n_orig(wl, SEED),
                            wl.protect + 6 + 3 * torch.arange(wl.n_layers, dtype=torch.int32))
    _say("arkv fused", case)
    a, b = Engine(wl), Engine(wl)
    if wl.prefill:
        _ingest(a, wl, SEED)
        _ingest(b, wl, SEED)
    for step in range(min(steps, 60)):
        q = synth.q_new(wl, step, SEED).cuda()
        k, v = (x.cuda() for x in synth.kv_new(wl, step, SEED))
        N, NO = (x.cuda() for x in _arkv_budgets(wl, step, n_orig0))
        layers = [-1] if step % 2 == 0 else list(range(wl.n_layers))
        for l in layers:
            ql, kl, vl = (x if l < 0 else x[l].contiguous() for x in (q, k, v))
            oa = a.attend(l, ql, kl, vl)
            a.arkv_ema_evict_compact(l, N, NO)
            ob = b.decode_attn(l, ql, kl, vl)
            b.arkv_evict_compact(l, N, NO)
            assert torch.equal(oa, ob), (step, l)
        if step % 5 == 4:
            for l in range(wl.n_layers):
                for s_ in range(wl.batch):
                    ea, eb = a.export(l, s_), b.export(l, s_)
                    for key in ea:
                        assert np.array_equal(np.asarray(ea[key]), np.asarray(eb[key])), \
                            (step, l, s_, key)
    assert a.status() == 0 and b.status() == 0


@pytest.mark.parametrize("name", ["mha_f16_d64", "gqa5_bf16_d128"])
def test_layer_views_on_two_streams_equal_the_whole_cache(name):
    """Two layer-range views of one cache, each with its own workspace, driven on
    two concurrent streams (the bench's layer split) leave exactly the cache and
    outputs of the whole cache driven on one stream."""
    wl = TINY[name].scaled(name=name + "_4l", n_layers=4)
    L = wl.n_layers
    _say("layer views", wl.name)
    a, b = Engine(wl), Engine(wl)
    if wl.prefill:
        _ingest(a, wl, SEED)
        _ingest(b, wl, SEED)
    halves = [(0, 2), (2, 4)]
    views = [b.layer_view(l0, l1 - l0) for l0, l1 in halves]
    main = torch.cuda.current_stream()
    streams = [main, torch.cuda.Stream()]
    out_b = torch.empty(L, wl.batch, wl.n_q_heads, wl.head_dim, dtype=torch.float32, device="cuda")
    for step in range(min(wl.steps, 60) if wl.prefill else 200):
        z = synth.logits(wl, step, SEED).cuda()
        q = synth.q_new(wl, step, SEED).cuda()
        k, v = (x.cuda() for x in synth.kv_new(wl, step, SEED))
        out_a = a.attend(-1, q, k, v)
        _, bud = a.confidence(z)
        a.ema_evict_compact(-1, bud)
        _, bud_b = b.confidence(z)
        cols = [bud_b[:, l0:l1].contiguous() for l0, l1 in halves]
        for st in streams[1:]:
            st.wait_stream(main)
        for (l0, l1), view, st, col in zip(halves, views, streams, cols):
            with torch.cuda.stream(st):
                view.attend(-1, q[l0:l1], k[l0:l1], v[l0:l1], out=out_b[l0:l1])
                view.ema_evict_compact(-1, col)
        for st in streams[1:]:
            main.wait_stream(st)
        assert torch.equal(out_a, out_b), step
        if step % 20 == 19:
            for l in range(L):
                for s_ in range(wl.batch):
                    ea, eb = a.export(l, s_), b.export(l, s_)
                    for key in ea:
                        assert np.array_equal(np.asarray(ea[key]), np.asarray(eb[key])), \
                            (step, l, s_, key)
    assert a.status() == 0 and b.status() == 0


def test_full_window_sets_the_status_bit_and_keeps_the_cache():
    """Full KV with a window of 64 slots and a 60-token prefill: four appends fit;
    from the fifth step on each new token is dropped, CONF_ST_WINDOW_FULL is set, and
    the cache keeps exactly the 64 tokens it holds (positions 0..63, bits unchanged),
    while the attention still runs over them."""
    from adaptive_kv_cache_amd.binding import ST_WINDOW_FULL
    wl = TINY["gqa8_bf16_d64"].scaled(name="full_window_64", prefill=60)
    wl = wl.baseline("full", 1).scaled(window=63, n_high=64, n_low=64)
    _say("window full", wl.name, "W", wl.window)
    eng = Engine(wl)
    _ingest(eng, wl, SEED)
    assert eng.cap16 == 64
    for step in range(8):
        z = synth.logits(wl, step, SEED).cuda()
        q = synth.q_new(wl, step, SEED).cuda()
        k, v = (x.cuda() for x in synth.kv_new(wl, step, SEED))
        before = [eng.export(l, b) for l in range(wl.n_layers) for b in range(wl.batch)]
        out, _, _ = eng.step(z, q, k, v)
        assert torch.isfinite(out).all()
        after = [eng.export(l, b) for l in range(wl.n_layers) for b in range(wl.batch)]
        full = step >= 4
        assert bool(eng.status() & ST_WINDOW_FULL) == full, step
        for x0, x1 in zip(before, after):
            assert x1["n16"] == min(60 + step + 1, 64)
            if full:   # nothing changes once the window is full
                for key in ("pos16", "k16", "v16"):
                    assert np.array_equal(x0[key], x1[key]), (step, key)
    assert sorted(after[0]["pos16"].tolist()) == list(range(64))


@pytest.mark.parametrize("name,policy", [("gqa5_bf16_d128", "confkv"), ("gqa8_bf16_d64", "trim"),
                                         ("mha16_f16_d128", "window")])
def test_ingest_all_layers_at_once(name, policy):
    """conf_cache_ingest (and conf_cache_set_retention) with layer = -1, every
    layer in one launch from [L][B][Hkv][L0][d], leaves exactly the cache of the
    per-layer calls."""
    base = TINY[name].scaled(name=name + "_3l", n_layers=3)
    wl = base if policy == "confkv" else base.baseline(policy, 4)
    _say("ingest all layers", wl.name)
    a, b = Engine(wl), Engine(wl)
    ks, vs, lbs = [], [], []
    for l in range(wl.n_layers):
        k, v = synth.prefill_kv(wl, l, SEED, device="cuda")
        a.ingest(l, k, v)
        ks.append(k)
        vs.append(v)
        if policy == "trim":
            lb = synth.log_beta_prefill(wl, l, SEED, device="cuda")
            a.set_retention(l, lb)
            lbs.append(lb)
    b.ingest(-1, torch.stack(ks).contiguous(), torch.stack(vs).contiguous())
    if policy == "trim":
        b.set_retention(-1, torch.stack(lbs).contiguous())
    for l in range(wl.n_layers):
        for s_ in range(wl.batch):
            ea, eb = a.export(l, s_), b.export(l, s_)
            for key in ea:
                assert np.array_equal(np.asarray(ea[key]), np.asarray(eb[key])), (l, s_, key)
    assert a.status() == 0 and b.status() == 0


@pytest.mark.parametrize("case", ["gqa5_bf16_d128", "gqa8_bf16_d64", "mha16_f16_d128",
                                  "gqa16_bf16_d64_long"])
def test_arkv_prefill_budgets(case):
    """ARKV's prefill phase through the C ABI: each (layer, sequence)'s concentration
    of the probe queries' attention over the prefill keys within 2e-5 of the
    oracle's float64 value, and the Original budgets bit-exact against the oracle's
    float32 mapping of the same (device) concentrations.  Six layers, so the
    per-sequence spread between the least and most concentrated layer is real;
    the one-layer shape takes the midpoint."""
    base = TINY[case]
    wl = _arkv_wl(base, 4)
    if case == "gqa5_bf16_d128":
        wl = wl.scaled(n_layers=6)
    eng = Engine(wl)
    q0 = synth.q_new(wl, 0, SEED)
    conc = torch.zeros(wl.n_layers, wl.batch, dtype=torch.float32, device="cuda")
    pre = []
    for l in range(wl.n_layers):
        k, v = synth.prefill_kv(wl, l, SEED)
        eng.arkv_prefill_stats(l, q0[l].cuda(), k.cuda(), conc)
        pre.append(bits16(k))
    n_orig = eng.arkv_orig_budgets(conc).cpu().numpy()
    conc_h = conc.cpu().numpy()
    qb = bits16(q0)
    worst = 0.0
    for l in range(wl.n_layers):
        for b in range(wl.batch):
            ref = O.arkv_prefill_concentration(O.decode16(qb[l, b], wl.dtype16),
                                               O.decode16(pre[l][b], wl.dtype16), wl.group)
            err = abs(float(conc_h[l, b]) - ref[-1])
            worst = max(worst, err)
            assert err <= 2e-5, (case, l, b, float(conc_h[l, b]), ref[-1])
    for b in range(wl.batch):
        want = O.arkv_orig_budgets(conc_h[:, b], wl.n_high, wl.protect)
        assert n_orig[b].tolist() == want.tolist(), (case, b)
    _say("arkv prefill", case, "worst concentration error", worst, "N_O", n_orig[0].tolist())


def test_arkv_prefill_special_inputs():
    """q = 0 gives uniform attention, concentration 0 exactly; a query aligned with
    one key of large norm gives almost one-hot attention; all layers alike give the
    midpoint ratio."""
    wl = _arkv_wl(TINY["gqa5_bf16_d128"], 4).scaled(n_layers=3)
    eng = Engine(wl)
    L0, d = 400, wl.head_dim
    g = torch.Generator().manual_seed(3)
    k = torch.randn(wl.n_layers, wl.batch, wl.n_kv_heads, L0, d, generator=g)
    q = torch.zeros(wl.n_layers, wl.batch, wl.n_q_heads, d)
    # layer 2: every head's query points at key 123 of its KV head, scaled far up
    for b in range(wl.batch):
        for h in range(wl.n_q_heads):
            kv = h // wl.group
            k[2, b, kv, 123] = 6.0 * torch.ones(d)
            q[2, b, h] = 6.0 * torch.ones(d)
    dt = eng.dtype16
    conc = eng.arkv_prefill_stats(-1, q.to(dt).cuda(), k.to(dt).cuda())
    c = conc.cpu()
    assert torch.all(c[0] == 0.0) and torch.all(c[1] == 0.0)
    assert torch.all(c[2] > 0.9)
    n = eng.arkv_orig_budgets(conc).cpu()
    assert torch.all(n[:, 2] == math.ceil(np.float32(0.95) * np.float32(wl.n_high)))
    assert torch.all(n[:, 0] == max(wl.protect, math.ceil(np.float32(0.75) * wl.n_high)))
    flat = eng.arkv_orig_budgets(torch.zeros_like(conc)).cpu()
    assert torch.all(flat == max(wl.protect, math.ceil(np.float32(0.85) * wl.n_high)))
