"""Full-size parity on sampled (layer, sequence) pairs, for every workload shape.

Each workload runs at its full size, exactly as the benchmark drives the library:
every layer and sequence in one launch per kernel.  The oracle cannot run every
(layer, sequence) pair, so it re-runs sampled pairs one by one from a snapshot of
their device state (teacher forcing) at chosen steps.  The steps of the
Qwen-32B-shaped batch-8 cache (the benchmark's) are the three kinds a decode
step can be:
  * step 0: the one-off cut of the prefilled 32769 tokens to the budget (the
    scores exceed the LDS rows, so most items keep theirs in the workspace);
  * step 1: a loose-budget step with 4097 tokens (also beyond the LDS rows);
  * step 66: after the first confident phase, about 2050 tokens (single pass,
    scores in LDS), the steady state the benchmark times.
The caches that start empty are checked at their first demotion into INT8, at
the first eviction and deep into their sawtooth.  Tolerances are those of the
small-shape parity tests.  Confidence and budgets are checked for every sequence
at every checked step.  The steps between checked ones run the benchmark's
launches (conf_attend, then the EMA fused into the selection + compaction; on
the caches whose attention launch has at least 2048 workgroups, on two layer
halves as views of the cache on two concurrent streams, as the benchmark does).  A
checked step runs conf_decode_attn, so that the EMA can be read before the
selection, and then on even steps the fused selection + compaction, on odd steps
the two separate ones; on a fused step the kept set is read off the cache after
compaction.
"""
import json
import os

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
C_TOL = 1e-5
EMA_RTOL = 1e-5
SEED = 0                                   # the benchmark's seed
# workload -> ((layer, sequence) samples, checked steps)
CASES = {
    "qwen32b_gqa_b8_32k": ([(0, 0), (37, 5), (63, 7)], (0, 1, 66)),
    "qwen32b_gqa_b1_32k": ([(0, 0), (63, 0)], (0, 66)),
    "qwen14b_gqa_b8_8k": ([(0, 3), (47, 6)], (0, 1, 66)),
    "gptoss20b_gqa_b32_16k": ([(0, 0), (23, 31), (11, 17)], (0, 1, 40)),
    # c near tau: sequence 31's confidence at step 318 is the threshold itself (the
    # median row); checked steps come in consecutive pairs, so budget flips show
    "gptoss20b_gqa_b32_16k_stress": ([(0, 31), (23, 31), (11, 17)],
                                     (0, 1, 317, 318)),
    "gpt2_1layer_b1": ([(0, 0)], (129, 600, 2047)),
    "gpt2_12layer_b8_pyramid": ([(0, 0), (11, 7), (5, 3)], (129, 700, 1500)),
}


def _say(*a):
    print(*a, flush=True)


def _check_conf(c_gpu, budget_gpu, z, wl):
    for b in range(z.shape[0]):
        ref = O.confidence(z[b], wl.w_H, wl.w_m, wl.w_p)["c"]
        assert abs(float(c_gpu[b]) - ref) <= C_TOL, (b, float(c_gpu[b]), ref)
        N = O.budget(ref, wl.tau, wl.n_high, wl.n_low)
        if abs(ref - wl.tau) <= C_TOL:
            N = wl.n_high if c_gpu[b] >= wl.tau else wl.n_low
        assert list(budget_gpu[b]) == [O.layer_budget(N, l, wl.n_layers, wl.pyramid)
                                       for l in range(wl.n_layers)]


@pytest.mark.parametrize("name", list(CASES))
def test_full_size_sampled_pairs(name):
    wl = WORKLOADS[name]
    SAMPLES, CHECKED = CASES[name]
    prm = oracle_params(wl)
    dev = torch.device("cuda", 0)
    _say("full size: allocating and ingesting", wl.name)
    eng = Engine(wl, dev)
    for l in range(wl.n_layers if wl.prefill else 0):
        k, v = synth.prefill_kv(wl, l, SEED, device=dev)
        eng.ingest(l, k, v)
        if l in {s[0] for s in SAMPLES}:
            # the ingest itself, for the sampled pairs
            for (sl, b) in SAMPLES:
                if sl != l:
                    continue
                ref = O.ingest(bits16(k[b]), bits16(v[b]), wl.window, wl.dtype16)
                assert_same_state(to_oracle_state(eng.export(l, b), wl.dtype16), ref,
                                  ema_rtol=0, what=("ingest", l, b))
        del k, v
    worst = 0.0
    # the bench's schedule on the large caches: layer halves as two views of the
    # cache on two concurrent streams, the confidence on a third
    split = wl.n_layers * wl.batch * wl.n_kv_heads >= 2048 and wl.n_layers >= 2
    if split:
        L, h = wl.n_layers, wl.n_layers // 2
        halves = [(0, h), (h, L)]
        views = [eng.layer_view(a, b - a) for a, b in halves]
        main = torch.cuda.current_stream(dev)
        streams = [main, torch.cuda.Stream(dev)]
        side = torch.cuda.Stream(dev)
    budgets, confs = {}, {}
    for step in range(max(CHECKED) + 1):
        check = step in CHECKED
        z = synth.logits(wl, step, SEED, device=dev)
        q = synth.q_new(wl, step, SEED, device=dev)
        k, v = synth.kv_new(wl, step, SEED, device=dev)
        if not check and split:
            for st in streams:
                side.wait_stream(st)
            with torch.cuda.stream(side):
                _, budget = eng.confidence(z)
                cols = [budget[:, a:b].contiguous() for a, b in halves]
            for (a, b), view, st, col in zip(halves, views, streams, cols):
                with torch.cuda.stream(st):
                    view.attend(-1, q[a:b], k[a:b], v[a:b])
                    st.wait_stream(side)
                    view.ema_evict_compact(-1, col)
            for st in (streams[1], side):
                main.wait_stream(st)
            continue
        if not check:
            eng.attend(-1, q, k, v)
            _, budget = eng.confidence(z)
            eng.ema_evict_compact(-1, budget)
            continue
        S0 = {s: eng.export(*s) for s in SAMPLES}
        out = eng.decode_attn(-1, q, k, v)
        S1 = {s: eng.export(*s) for s in SAMPLES}
        c, budget = eng.confidence(z)
        fused = step % 2 == 0
        if fused:
            eng.evict_compact(-1, budget)
        else:
            keep = eng.rank_evict(-1, budget)
            eng.compact_demote(-1, keep)
        _say("  checking step", step)
        S2 = {s: eng.export(*s) for s in SAMPLES}
        budget_h = budget.cpu().numpy()
        budgets[step], confs[step] = budget_h, c.cpu().numpy()
        _check_conf(confs[step], budget_h, z.cpu().numpy().astype(np.float64), wl)
        keep_h = None if fused else keep.cpu().numpy()
        out_h = out.cpu().numpy()
        qb, kb, vb = bits16(q), bits16(k), bits16(v)
        for (l, b) in SAMPLES:
            what = (wl.name, step, l, b)
            st = to_oracle_state(S0[(l, b)], wl.dtype16)
            new_pos = np.append(st.pos, st.t + 1)
            e_gpu = ema_by_pos(S1[(l, b)])
            override = np.array([e_gpu[p] for p in new_pos.tolist()], np.float32)
            r = O.step_layer(st, qb[l, b], kb[l, b], vb[l, b], int(budget_h[b, l]), prm,
                             ema32_override=override)
            err = attn_rel_err(out_h[l, b], r["o"])
            worst = max(worst, err)
            assert err <= ATTN_TOL, (what, err)
            np.testing.assert_allclose(override, r["ema"], rtol=EMA_RTOL, atol=1e-12,
                                       err_msg=str(what))
            if fused:
                got = set(S2[(l, b)]["pos8"].tolist()) | set(S2[(l, b)]["pos16"].tolist())
            else:
                got = kept_positions(S1[(l, b)], keep_h[l, b], eng.cap8)
            assert got == set(new_pos[r["keep"]].tolist()), what
            assert_same_state(to_oracle_state(S2[(l, b)], wl.dtype16), st, ema_rtol=0, what=what)
            _say(f"    {what}: n={len(new_pos)} attention rel err {err:.2e}")
    assert eng.status() == 0
    _say("  worst attention rel err", worst)
    if name.endswith("_stress"):
        gold = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                           "gptoss20b_tau_stress.json")))
        s_, b_ = gold["median_step"], gold["median_seq"]
        # the threshold's own row: c within the tolerance of tau, so both budgets were
        # accepted there and the GPU's choice drove the oracle (teacher forcing)
        assert abs(float(confs[s_][b_]) - wl.tau) <= C_TOL
        z_row = synth.logits(wl, s_, SEED, device=dev)[b_].cpu().numpy().astype(np.float64)
        assert O.confidence(z_row, wl.w_H, wl.w_m, wl.w_p)["c"] == gold["tau"]
        flips = [int((budgets[a][:, 0] != budgets[a + 1][:, 0]).sum())
                 for a in CHECKED if a + 1 in CHECKED]
        _say("  budget flips between consecutive checked steps:", flips)
        assert min(flips) >= 1
    del eng, out, q, k, v, z
    torch.cuda.empty_cache()
