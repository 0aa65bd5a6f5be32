"""The gpt-oss-20b-shaped stress workload's threshold (CPU only).

Its tau is the oracle's median confidence over the workload's own seeded logits,
written by tests/golden/make_tau_stress.py.  These checks tie the constant in
workloads.py to that file and re-derive its defining row with the oracle."""
import json
import os

import numpy as np

import oracle as O
from adaptive_kv_cache_amd import synth
from adaptive_kv_cache_amd.workloads import TAU_STRESS_GPTOSS, WORKLOADS

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                    "gptoss20b_tau_stress.json")


def test_constant_matches_the_golden_file():
    g = json.load(open(GOLD))
    assert TAU_STRESS_GPTOSS == g["tau_f32"] == float(np.float32(g["tau"]))
    wl = WORKLOADS["gptoss20b_gqa_b32_16k_stress"]
    base = WORKLOADS["gptoss20b_gqa_b32_16k"]
    assert wl.tau == TAU_STRESS_GPTOSS
    # everything but the threshold is the base workload
    assert wl.scaled(tau=base.tau, name=base.name) == base
    assert g["rows"] == base.steps * base.batch


def test_threshold_splits_the_logit_distribution():
    """The golden threshold was computed on logits drawn on the GPU (the bench's);
    the same workload's logits drawn on the CPU have the same distribution, so a
    sample of their oracle confidences falls on both sides of tau, with a median
    close to it.  (The row that sits exactly at tau is checked on the GPU, in the
    full-size test.)"""
    g = json.load(open(GOLD))
    assert g["device"] == "cuda"
    wl = WORKLOADS["gptoss20b_gqa_b32_16k_stress"]
    cs = []
    for step in (3, 200, 411, 500):
        zz = synth.logits(wl, step, 0).numpy().astype(np.float64)
        cs += [O.confidence(zz[b])["c"] for b in range(0, wl.batch, 2)]
    cs = np.array(cs)
    assert (cs >= wl.tau).sum() >= 8 and (cs < wl.tau).sum() >= 8
    assert abs(np.median(cs) - wl.tau) <= 0.03
    assert g["c_min"] <= wl.tau <= g["c_max"]
    assert 0.4 <= g["fraction_at_or_above_tau_f32"] <= 0.6
    assert g["budget_flip_rate"] >= 0.3
