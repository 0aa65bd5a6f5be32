"""Pins of the oracle's confidence and budget steps against closed forms.

CONF-KV explainer, Methodology, confidence estimation and adaptive budget
selection: c = w_H(1 - H^) + w_m sigma(m) + w_p p(1) with weights (0.4, 0.3, 0.3);
c >= tau picks N_high, c < tau picks N_low; CONF-KV-L spreads budgets over layers.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import budget, confidence, layer_budget

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "confkv_page_constants.json")


def test_default_weights_are_the_pages():
    w = json.load(open(GOLDEN))["confidence_weights"]
    import inspect
    sig = inspect.signature(confidence).parameters
    assert (sig["w_H"].default, sig["w_m"].default, sig["w_p"].default) == (
        w["w_H"], w["w_m"], w["w_p"])


@pytest.mark.parametrize("V", [2, 7, 50257, 152064])
def test_uniform_logits(V):
    # Uniform: H = ln V so H^ = 1, m = 0 so sigma = 1/2, p(1) = 1/V.
    r = confidence(np.full(V, 3.25))
    assert abs(r["H_hat"] - 1.0) < 1e-12
    assert r["m"] == 0.0
    assert abs(r["c"] - (0.15 + 0.3 / V)) < 1e-12


def test_uniform_value_at_gpt2_vocab():
    assert abs(confidence(np.zeros(50257))["c"] - 0.150005969) < 1e-9


def test_one_hot_gap_100_is_one():
    z = np.zeros(50257)
    z[1234] = 100.0
    r = confidence(z)
    assert abs(r["c"] - 1.0) < 1e-12
    assert r["m"] == 100.0


@pytest.mark.parametrize("k,a,b,V", [(1, 2.0, 0.0, 1000), (1, 0.3, -1.7, 17),
                                     (3, 1.5, 0.5, 5000), (40, 0.0, -2.0, 100),
                                     (1, 9.0, 0.0, 152064)])
def test_two_level_closed_form(k, a, b, V):
    # k logits at a, V-k at b (a > b).  With x = e^(b-a) and D = k + (V-k) x:
    # p_a = 1/D, p_b = x/D, H = ln D - (V-k) x (b-a) / D, m = a-b if k == 1 else 0.
    z = np.full(V, b, dtype=np.float64)
    z[:k] = a
    np.random.default_rng(k + V).shuffle(z)
    x = math.exp(b - a)
    D = k + (V - k) * x
    H = math.log(D) - (V - k) * x * (b - a) / D
    m = (a - b) if k == 1 else 0.0
    c = 0.4 * (1 - H / math.log(V)) + 0.3 / (1 + math.exp(-m)) + 0.3 / D
    r = confidence(z)
    assert abs(r["H_hat"] - H / math.log(V)) < 1e-12
    assert abs(r["p1"] - 1 / D) < 1e-12
    assert r["m"] == pytest.approx(m, abs=1e-12)
    assert abs(r["c"] - c) < 1e-12


def test_shift_and_permutation_invariance():
    rng = np.random.default_rng(0)
    z = rng.standard_normal(10007) * 3
    c0 = confidence(z)["c"]
    assert abs(confidence(z + 17.5)["c"] - c0) < 1e-12
    assert abs(confidence(rng.permutation(z))["c"] - c0) < 1e-12


@pytest.mark.parametrize("T", [0.1, 0.5, 1, 2, 8, 30])
def test_bounds(T):
    V = 4099
    z = np.random.default_rng(int(T * 10)).standard_normal(V) * T
    c = confidence(z)["c"]
    assert 0.15 + 0.3 / V - 1e-12 <= c <= 1.0 + 1e-12


def test_temperature_moves_c_across_tau():
    # Logits N(0,1)*T: a small multiplier gives a flat, unconfident distribution
    # and a large one a peaked distribution.
    rng = np.random.default_rng(1)
    z = rng.standard_normal(50257)
    assert confidence(0.5 * z)["c"] < 0.5 < confidence(8.0 * z)["c"]


def test_non_finite_gives_nan_and_loose_budget():
    z = np.zeros(100)
    z[3] = np.nan
    c = confidence(z)["c"]
    assert math.isnan(c)
    assert budget(c, 0.5, 10, 20) == 20
    z[3] = np.inf
    assert math.isnan(confidence(z)["c"])


def test_budget_rule_and_tie():
    assert budget(0.5, 0.5, 384, 768) == 384          # c = tau is "c >= tau"
    assert budget(0.5 - 1e-9, 0.5, 384, 768) == 768
    assert budget(0.9, 0.5, 384, 768) == 384


def test_pyramid_budgets():
    L = 12
    got = [layer_budget(384, l, L, True) for l in range(L)]
    assert got[0] == 384 and got[-1] == 192
    assert all(a >= b for a, b in zip(got, got[1:]))
    # floor(384 * (22 - l) / 22) written out for l = 1 and l = 5
    assert got[1] == 366 and got[5] == 296
    assert [layer_budget(777, l, L, False) for l in range(L)] == [777] * L
    assert layer_budget(100, 0, 1, True) == 100
    assert layer_budget(4097, 63, 64, True) == 2048
