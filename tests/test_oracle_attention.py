"""Pins of the oracle's attention, token-mass and EMA steps.

CONF-KV explainer, Key contributions (system design: block-wise online-softmax
attention) and Methodology (implementation: dequantisation fused into the
block-wise attention reads; token ranking: EMA attention mass).
"""
import math

import numpy as np
import pytest
import torch

from oracle import (attention, attention_online, dequantize, ema_update, quant_codes,
                    token_mass)


def _rand(n, Hq, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((Hq, d)), rng.standard_normal((n, Hkv, d)),
            rng.standard_normal((n, Hkv, d)))


@pytest.mark.parametrize("n,Hq,Hkv,d", [(1, 4, 4, 8), (37, 5, 1, 16), (200, 40, 8, 32),
                                        (129, 12, 12, 64), (513, 8, 2, 128)])
def test_matches_torch_sdpa(n, Hq, Hkv, d):
    # A library routine computes the same softmax attention independently.
    q, K, V = _rand(n, Hq, Hkv, d, n + d)
    o, p = attention(q, K, V, Hq // Hkv)
    g = Hq // Hkv
    Kt = torch.from_numpy(np.repeat(K, g, axis=1)).permute(1, 0, 2)[None]   # [1,Hq,n,d]
    Vt = torch.from_numpy(np.repeat(V, g, axis=1)).permute(1, 0, 2)[None]
    qt = torch.from_numpy(q)[None, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt)[0, :, 0, :].numpy()
    assert np.max(np.abs(o - ref)) < 1e-12
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-13)


@pytest.mark.parametrize("block", [1, 7, 64, 100, 1000])
def test_online_blockwise_equals_two_pass(block):
    q, K, V = _rand(333, 10, 2, 32, block)
    K[17] *= 6.0      # a late maximum forces rescaling in the running sums
    K[300] *= 5.0
    o, _ = attention(q, K, V, 5)
    assert np.max(np.abs(attention_online(q, K, V, 5, block) - o)) < 1e-12


def test_single_token_returns_its_value():
    q, K, V = _rand(1, 6, 3, 16, 3)
    o, p = attention(q, K, V, 2)
    assert np.allclose(p, 1.0)
    assert np.max(np.abs(o - np.repeat(V[0], 2, axis=0))) < 1e-15


def test_equal_keys_or_zero_query_average_values():
    q, K, V = _rand(50, 4, 2, 16, 4)
    K[:] = K[0]
    o, _ = attention(q, K, V, 2)
    assert np.max(np.abs(o - np.repeat(V.mean(axis=0), 2, axis=0))) < 1e-13
    q2, K2, V2 = _rand(50, 4, 2, 16, 5)
    o2, _ = attention(np.zeros_like(q2), K2, V2, 2)
    assert np.max(np.abs(o2 - np.repeat(V2.mean(axis=0), 2, axis=0))) < 1e-13


def test_permutation_invariance():
    q, K, V = _rand(90, 8, 4, 16, 6)
    perm = np.random.default_rng(0).permutation(90)
    o, p = attention(q, K, V, 2)
    o2, p2 = attention(q, K[perm], V[perm], 2)
    assert np.max(np.abs(o - o2)) < 1e-13
    assert np.max(np.abs(p[:, perm] - p2)) < 1e-15


def test_group_mapping_reads_kv_head_h_div_g():
    # Query head h must read KV head h // g: make KV head 1 hold a distinct value.
    q, K, V = _rand(20, 6, 3, 8, 7)
    V[:, 1, :] = 5.0
    o, _ = attention(q, K, V, 2)
    assert np.allclose(o[2:4], 5.0) and not np.allclose(o[0], 5.0)


def test_fused_dequant_equals_dequant_then_attend():
    # Per-channel scales fold into the query (keys) and the output (values):
    # q.(code*sK) = (q*sK).code and sum_j p_j code_j sV = sV * sum_j p_j code_j.
    rng = np.random.default_rng(8)
    n, Hq, Hkv, d = 77, 6, 2, 32
    x_k = rng.standard_normal((n, Hkv, d)).astype(np.float32)
    x_v = rng.standard_normal((n, Hkv, d)).astype(np.float32)
    ak = np.abs(x_k).max(axis=0)
    av = np.abs(x_v).max(axis=0)
    ck = quant_codes(x_k, ak / np.float32(127))
    cv = quant_codes(x_v, av / np.float32(127))
    q = rng.standard_normal((Hq, d))
    o_ref, _ = attention(q, dequantize(ck, ak), dequantize(cv, av), 3)
    sk = (ak / np.float32(127)).astype(np.float64)
    sv = (av / np.float32(127)).astype(np.float64)
    o = np.zeros((Hq, d))
    for h in range(Hq):
        hk = h // 3
        sig = (ck[:, hk, :].astype(np.float64) @ (q[h] * sk[hk])) / math.sqrt(d)
        w = np.exp(sig - sig.max())
        o[h] = sv[hk] * (w @ cv[:, hk, :].astype(np.float64)) / w.sum()
    assert np.max(np.abs(o - o_ref)) < 1e-13


def test_token_mass_is_a_distribution():
    q, K, V = _rand(64, 8, 2, 16, 9)
    _, p = attention(q, K, V, 4)
    m = token_mass(p)
    assert abs(m.sum() - 1.0) < 1e-13 and np.all(m > 0)
    assert np.allclose(m, p.mean(axis=0))


def test_ema_closed_form():
    # Constant mass a for k steps from e = 0: e_k = a (1 - decay^k).
    a, decay = 0.0123, 0.9
    e = np.zeros(3)
    for k in range(1, 40):
        e = ema_update(e, np.full(3, a), decay)
        assert np.allclose(e, a * (1 - decay ** k), rtol=1e-13, atol=0)
    # A token that stops receiving mass decays geometrically.
    e2 = ema_update(e, np.zeros(3), decay)
    assert np.allclose(e2, decay * e, rtol=1e-15)
