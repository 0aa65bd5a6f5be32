"""Pins of the oracle's INT8 quantiser (textbook symmetric absmax, per channel).

CONF-KV explainer, Methodology, system integration, mixed-precision storage:
the newest W tokens stay 16-bit, older kept tokens are INT8 per head and channel.
"""
import numpy as np
import pytest

from oracle import (LayerSeqState, decode16, demote_token, encode16, ingest, quant_codes,
                    requant_codes)

F32 = np.float32


def test_round_half_even_and_clamp():
    s = np.full(6, F32(1.0))
    x = np.array([2.5, 3.5, -2.5, 200.0, -200.0, 0.49999997], F32)
    assert list(quant_codes(x, s)) == [2, 4, -2, 127, -127, 0]
    assert list(quant_codes(x, np.zeros(6, F32))) == [0] * 6


@pytest.mark.parametrize("seed", range(5))
def test_absmax_maps_to_127_and_error_bound(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((300, 4, 16)) * rng.uniform(0.01, 10)).astype(F32)
    amax = np.abs(x).max(axis=0)
    s = (amax / F32(127)).astype(F32)
    q = quant_codes(x, s)
    assert q.min() >= -127 and q.max() <= 127
    arg = np.abs(x).argmax(axis=0)
    top = np.take_along_axis(q, arg[None], axis=0)[0]
    assert np.all(np.abs(top) == 127)
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * s.astype(np.float64))
    assert np.all(err <= s.astype(np.float64) / 2 * (1 + 1e-6))


def test_requantisation_bound():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(1000).astype(F32)
    s_old = F32(np.abs(x).max() / F32(127))
    q = quant_codes(x, s_old)
    s_new = F32(s_old * F32(1.7))
    q2 = requant_codes(q, s_old, s_new)
    err = np.abs(x.astype(np.float64) - q2.astype(np.float64) * float(s_new))
    assert np.all(err <= (float(s_old) + float(s_new)) / 2 * (1 + 1e-6))


def test_demote_grows_scale_and_requantises():
    codes = np.array([[[127, -64]], [[10, 20]]], np.int8)   # n8 = 2, Hkv = 1, d = 2
    amax = np.array([[1.0, 2.0]], F32)
    x = np.array([[2.0, -1.0]], F32)                        # channel 0 gets a new max
    ck = codes.copy()
    code, amax2 = demote_token(x, amax, ck)
    assert amax2[0, 0] == F32(2.0) and amax2[0, 1] == F32(2.0)
    assert code[0, 0] == 127 and code[0, 1] == -64          # -1/(2/127) = -63.5 -> -64
    # channel 0 codes re-expressed at the doubled scale (half-even): 127 -> 64 (63.5), 10 -> 5
    assert ck[0, 0, 0] == 64 and ck[1, 0, 0] == 5
    assert ck[0, 0, 1] == -64 and ck[1, 0, 1] == 20          # channel 1 untouched


@pytest.mark.parametrize("dtype16", ["f16", "bf16"])
def test_encode_decode_16bit(dtype16):
    x = np.array([1.0, -2.5, 0.0, 1e-3, 3.1415926], F32)
    y = decode16(encode16(x, dtype16), dtype16)
    tol = 2 ** -11 if dtype16 == "f16" else 2 ** -8
    assert np.all(np.abs(y - x) <= tol * np.abs(x))
    assert decode16(encode16(np.array([1.0 + 2 ** -9], F32), "bf16"), "bf16")[0] == 1.0  # tie -> even


def test_ingest_split_and_scales():
    rng = np.random.default_rng(2)
    H, L0, d, W = 2, 40, 8, 16
    k = encode16(rng.standard_normal((H, L0, d)), "bf16")
    v = encode16(rng.standard_normal((H, L0, d)), "bf16")
    st = ingest(k, v, W, "bf16")
    assert st.t == L0 - 1 and st.n == L0
    assert np.array_equal(st.is8, np.arange(L0) < L0 - W)
    xk = decode16(k, "bf16")[:, : L0 - W, :]
    assert np.array_equal(st.amax_k, np.abs(xk).max(axis=1))
    K, _ = st.kv_values()
    s = st.amax_k / F32(127)
    assert np.all(np.abs(K[: L0 - W] - xk.transpose(1, 0, 2)) <= s / 2 * (1 + 1e-6))
    assert np.array_equal(K[L0 - W:], decode16(k, "bf16")[:, L0 - W:, :].transpose(1, 0, 2))


def test_short_prefill_stays_16bit():
    k = encode16(np.ones((1, 5, 4)), "f16")
    st = ingest(k, k, 8, "f16")
    assert not st.is8.any() and np.all(st.amax_k == 0)


def test_state_demotes_position_t_minus_w():
    st = LayerSeqState(1, 4, "f16")
    W = 3
    for i in range(6):
        st.append(encode16(np.full(4, i + 1.0), "f16"), encode16(np.full(4, -(i + 1.0)), "f16"))
        st.demote(W)
    # after step t = 5 the window holds (2, 5]: positions 3, 4, 5
    assert list(st.pos[~st.is8]) == [3, 4, 5] and list(st.pos[st.is8]) == [0, 1, 2]
    K, V = st.kv_values()
    # token 1 was coded at absmax 1, then requantised at absmax 2 and 3: each pass
    # adds at most half a step, so the error is at most (1 + 2 + 3) / 127 / 2
    assert abs(K[0, 0, 0] - 1) <= 6 / 127 / 2 + 1e-6
    assert abs(K[1, 0, 0] - 2) <= 5 / 127 / 2 + 1e-6
    assert K[2, 0, 0] == pytest.approx(3.0 / 127 * 127, abs=1e-6)     # the absmax itself



def _fl32_quotient(x, s):
    """fl32(x / s) with one rounding: the binary64 quotient of two binary32 values
    rounded to binary32 (53 >= 2*24 + 2, so the double rounding is innocuous)."""
    return (np.asarray(x, F32).astype(np.float64) / np.asarray(s, F32).astype(np.float64)).astype(F32)


def _near_halves(rng, n):
    """fp32 pairs (x, s) whose quotient lies within a few ulps of k + 1/2 (k = 0..126):
    the inputs on which the rounding of the quotient decides the code."""
    s = rng.uniform(0.005, 0.05, n).astype(F32)
    k = rng.integers(0, 127, n)
    x = ((k + 0.5) * s.astype(np.float64)).astype(F32)
    step = rng.integers(-3, 4, n)
    for _ in range(3):  # move x by up to three ulps either way
        x = np.where(step > 0, np.nextafter(x, F32(np.inf)), np.where(step < 0, np.nextafter(x, F32(-np.inf)), x))
        step = step - np.sign(step)
    sign = np.where(rng.random(n) < 0.5, F32(-1), F32(1))
    return (x * sign).astype(F32), s


def test_code_is_one_rounded_division_not_a_reciprocal_product():
    """R19 reads the quotient x / s as one fp32 division.  On inputs where that and
    x * fl32(1 / s) round to different codes, the oracle follows the division, both
    for a fresh code and for a requantised one."""
    rng = np.random.default_rng(7)
    x, s = _near_halves(rng, 200_000)
    div = np.clip(np.rint(_fl32_quotient(x, s)), -127, 127)
    recip = np.clip(np.rint((x * (F32(1) / s).astype(F32)).astype(F32)), -127, 127)
    differ = div != recip
    assert differ.sum() >= 100, "the sample must hold cases that tell the two forms apart"
    q = quant_codes(x, s)
    assert np.array_equal(q.astype(np.float64), div)
    # requantisation: clamp(rne(fl32(code * s_old) / s_new)), on products near k + 1/2
    codes = rng.integers(-127, 128, 200_000).astype(np.int8)
    s_old = rng.uniform(0.005, 0.05, codes.shape).astype(F32)
    prod = (codes.astype(F32) * s_old).astype(F32)
    k = np.floor(np.abs(codes.astype(np.float64)) * rng.uniform(0.3, 0.99, codes.shape))
    s_new = (np.abs(prod).astype(np.float64) / (k + 0.5)).astype(F32)
    ok = (codes != 0) & (s_new > s_old)
    codes, s_old, s_new, prod = codes[ok], s_old[ok], s_new[ok], prod[ok]
    div2 = np.clip(np.rint(_fl32_quotient(prod, s_new)), -127, 127)
    recip2 = np.clip(np.rint((prod * (F32(1) / s_new).astype(F32)).astype(F32)), -127, 127)
    assert (div2 != recip2).sum() >= 100
    q2 = requant_codes(codes, s_old, s_new)
    assert np.array_equal(q2.astype(np.float64), div2)
