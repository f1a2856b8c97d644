"""Pins of the fp8 (e4m3) cache oracle (oracle/kv_fp8.py) against facts
fixed by the format's definition and by arithmetic, not by retyping the
oracle's formulas:

* the value set: 254 finite codes (126 positive magnitudes, signed zeros),
  strictly increasing over codes 0..126, largest 448, smallest subnormal
  2^-9, smallest normal 2^-6, powers of two at exponent-field boundaries,
  sign symmetry;
* rounding: against brute force (nearest of all finite values, ties to the
  even code) on a dense sweep; round trip of every finite code;
  saturation and NaN;
* quantization error within half a grid step (relative 2^-4 in the normal
  range), and exactness for values on the scaled grid with power-of-two
  scales;
* the scatter's slot handling and the attention composition (exactly the
  16-bit oracle over the dequantized values).
"""
import numpy as np
import pytest

import oracle
from oracle import kv_fp8 as F

CODES = np.arange(256, dtype=np.uint8)


def _finite_codes():
    v = F.e4m3_decode(CODES)
    return CODES[~np.isnan(v)], v[~np.isnan(v)]


def test_value_set():
    codes, vals = _finite_codes()
    assert len(codes) == 254                       # 0x7F and 0xFF are NaN
    assert np.isnan(F.e4m3_decode([0x7F, 0xFF])).all()
    pos = F.e4m3_decode(np.arange(127, dtype=np.uint8))
    assert (np.diff(pos) > 0).all()                # monotone magnitudes
    assert pos[0] == 0.0 and pos[-1] == 448.0
    assert pos[1] == 2.0 ** -9 and pos[8] == 2.0 ** -6 and pos[7] == 7 * 2.0 ** -9
    # one binade per exponent field: codes 8e..8e+7 span [2^(e-7), 2^(e-6))
    for e in range(1, 16):
        assert pos[8 * e] == 2.0 ** (e - 7)
    assert F.e4m3_decode([0x38])[0] == 1.0 and F.e4m3_decode([0xB8])[0] == -1.0
    np.testing.assert_array_equal(F.e4m3_decode(CODES[:127] | 0x80), -pos)
    assert np.signbit(F.e4m3_decode([0x80])[0])


def test_round_trip_every_finite_code():
    codes, vals = _finite_codes()
    np.testing.assert_array_equal(F.e4m3_encode(vals.astype(np.float32)), codes)


def _brute_force(x):
    """Nearest finite e4m3 value by exhaustive search; ties to the even code."""
    codes, vals = _finite_codes()
    out = []
    for xi in np.asarray(x, dtype=np.float64):
        if np.isnan(xi):
            out.append(0xFF)
            continue
        a = min(abs(xi), 448.0)
        best, bestc = None, None
        for c, v in zip(codes, vals):
            if c & 0x80 or (v != abs(v)):
                continue
            d = abs(v - a)
            if best is None or d < best or (d == best and (c & 1) == 0):
                best, bestc = d, int(c)
        out.append(bestc | (0x80 if np.signbit(xi) else 0))
    return np.array(out, dtype=np.uint8)


def test_rounding_matches_brute_force():
    rng = np.random.default_rng(5)
    codes, vals = _finite_codes()
    pos = np.sort(vals[vals > 0])
    mids = (pos[:-1] + pos[1:]) / 2                 # exact ties
    x = np.concatenate([
        rng.uniform(-500, 500, 3000), rng.uniform(-0.05, 0.05, 2000),
        rng.uniform(-2 ** -6, 2 ** -6, 1000), mids, -mids,
        np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
        np.nextafter(mids.astype(np.float32), np.float32(0)),
        [0.0, -0.0, 448.0, 449.0, 464.0, 465.0, 1e30, np.inf, -np.inf, 2.0 ** -10]]).astype(np.float32)
    np.testing.assert_array_equal(F.e4m3_encode(x), _brute_force(x))


def test_saturation_and_nan():
    e = F.e4m3_encode(np.array([448.5, 1e6, np.inf, -np.inf, -1e6, np.nan], dtype=np.float32))
    assert list(e) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0xFF]


def test_quantization_error_bound():
    """|dequantize(quantize(x)) - x| <= half a grid step: relative 2^-4 when
    |x / s| lies in the normal range, absolute 2^-10 * s below it (the
    float32 rounding of x * (1/s) adds at most a relative 2^-23)."""
    rng = np.random.default_rng(6)
    s = rng.uniform(0.002, 0.05, size=(4, 32)).astype(np.float32)
    x = (rng.uniform(-1.0, 1.0, size=(500, 4, 32)) * rng.choice([1e-3, 0.1, 1.0, 10.0],
                                                                size=(500, 1, 1))).astype(np.float32)
    y = np.abs(x.astype(np.float64) / s.astype(np.float64))
    xq = F.dequantize(F.quantize(x, s), s)
    err = np.abs(xq - x)
    s64 = np.broadcast_to(s.astype(np.float64), x.shape)
    normal = (y >= 2.0 ** -6) & (y <= 448.0)
    assert (err[normal] <= np.abs(x[normal]) * (2.0 ** -4 + 1e-6)).all()
    assert (err[y < 2.0 ** -6] <= s64[y < 2.0 ** -6] * (2.0 ** -10 + 1e-9)).all()
    big = y > 448.0 * (1 + 2.0 ** -20)
    assert np.allclose(np.abs(xq[big]), 448.0 * s64[big], rtol=0, atol=0)


def test_grid_values_with_power_of_two_scales_are_exact():
    codes, vals = _finite_codes()
    for k in (-8, -3, 0, 2):
        s = np.float32(2.0 ** k)
        np.testing.assert_array_equal(F.quantize((vals * 2.0 ** k).astype(np.float32), s), codes)


def test_scatter_fp8_slots_and_skip():
    rng = np.random.default_rng(7)
    hk, d, bs, nb = 2, 16, 4, 3
    ks = rng.uniform(0.01, 0.02, size=(hk, d)).astype(np.float32)
    vs = rng.uniform(0.01, 0.02, size=(hk, d)).astype(np.float32)
    kn = rng.uniform(-1, 1, size=(3, hk, d)).astype(np.float32)
    vn = rng.uniform(-1, 1, size=(3, hk, d)).astype(np.float32)
    kc = np.full((nb, bs, hk, d), 0x7F, np.uint8)
    vc = np.full((nb, bs, hk, d), 0x7F, np.uint8)
    F.scatter_kv_fp8(kn, vn, np.array([5, -1, 11]), ks, vs, kc, vc, bs)
    np.testing.assert_array_equal(kc[1, 1], F.quantize(kn[0], ks))
    np.testing.assert_array_equal(vc[2, 3], F.quantize(vn[2], vs))
    touched = np.zeros((nb, bs), bool)
    touched[1, 1] = touched[2, 3] = True
    assert (kc[~touched] == 0x7F).all() and (vc[~touched] == 0x7F).all()


def test_attention_fp8_is_attention_over_dequantized_values():
    """Caches whose values sit on the scaled e4m3 grid: fp8 attention equals
    the 16-bit oracle over those values exactly, for a mixed batch."""
    rng = np.random.default_rng(8)
    hq, hk, d, bs = 4, 2, 16, 4
    lens = np.array([5, 9, 1])
    q_lens = np.array([1, 3, 1])
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    nb = 10
    table = np.array([[0, 1, 2], [3, 4, 5], [6, 7, 8]], dtype=np.int32)
    codes_k = rng.integers(0, 256, size=(nb, bs, hk, d)).astype(np.uint8)
    codes_v = rng.integers(0, 256, size=(nb, bs, hk, d)).astype(np.uint8)
    codes_k[(codes_k & 0x7F) == 0x7F] = 0x38   # no NaN codes
    codes_v[(codes_v & 0x7F) == 0x7F] = 0x38
    codes_k &= 0xBF                            # exponent field <= 7: magnitudes below 2
    codes_v &= 0xBF
    ks = np.exp2(rng.integers(-6, -2, size=(hk, d))).astype(np.float32)
    vs = rng.uniform(0.5, 2.0, size=(hk, d)).astype(np.float32)
    q = rng.uniform(-1, 1, size=(int(cu[-1]), hq, d))
    got = F.attention_fp8(q, cu, lens, table, codes_k, codes_v, ks, vs, 0.25, hq, hk, bs)
    want = oracle.attention(q, cu, lens, table, F.dequantize(codes_k, ks),
                            F.dequantize(codes_v, vs), 0.25, hq, hk, bs)
    np.testing.assert_array_equal(got, want)
    # and a per-channel K scale is the same as scaling that channel of q
    ks2 = ks.copy()
    ks2[0, 3] *= 2
    got2 = F.attention_fp8(q, cu, lens, table, codes_k, codes_v, ks2, vs, 0.25, hq, hk, bs)
    q2 = q.copy()
    q2[:, 0:2, 3] *= 2                         # heads 0, 1 read KV head 0
    np.testing.assert_allclose(got2, F.attention_fp8(q2, cu, lens, table, codes_k, codes_v, ks,
                                                     vs, 0.25, hq, hk, bs), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bad", ["channel_order", "no_inv"])
def test_planted_mistakes_fail(bad):
    """Mistakes a reader could make in quantize() break the error bound
    (planted here on the CPU, in a copy of the oracle's steps)."""
    rng = np.random.default_rng(9)
    s = rng.uniform(0.01, 0.05, size=(2, 8)).astype(np.float32)
    x = rng.uniform(-1, 1, size=(64, 2, 8)).astype(np.float32)
    if bad == "channel_order":                 # scales of the wrong channel
        wrong = F.dequantize(F.quantize(x, s[:, ::-1]), s)
    else:                                      # multiply by the scale
        wrong = F.dequantize(F.e4m3_encode((x * s).astype(np.float32)), s)
    right = F.dequantize(F.quantize(x, s), s)
    assert np.abs(right - x).max() <= np.abs(x).max() * 2.0 ** -4 + 1e-6
    assert np.abs(wrong - x).max() > np.abs(x).max() * 2.0 ** -4
