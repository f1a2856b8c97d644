"""Pins of the rotary / packed-QKV oracle (oracle/rotary.py) against facts
that do not retype its formulas:

* the rotation of a pair is complex multiplication by cos + i sin
  (numpy's complex arithmetic), for both pairings;
* an angle of zero is the identity; pair norms are kept; dimensions from
  rotary_dim on pass through bit for bit;
* split pairing is interleaved pairing after de-interleaving the first
  rotary_dim dimensions;
* with RoPE's own tables, scores depend only on the position difference
  (shifting every position leaves attention unchanged), and a sign
  mistake planted in a copy breaks that;
* a pure-Python loop over tokens, heads and pairs equals the vectorised
  oracle;
* the packed layout is Q heads, then K heads, then V heads; the composed
  step writes rotated K and plain V at the block table's slots and returns
  rotated Q; positions are past_b + i.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import rotary as R


def _tables(max_pos, rotary_dim, base=10000.0):
    """RoPE's tables: angle p * base^(-2k / rotary_dim) for pair k."""
    k = np.arange(rotary_dim // 2)
    ang = np.arange(max_pos)[:, None] * base ** (-2.0 * k / rotary_dim)[None, :]
    return np.cos(ang), np.sin(ang)


def _random_tables(rng, max_pos, rotary_dim):
    ang = rng.uniform(-math.pi, math.pi, size=(max_pos, rotary_dim // 2))
    return np.cos(ang), np.sin(ang)


@pytest.mark.parametrize("interleaved", [True, False])
@pytest.mark.parametrize("rdim", [8, 16])
def test_rotation_is_complex_multiplication(interleaved, rdim):
    rng = np.random.default_rng(1)
    T, H, D = 5, 3, 16
    x = rng.uniform(-1, 1, size=(T, H, D))
    cos, sin = _random_tables(rng, 40, rdim)
    pos = rng.integers(0, 40, size=T)
    out = R.rotary_embedding(x, pos, cos, sin, interleaved)
    half = rdim // 2
    if interleaved:
        z = x[..., 0:rdim:2] + 1j * x[..., 1:rdim:2]
    else:
        z = x[..., :half] + 1j * x[..., half:rdim]
    w = z * (cos[pos] + 1j * sin[pos])[:, None, :]
    if interleaved:
        got = out[..., 0:rdim:2] + 1j * out[..., 1:rdim:2]
    else:
        got = out[..., :half] + 1j * out[..., half:rdim]
    np.testing.assert_allclose(got, w, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(out[..., rdim:], x[..., rdim:])   # pass-through


def test_zero_angle_is_identity_and_norms_are_kept():
    rng = np.random.default_rng(2)
    x = rng.uniform(-1, 1, size=(4, 2, 16))
    cos, sin = _tables(9, 16)
    np.testing.assert_array_equal(R.rotary_embedding(x, np.zeros(4, int), cos, sin, True), x)
    np.testing.assert_array_equal(R.rotary_embedding(x, np.zeros(4, int), cos, sin, False), x)
    for inter in (True, False):
        out = R.rotary_embedding(x, np.array([1, 3, 5, 8]), cos, sin, inter)
        a, b = R.pair_indices(16, inter)
        np.testing.assert_allclose(out[..., a] ** 2 + out[..., b] ** 2,
                                   x[..., a] ** 2 + x[..., b] ** 2, rtol=1e-14, atol=1e-15)


def test_split_is_interleaved_after_deinterleaving():
    rng = np.random.default_rng(3)
    D, rdim = 16, 12
    x = rng.uniform(-1, 1, size=(3, 2, D))
    cos, sin = _random_tables(rng, 10, rdim)
    pos = np.array([0, 4, 9])
    perm = np.arange(D)
    perm[0:rdim:2] = np.arange(rdim // 2)               # slot 2k takes dim k
    perm[1:rdim:2] = np.arange(rdim // 2) + rdim // 2   # slot 2k+1 takes dim k + R/2
    inter = R.rotary_embedding(x[..., perm], pos, cos, sin, True)
    back = np.empty_like(inter)
    back[..., perm] = inter
    np.testing.assert_allclose(R.rotary_embedding(x, pos, cos, sin, False), back, rtol=0,
                               atol=1e-15)


def _shifted_attention(interleaved, shift, rotate=R.rotary_embedding):
    """Attention of a 3-token chunk over a 20-key sequence with RoPE applied
    to Q and to every key at its position, all positions shifted by `shift`."""
    rng = np.random.default_rng(4)
    hq, hk, d, bs = 4, 2, 16, 4
    L, ql = 20, 3
    cos, sin = _tables(64, d)
    k_all = rng.uniform(-1, 1, size=(L, hk, d))
    v_all = rng.uniform(-1, 1, size=(L, hk, d))
    q = rng.uniform(-1, 1, size=(ql, hq, d))
    k_rot = rotate(k_all, np.arange(L) + shift, cos, sin, interleaved)
    q_rot = rotate(q, np.arange(L - ql, L) + shift, cos, sin, interleaved)
    nb = L // bs
    kc = k_rot.reshape(nb, bs, hk, d)
    vc = v_all.reshape(nb, bs, hk, d)
    table = np.arange(nb)[None, :]
    return oracle.attention(q_rot, np.array([0, ql]), np.array([L]), table, kc, vc, 0.5, hq, hk,
                            bs)


@pytest.mark.parametrize("interleaved", [True, False])
def test_attention_depends_on_position_differences_only(interleaved):
    a = _shifted_attention(interleaved, 0)
    for s in (1, 7, 30):
        np.testing.assert_allclose(_shifted_attention(interleaved, s), a, rtol=1e-12,
                                   atol=1e-12)


def test_planted_sign_mistake_breaks_translation_invariance():
    """Rotating by x_a cos + x_b sin (the sign on the wrong element) in a
    copy of the step, on the CPU: shifted positions then change the result."""
    def wrong(x, positions, cos_cache, sin_cache, interleaved):
        x = np.asarray(x, dtype=np.float64)
        cos = cos_cache[positions][:, None, :]
        sin = sin_cache[positions][:, None, :]
        a, b = R.pair_indices(2 * cos.shape[-1], interleaved)
        out = x.copy()
        out[..., a] = x[..., a] * cos + x[..., b] * sin
        out[..., b] = x[..., b] * cos + x[..., a] * sin
        return out
    a = _shifted_attention(True, 0, wrong)
    b = _shifted_attention(True, 7, wrong)
    assert np.abs(a - b).max() > 1e-3


def _loops(x, positions, cos, sin, interleaved):
    T, H, D = x.shape
    rdim = 2 * cos.shape[1]
    out = [[list(map(float, x[t, h])) for h in range(H)] for t in range(T)]
    for t in range(T):
        p = int(positions[t])
        for h in range(H):
            for k in range(rdim // 2):
                ia, ib = (2 * k, 2 * k + 1) if interleaved else (k, k + rdim // 2)
                xa, xb = float(x[t, h, ia]), float(x[t, h, ib])
                c, s = float(cos[p, k]), float(sin[p, k])
                out[t][h][ia] = xa * c - xb * s
                out[t][h][ib] = xb * c + xa * s
    return np.array(out)


@pytest.mark.parametrize("interleaved", [True, False])
def test_loops_equal_vectorised(interleaved):
    rng = np.random.default_rng(5)
    x = rng.uniform(-1, 1, size=(6, 3, 16))
    cos, sin = _random_tables(rng, 12, 8)
    pos = rng.integers(0, 12, size=6)
    np.testing.assert_array_equal(R.rotary_embedding(x, pos, cos, sin, interleaved),
                                  _loops(x, pos, cos, sin, interleaved))


def test_positions_and_packed_layout():
    cu = np.array([0, 3, 3, 4])
    lens = np.array([10, 2, 1])
    np.testing.assert_array_equal(R.token_positions(cu, lens), [7, 8, 9, 0])
    T, hq, hk, d = 4, 4, 2, 3
    q = np.arange(T * hq * d).reshape(T, hq, d)
    k = 1000 + np.arange(T * hk * d).reshape(T, hk, d)
    v = 2000 + np.arange(T * hk * d).reshape(T, hk, d)
    packed = np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], axis=1)
    q2, k2, v2 = R.split_packed_qkv(packed, hq, hk)
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(k2, k)
    np.testing.assert_array_equal(v2, v)


@pytest.mark.parametrize("packed", [False, True])
def test_composed_step(packed):
    """Rotated K and plain V land at the slots of positions past_b + i;
    the returned Q is rotated Q; without tables it is the plain scatter."""
    rng = np.random.default_rng(6)
    hq, hk, d, bs, nb = 4, 2, 8, 4, 8
    cu = np.array([0, 2, 5])
    lens = np.array([6, 3])
    table = np.array([[5, 1], [2, 7]])
    T = 5
    q = rng.uniform(-1, 1, size=(T, hq, d))
    k = rng.uniform(-1, 1, size=(T, hk, d))
    v = rng.uniform(-1, 1, size=(T, hk, d))
    cos, sin = _random_tables(rng, 16, 8)
    args = (np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], axis=1),
            None, None) if packed else (q, k, v)
    kc = np.full((nb, bs, hk, d), np.nan)
    vc = np.full((nb, bs, hk, d), np.nan)
    q_out = R.rotary_scatter_kv(*args, cos, sin, False, cu, lens, table, kc, vc, bs, hq, hk)
    pos = np.array([4, 5, 0, 1, 2])
    np.testing.assert_array_equal(q_out, R.rotary_embedding(q, pos, cos, sin, False))
    k_rot = R.rotary_embedding(k, pos, cos, sin, False)
    where = [(1, 0), (1, 1), (2, 0), (2, 1), (2, 2)]   # block table entries of each position
    for t, (blk, off) in enumerate(where):
        np.testing.assert_array_equal(kc[blk, off], k_rot[t])
        np.testing.assert_array_equal(vc[blk, off], v[t])
    assert np.isnan(kc[5]).all() and np.isnan(kc[7]).all()
    kc2 = np.full((nb, bs, hk, d), np.nan)
    vc2 = np.full((nb, bs, hk, d), np.nan)
    q_plain = R.rotary_scatter_kv(*args, None, None, False, cu, lens, table, kc2, vc2, bs, hq, hk)
    np.testing.assert_array_equal(q_plain, q)
    np.testing.assert_array_equal(kc2[1, 0], k[0])
    with pytest.raises(ValueError):
        R.rotary_scatter_kv(*args, cos[:5], sin[:5], False, cu, lens, table, kc, vc, bs, hq, hk)
