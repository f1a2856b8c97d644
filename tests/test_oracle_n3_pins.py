"""Pins of the oracle's sliding window (local_window_size) and score soft cap
(softcap) against closed forms, special cases that reduce to the plain
routine, and brute force:

* window >= every length changes nothing; window 1 returns the row's own
  V row exactly; window W equals plain attention over the sequence's last
  W keys (a shorter cache), for decode rows;
* a cap far above every score changes nothing (to 1e-12); with scores
  saturated at +-cap the weights of two keys are the closed form
  1 / (1 + e^(-2 cap)); equal scores stay a plain mean;
* the pure-Python loops (scalar math.tanh, a key range) equal the
  vectorised oracle with both options on; incremental decoding (each new
  row as its own q_len=1 step) equals the chunk with both options on.
"""
import math

import numpy as np
import pytest

import oracle


def _batch(rng, q_lens, lens, hq, hk, d, bs):
    q_lens = np.asarray(q_lens)
    lens = np.asarray(lens)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    need = -(-lens // bs)
    nb = int(need.sum()) + 2
    perm = rng.permutation(nb)
    table = np.zeros((len(lens), int(need.max())), np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    kc = rng.uniform(-1, 1, size=(nb, bs, hk, d))
    vc = rng.uniform(-1, 1, size=(nb, bs, hk, d))
    q = rng.uniform(-1, 1, size=(int(cu[-1]), hq, d))
    return q, cu, lens, table, kc, vc


def test_window_covering_everything_changes_nothing():
    rng = np.random.default_rng(1)
    q, cu, lens, table, kc, vc = _batch(rng, [1, 3, 2], [9, 20, 5], 4, 2, 8, 4)
    a = oracle.attention(q, cu, lens, table, kc, vc, 0.3, 4, 2, 4)
    b = oracle.attention(q, cu, lens, table, kc, vc, 0.3, 4, 2, 4, local_window_size=20)
    np.testing.assert_array_equal(a, b)


def test_window_one_is_the_rows_own_value():
    rng = np.random.default_rng(2)
    q, cu, lens, table, kc, vc = _batch(rng, [1, 3, 2], [9, 20, 5], 4, 2, 8, 4)
    out = oracle.attention(q, cu, lens, table, kc, vc, 0.3, 4, 2, 4, local_window_size=1)
    for b in range(len(lens)):
        ql = int(cu[b + 1] - cu[b])
        past = int(lens[b]) - ql
        for i in range(ql):
            j = past + i
            blk = table[b, j // 4]
            for h in range(4):
                np.testing.assert_array_equal(out[cu[b] + i, h], vc[blk, j % 4, h // 2])


@pytest.mark.parametrize("W", [1, 3, 7, 16])
def test_window_equals_attention_over_the_last_w_keys(W):
    """Decode rows: the window is plain attention over a cache that holds
    only the sequence's last W keys (a different block table and length)."""
    rng = np.random.default_rng(3)
    bs = 4
    q, cu, lens, table, kc, vc = _batch(rng, [1, 1, 1], [9, 23, 30], 6, 3, 8, bs)
    got = oracle.attention(q, cu, lens, table, kc, vc, 0.25, 6, 3, bs, local_window_size=W)
    for b in range(3):
        L = int(lens[b])
        keep = list(range(max(0, L - W), L))
        kk = np.stack([kc[table[b, j // bs], j % bs] for j in keep])[:, None]
        vv = np.stack([vc[table[b, j // bs], j % bs] for j in keep])[:, None]
        n = len(keep)
        tab = np.arange(n, dtype=np.int32)[None, :]
        want = oracle.attention(q[cu[b]:cu[b + 1]], np.array([0, 1], np.int32),
                                np.array([n], np.int32), tab, kk, vv, 0.25, 6, 3, 1)
        np.testing.assert_allclose(got[cu[b]:cu[b + 1]], want, rtol=1e-13, atol=1e-13)


def test_huge_cap_changes_nothing():
    rng = np.random.default_rng(4)
    q, cu, lens, table, kc, vc = _batch(rng, [2, 1], [12, 30], 4, 4, 8, 4)
    a = oracle.attention(q, cu, lens, table, kc, vc, 0.5, 4, 4, 4)
    b = oracle.attention(q, cu, lens, table, kc, vc, 0.5, 4, 4, 4, softcap=1e9)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("cap", [0.5, 2.0, 7.0])
def test_saturated_scores_give_closed_form_weights(cap):
    """Two keys whose scaled scores are +1e4 and -1e4: capped to +cap and
    -cap, so the weights are 1/(1+e^-2cap) and e^-2cap/(1+e^-2cap)."""
    d = 4
    q = np.zeros((1, 1, d)); q[0, 0, 0] = 100.0
    kc = np.zeros((1, 2, 1, d)); kc[0, 0, 0, 0] = 1.0; kc[0, 1, 0, 0] = -1.0
    vc = np.zeros((1, 2, 1, d)); vc[0, 0, 0] = [1, 2, 3, 4]; vc[0, 1, 0] = [-5, 0, 5, 10]
    out = oracle.attention(q, np.array([0, 1]), np.array([2]), np.array([[0]]), kc, vc, 100.0,
                           1, 1, 2, softcap=cap)
    p1 = 1.0 / (1.0 + math.exp(-2.0 * cap))
    want = p1 * vc[0, 0, 0] + (1 - p1) * vc[0, 1, 0]
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-14, atol=1e-14)
    # without the cap the first key takes everything
    np.testing.assert_allclose(oracle.attention(q, np.array([0, 1]), np.array([2]),
                                                np.array([[0]]), kc, vc, 100.0, 1, 1, 2)[0, 0],
                               vc[0, 0, 0], rtol=0, atol=1e-12)


def test_cap_keeps_equal_scores_a_mean():
    d = 4
    q = np.zeros((1, 1, d))
    rng = np.random.default_rng(5)
    kc = rng.uniform(-1, 1, size=(1, 4, 1, d))
    vc = rng.uniform(-1, 1, size=(1, 4, 1, d))
    out = oracle.attention(q, np.array([0, 1]), np.array([4]), np.array([[0]]), kc, vc, 1.0, 1,
                           1, 4, softcap=0.7)
    np.testing.assert_allclose(out[0, 0], vc[0, :, 0].mean(axis=0), rtol=1e-14, atol=1e-15)


def test_loops_equal_vectorised_with_both_options():
    rng = np.random.default_rng(6)
    q, cu, lens, table, kc, vc = _batch(rng, [1, 3, 0, 2], [7, 11, 3, 5], 4, 2, 8, 4)
    for cap, W in ((0.8, 3), (3.0, 1), (0.0, 4), (1.5, 0)):
        a = oracle.attention(q, cu, lens, table, kc, vc, 0.4, 4, 2, 4, softcap=cap,
                             local_window_size=W)
        b = oracle.attention_loops(q, cu, lens, table, kc, vc, 0.4, 4, 2, 4, softcap=cap,
                                   local_window_size=W)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_incremental_decoding_with_both_options():
    rng = np.random.default_rng(7)
    q, cu, lens, table, kc, vc = _batch(rng, [5], [19], 4, 2, 8, 4)
    chunk = oracle.attention(q, cu, lens, table, kc, vc, 0.3, 4, 2, 4, softcap=1.2,
                             local_window_size=6)
    past = 19 - 5
    for i in range(5):
        row = oracle.attention(q[i:i + 1], np.array([0, 1]), np.array([past + i + 1]), table,
                               kc, vc, 0.3, 4, 2, 4, softcap=1.2, local_window_size=6)
        np.testing.assert_allclose(row[0], chunk[i], rtol=1e-13, atol=1e-13)
