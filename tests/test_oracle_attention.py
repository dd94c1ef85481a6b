"""Pins of the oracle's sparse core attention over the top-k: hand-computed
cases, softmax special cases (one token, equal scores, scale 0), a
pure-Python loop on small shapes, invariance under the order of the top-k
list and under a shift of all scores, and the page indirection."""
import math

import numpy as np
import pytest

from oracle import spin_oracle as O

NEG = float("-inf")


def _pool(rng, pages, d):
    return rng.normal(size=(pages, 64, d))


def test_one_token_returns_its_value():
    rng = np.random.default_rng(0)
    kv = _pool(rng, 3, 6)
    table = np.array([2, 0, 1])
    q = rng.normal(size=(2, 6))
    o, lse = O.sparse_attention(q, kv, table, [70, -1, -1], 100, 0.5, 4)
    row = kv[table[1], 6]                                  # slot 70: block 1, row 6
    assert np.allclose(o, np.tile(row[:4], (2, 1)), rtol=0, atol=1e-15)
    assert np.allclose(lse, 0.5 * q @ row, rtol=1e-15)


def test_hand_case():
    # one head, d = 2, d_v = 1; keys (1, 0) and (0, 1) in slots 0 and 1
    kv = np.zeros((1, 64, 2))
    kv[0, 0] = [1.0, 0.0]
    kv[0, 1] = [0.0, 1.0]
    q = np.array([[math.log(3.0), 0.0]])                   # scores log 3 and 0
    o, lse = O.sparse_attention(q, kv, [0], [0, 1], 1, 1.0, 1)
    # weights 3/4 and 1/4 on values 1 and 0
    assert o[0, 0] == pytest.approx(0.75, abs=1e-15)
    assert lse[0] == pytest.approx(math.log(4.0), abs=1e-15)


def test_equal_scores_and_zero_scale_average_the_values():
    rng = np.random.default_rng(1)
    kv = _pool(rng, 2, 8)
    q = rng.normal(size=(3, 8))
    top = [3, 17, 64 + 5, 100]
    o, lse = O.sparse_attention(q, kv, [0, 1], top, 127, 0.0, 5)
    rows = np.array([kv[p // 64, p % 64] for p in top])
    assert np.allclose(o, np.tile(rows[:, :5].mean(axis=0), (3, 1)), atol=1e-14)
    assert np.allclose(lse, math.log(4.0), atol=1e-15)


def test_matches_loops_and_ignores_invalid_entries():
    rng = np.random.default_rng(2)
    H, d, dv, P = 3, 7, 4, 5
    kv = _pool(rng, P, d)
    table = rng.permutation(P)
    q = rng.normal(size=(H, d))
    qpos = 4 * 64 + 10
    top = np.array([5, 300, 64 * 2 + 3, -1, qpos + 1, qpos, 0, 64 * 4 + 11])
    o, lse = O.sparse_attention(q, kv, table, top, qpos, 0.3, dv)
    valid = [p for p in top if 0 <= p <= qpos]
    for h in range(H):
        s = [0.3 * sum(q[h, j] * kv[table[p // 64], p % 64, j] for j in range(d)) for p in valid]
        z = sum(math.exp(x) for x in s)
        for c in range(dv):
            want = sum(math.exp(x) * kv[table[p // 64], p % 64, c] for x, p in zip(s, valid)) / z
            assert o[h, c] == pytest.approx(want, rel=1e-12, abs=1e-14)
        assert lse[h] == pytest.approx(math.log(z), rel=1e-13)


def test_order_and_shift_invariance():
    rng = np.random.default_rng(3)
    kv = _pool(rng, 4, 16)
    q = rng.normal(size=(2, 16))
    top = rng.choice(4 * 64, size=40, replace=False)
    o1, l1 = O.sparse_attention(q, kv, np.arange(4), top, 255, 0.25, 8)
    o2, l2 = O.sparse_attention(q, kv, np.arange(4), rng.permutation(top), 255, 0.25, 8)
    assert np.allclose(o1, o2, atol=1e-14) and np.allclose(l1, l2, atol=1e-13)
    # setting one key component to 2 everywhere (where q's component is 1)
    # adds 0.25 * 1 * 2 to every score: the output is unchanged, lse moves by 0.5
    q2 = q.copy()
    q2[:, 15] = 1.0
    kv2, kv3 = kv.copy(), kv.copy()
    kv2[:, :, 15] = 2.0
    kv3[:, :, 15] = 0.0
    ob, lb = O.sparse_attention(q2, kv2, np.arange(4), top, 255, 0.25, 8)
    oc, lc = O.sparse_attention(q2, kv3, np.arange(4), top, 255, 0.25, 8)
    assert np.allclose(ob, oc, atol=1e-13) and np.allclose(lb, lc + 0.5, atol=1e-13)


def test_empty_row():
    o, lse = O.sparse_attention(np.ones((2, 4)), np.ones((1, 64, 4)), [0], [-1, 70, -1], 63,
                                1.0, 3)
    assert np.all(o == 0.0) and np.all(lse == NEG)
