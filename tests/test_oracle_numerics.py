"""Pins of the oracle's number formats and RNG against library routines.

fp8 e4m3fn decode/encode against torch's float8_e4m3fn, the query exponent
rule by brute force, Philox4x64-10 against numpy.random.Philox.
"""
import math

import numpy as np
import pytest
import torch

from oracle import spin_oracle as O


def test_e4m3fn_decode_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = O.e4m3fn_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(mine))
    assert nan.sum() == 2                                   # 0x7F and 0xFF only
    assert np.array_equal(ref[~nan], mine[~nan])
    # OCP spec points: largest normal, smallest normal, smallest subnormal
    assert mine[0x7E] == 448.0 and mine[0x08] == 2.0 ** -6 and mine[0x01] == 2.0 ** -9


def _torch_e4m3(x):
    t = torch.tensor(np.asarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3fn_encode_grid_and_ties_match_torch():
    pos = O.E4M3FN[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2.0                        # exact ties
    eps = np.concatenate([mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20)])
    x = np.concatenate([pos, mids, eps, [0.0, 2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -11]])
    x = np.concatenate([x, -x])
    x = x[np.abs(x) <= 448.0]
    x32 = x.astype(np.float32).astype(np.float64)           # what torch sees
    assert np.array_equal(O.e4m3fn_encode(x32), _torch_e4m3(x32))


def test_quantize_every_finite_bf16_value_matches_torch():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    vals = bits.view(torch.bfloat16).to(torch.float64).numpy()
    vals = vals[np.isfinite(vals)]
    # each value is its own (row, head) vector of length 1: e from |v|
    codes, e, q8 = O.quantize_q(vals[:, None])
    scaled = vals * np.exp2(-e.astype(np.float64))
    assert np.all(np.abs(scaled) <= 448.0)
    assert np.array_equal(codes[:, 0], _torch_e4m3(scaled))
    # and inside a longer vector the smaller entries use the big entry's exponent
    rng = np.random.default_rng(1)
    v = torch.randn(4096, 128, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    v[rng.integers(0, 4096, 64)] *= 2.0 ** rng.integers(-30, 30, (64, 1))
    codes, e, _ = O.quantize_q(v)
    scaled = v * np.exp2(-e.astype(np.float64))[:, None]
    assert np.array_equal(codes, _torch_e4m3(scaled))


@pytest.mark.parametrize("amax", [1e-30, 2.0 ** -20, 0.3, 1.0, 3.5, 447.9, 448.0, 448.1,
                                  896.0, 1e6, 3.0e38])
def test_q_exponent_is_smallest_by_brute_force(amax):
    e = O.q_exponent(amax)
    assert amax * 2.0 ** -e <= 448.0
    assert amax * 2.0 ** -(e - 1) > 448.0
    # brute force over a wide integer range
    ok = [k for k in range(-400, 400) if amax * 2.0 ** -k <= 448.0]
    assert e == min(ok)
    assert O.q_exponent(0.0) == 0


def _numpy_philox_block(counter, key):
    """philox(counter) via numpy, whose bit generator advances before use."""
    c = (sum(int(v) << (64 * i) for i, v in enumerate(counter)) - 1) % (1 << 256)
    words = np.array([(c >> (64 * i)) & O.MASK64 for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(counter=words, key=np.array(key, dtype=np.uint64))
    return tuple(int(x) for x in bg.random_raw(4))


@pytest.mark.parametrize("seed", range(6))
def test_philox_matches_numpy(seed):
    rng = np.random.default_rng(seed)
    ctr = [int(x) for x in rng.integers(0, 2 ** 63, 4, dtype=np.int64)]
    key = [int(x) for x in rng.integers(0, 2 ** 63, 2, dtype=np.int64)]
    if seed == 0:
        ctr, key = [0, 0, 0, 0], [0, 0]
    assert O.philox4x64_10(ctr, key) == _numpy_philox_block(ctr, key)


def test_explore_keys_word_layout():
    seed, layer, step, rid = 0x5350494E, 3, 17, 12345
    keys = O.explore_keys(10, seed, layer, step, rid)
    for j in range(10):
        blk = _numpy_philox_block((j // 4, step, rid, 0), (seed, layer))
        assert keys[j] == blk[j % 4]


def test_ema_weights_are_fp32_values():
    a, b = O.ema_weights(0.9)
    assert a == float(np.float32(0.9)) and b == float(np.float32(np.float32(1) - np.float32(0.9)))
    assert abs(a + b - 1.0) < 1e-7
    assert math.isclose(b, 0.1, rel_tol=1e-6)


def _plain_scores(qv, wv, keys):
    """sum_h wv[h] * max(0, sum_d qv[h][d] * keys[t][d]) for every token t, in
    plain Python loops (the DSA indexer formula written out)."""
    out = []
    for t in range(len(keys)):
        s = 0.0
        for h in range(len(qv)):
            dot = 0.0
            for d in range(len(keys[t])):
                dot += float(qv[h][d]) * float(keys[t][d])
            s += float(wv[h]) * max(dot, 0.0)
        out.append(s)
    return np.array(out)


def _smallest_exponent(amax):
    """Smallest integer k with amax * 2**-k <= 448, in exact rational arithmetic."""
    from fractions import Fraction
    a = Fraction(amax)
    k = -200
    while a / Fraction(2) ** k > 448:
        k += 1
    assert a / Fraction(2) ** (k - 1) > 448 or a == 0
    return k


def test_fp8_query_operands_exponent_weights_and_scores():
    """fp8_query_operands returns the decoded codes q8 and w' = w * 2**e with e
    the per-(row, head) exponent of the query quantisation: the score of
    (q8, w') must equal that of (q8 * 2**e, w) -- the queries at their own
    scale -- and stay within the e4m3fn rounding bound of the bf16-query
    score.  A sign slip in e (w * 2**-e) would move every score by 2**(2e)."""
    rng = np.random.default_rng(11)
    R, H, d, T = 2, 6, 16, 9
    q = rng.standard_normal((R, H, d))
    # head magnitudes 2**-30 .. 2**30 so no exponent is 0; one head with a
    # single large entry (the others fall into the e4m3fn subnormals)
    q *= np.exp2(rng.integers(-30, 31, (R, H, 1)).astype(np.float64))
    q[1, 2, :] *= 1e-3
    q[1, 2, 5] = 3.0e4
    q = torch.tensor(q, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    w = rng.uniform(-1.5, 1.5, (R, H))
    w = w.astype(np.float32).astype(np.float64)
    keys = rng.standard_normal((T, d))

    q8, wv, codes, e = O.fp8_query_operands(q, w)
    assert q8.shape == q.shape and wv.shape == w.shape and e.shape == w.shape
    for r in range(R):
        for h in range(H):
            k = _smallest_exponent(np.abs(q[r, h]).max())
            assert e[r, h] == k != 0
            assert wv[r, h] / w[r, h] == 2.0 ** k           # exact: w' = w * 2**e
            # the codes are the RNE e4m3fn codes of q * 2**-e, and q8 their values
            assert np.array_equal(codes[r, h], _torch_e4m3(q[r, h] * 2.0 ** -k))
            assert np.array_equal(q8[r, h], O.E4M3FN[codes[r, h]])
            # rounding bound of e4m3fn at scale 2**e: half an ulp of a normal
            # (2**-4 relative) or of the subnormal spacing (2**-10 absolute)
            err = np.abs(q8[r, h] * 2.0 ** k - q[r, h])
            assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(q[r, h]), 2.0 ** (k - 10)))

    for r in range(R):
        scaled_q = q8[r] * np.exp2(e[r].astype(np.float64))[:, None]
        a = _plain_scores(q8[r], wv[r], keys)
        b = _plain_scores(scaled_q, w[r], keys)
        assert np.allclose(a, b, rtol=1e-12, atol=0)
        # against the bf16-query score: ReLU is 1-Lipschitz, so the gap is at
        # most sum_h |w_h| sum_d |q8*2**e - q| |k|
        exact = _plain_scores(q[r], w[r], keys)
        bound = np.array([sum(abs(w[r, h]) * np.dot(np.abs(scaled_q[h] - q[r, h]), np.abs(keys[t]))
                              for h in range(H)) for t in range(T)])
        assert np.all(np.abs(a - exact) <= bound * (1 + 1e-9) + 1e-300)
        # the oracle's indexer formula on these operands gives the same scores
        table = np.arange(1)
        kv = np.zeros((1, 64, d))
        kv[0, :T] = keys
        s = O.indexer_scores(q8[r][None], wv[r][None], kv, np.ones(1), table, [0], 63)
        assert np.allclose(s[0, :T], a, rtol=1e-12, atol=1e-300)
