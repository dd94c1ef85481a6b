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
