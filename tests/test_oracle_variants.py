"""Pins of the oracle's predictor variants: Mean and Top-4 block pooling, and the
row-0 mask policy (v1, Figure 3 caption and Table 7 / Figure 2).

The pooling definitions are checked against plain loops over slots on tiny
inputs with never-observed entries and ragged last blocks, and against the
invariants that hold between the poolings; the row-0 policy against its
construction from a single row's mask."""
import math

import numpy as np
import pytest

from oracle import spin_oracle as O

NEG = float("-inf")


def _state(rng, n, unobserved=0.2):
    V = rng.normal(size=n) * 3.0
    D = rng.normal(size=n) * 3.0
    V[rng.random(n) < unobserved] = NEG
    D[rng.random(n) < unobserved] = NEG
    return V, D


def _pool_by_loops(V, D, q, how):
    """Block scores by definition: loop over blocks, then over their slots."""
    n = (q + 64) // 64
    out = []
    for j in range(n):
        vals = []
        for i in range(64 * j, min(64 * j + 64, q + 1)):
            z = max(V[i], D[q - i])                    # max(-inf, x) = x
            if z != NEG:
                vals.append(float(z))
        if not vals:
            out.append(NEG)
        elif how == "max":
            out.append(max(vals))
        elif how == "mean":
            out.append(math.fsum(vals) / len(vals))
        else:
            top = sorted(vals, reverse=True)[:4]
            out.append(math.fsum(top) / len(top))
    return np.array(out)


@pytest.mark.parametrize("how", ["max", "mean", "top4"])
@pytest.mark.parametrize("q", [0, 3, 63, 64, 200, 511, 700])
def test_pooling_matches_loops(how, q):
    rng = np.random.default_rng(q * 7 + len(how))
    V, D = _state(rng, 800)
    got = O.block_scores(V, D, q, how)
    ref = _pool_by_loops(V, D, q, how)
    assert got.shape == ref.shape
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got))
    assert np.allclose(got[fin], ref[fin], rtol=1e-13, atol=0)


def test_pooling_invariants():
    rng = np.random.default_rng(5)
    for q in (100, 333, 640, 1000):
        V, D = _state(rng, 1100, unobserved=0.5)
        mx = O.block_scores(V, D, q, O.POOL_MAX)
        mean = O.block_scores(V, D, q, O.POOL_MEAN)
        top4 = O.block_scores(V, D, q, O.POOL_TOP4)
        fin = np.isfinite(mx)
        assert np.array_equal(fin, np.isfinite(mean)) and np.array_equal(fin, np.isfinite(top4))
        assert np.all(mean[fin] <= top4[fin] + 1e-12)
        assert np.all(top4[fin] <= mx[fin] + 1e-12)


def test_pooling_special_cases():
    q = 127
    V = np.full(200, NEG)
    D = np.full(200, NEG)
    V[70] = 2.5                                        # one finite slot in block 1
    for how in ("max", "mean", "top4"):
        S = O.block_scores(V, D, q, how)
        assert S[0] == NEG and S[1] == 2.5
    V[64:68] = [1.0, 2.0, 3.0, 4.0]                    # block 1: 5 finite values
    S = O.block_scores(V, D, q, "top4")
    assert S[1] == (4.0 + 3.0 + 2.5 + 2.0) / 4
    S = O.block_scores(V, D, q, "mean")
    assert S[1] == (1.0 + 2.0 + 3.0 + 4.0 + 2.5) / 5
    # at most 4 finite values: top-4 is the plain mean
    V[64] = NEG
    assert O.block_scores(V, D, q, "top4")[1] == O.block_scores(V, D, q, "mean")[1]
    # every slot equal: all poolings agree
    V[:] = 1.5
    D[:] = 1.5
    for how in ("max", "mean", "top4"):
        assert np.all(O.block_scores(V, D, q, how) == 1.5)


@pytest.mark.parametrize("rows", [1, 2, 4])
def test_row0_mask_policy(rows):
    rng = np.random.default_rng(rows)
    V, D = _state(rng, 3000, unobserved=0.0)
    q = 64 * 30 - 2                                    # later rows cross into a new block
    args = dict(qpos=q, rows=rows, keep_bp=5000, explore_bp=1000, seed=11, layer=1, step=4,
                request_id=7)
    kept0, flags0 = O.predict_blocks(V, D, mask=O.MASK_ROW0, **args)
    n0 = O.num_blocks(q)
    n_last = O.num_blocks(q + rows - 1)
    keys = O.explore_keys(n_last, 11, 1, 4, 7)
    pred, expl = O.predict_row(V, D, q, 5000, 1000, keys, False)
    want = np.zeros(n_last, dtype=np.uint8)
    want[:n0][pred] = 1
    want[:n0][expl & ~pred] = 2
    want[n0:] = 1                                      # draft blocks past row 0's last block
    assert np.array_equal(flags0, want)
    assert np.array_equal(kept0, np.nonzero(want)[0])
    kept_u, flags_u = O.predict_blocks(V, D, **args)
    if rows == 1:
        assert np.array_equal(kept0, kept_u) and np.array_equal(flags0, flags_u)
    else:
        # row 0's own mask is part of both
        assert set(np.nonzero(want[:n0])[0]) <= set(kept_u.tolist())
