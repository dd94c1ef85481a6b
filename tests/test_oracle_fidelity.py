"""Pins of the oracle's selection-fidelity functions: the online miss
estimate (exploration hits scaled by skipped / explored blocks), Pearson
correlation and top-k recall of slot predictors (v1 Table 1).

The miss estimate is checked by brute force over every exploration draw of
tiny cases (its mean over all equally likely draws must equal the true miss
exactly); Pearson and recall against hand-computed values, closed forms and
exhaustive averages over all predictor rankings."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import spin_oracle as O

NEG = float("-inf")


def _case(n_blocks, k, seed):
    """True slot scores over n_blocks full blocks and their all-keep top-k."""
    rng = np.random.default_rng(seed)
    q = 64 * n_blocks - 1
    scores = rng.permutation(q + 1).astype(np.float64)          # distinct
    full = O.topk_positions(scores, np.arange(n_blocks), q, k)
    return q, scores, full


@pytest.mark.parametrize("n_blocks,pred,n_exp,k,seed", [
    (6, [0, 3], 2, 40, 1), (7, [1], 3, 100, 2), (8, [0, 2, 5], 1, 64, 3), (5, [], 2, 200, 4)])
def test_estimate_is_unbiased_over_all_draws(n_blocks, pred, n_exp, k, seed):
    q, scores, full = _case(n_blocks, k, seed)
    U = [j for j in range(n_blocks) if j not in pred]
    total = Fraction(0)
    draws = 0
    for E in itertools.combinations(U, n_exp):
        flags = np.zeros(n_blocks, dtype=np.uint8)
        flags[pred] = 1
        flags[list(E)] = 2
        true_miss = O.miss_rate(full, flags)
        # with h counted on the all-keep top-k itself the estimate is the
        # plain ratio estimator; no clamp is reached in these cases
        est = O.estimate_miss(full, flags, q, k)
        assert 0.0 <= est < 1.0
        total += Fraction(est)
        draws += 1
        # the sparse round's own top-k can only count more hits
        kept = np.nonzero(flags)[0]
        row = scores[(kept[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)]
        sparse = O.topk_positions(row, kept, q, k)
        assert O.estimate_miss(sparse, flags, q, k) >= est
    flags = np.zeros(n_blocks, dtype=np.uint8)
    flags[pred] = 1
    true_u = float(np.isin(full // 64, U).sum()) / k            # miss with E empty
    # E[h] = (n_exp / |U|) * (top-k slots in U); E[est] = E[h] (|U| - n_exp) / (n_exp k)
    want = true_u * (len(U) - n_exp) / len(U)
    assert math.isclose(float(total / draws), want, rel_tol=1e-6, abs_tol=1e-7)
    # and that is the mean true miss over the draws as well
    mean_true = np.mean([O.miss_rate(full, np.where(np.isin(np.arange(n_blocks), E), 2,
                                                    np.where(np.isin(np.arange(n_blocks), pred),
                                                             1, 0)))
                         for E in itertools.combinations(U, n_exp)])
    assert math.isclose(float(total / draws), mean_true, rel_tol=1e-6, abs_tol=1e-7)


def test_estimate_special_cases():
    q, scores, full = _case(4, 64, 9)
    all_kept = np.array([1, 2, 1, 1], dtype=np.uint8)
    assert O.estimate_miss(full, all_kept, q, 64) == 0.0          # nothing skipped
    no_expl = np.array([1, 0, 1, 0], dtype=np.uint8)
    assert O.estimate_miss(full, no_expl, q, 64) == -1.0          # no estimate
    # one explored block holding the whole top-k, three skipped: clamps to 1
    flags = np.array([2, 0, 0, 0], dtype=np.uint8)
    top = np.arange(64)
    assert O.estimate_miss(top, flags, q, 64) == 1.0
    # h = 16 of k = 64 in the one explored block, 2 skipped: 16 * 2 / (1 * 64)
    flags = np.array([1, 2, 0, 0], dtype=np.uint8)
    top = np.concatenate([np.arange(48), 64 + np.arange(16)])
    assert O.estimate_miss(top, flags, q, 64) == 0.5
    # positions past the row's query and -1 padding are not hits; k_r = q + 1
    q2 = 64 + 9
    flags = np.array([1, 2], dtype=np.uint8)
    assert O.estimate_miss(np.array([64, 65, 200, -1]), flags, q2, 4096) == 0.0


def test_pearson_values():
    assert O.pearson([1, 2, 3], [1, 3, 2]) == pytest.approx(0.5, abs=1e-15)
    x = np.array([0.5, -1.0, 2.0, 7.0, 3.0])
    assert O.pearson(x, 3.0 * x - 2.0) == pytest.approx(1.0, abs=1e-15)
    assert O.pearson(x, -0.25 * x + 9.0) == pytest.approx(-1.0, abs=1e-15)
    # hand value: x = (1, 2, 3, 4), y = (2, 1, 4, 3): cov 0.8 / var 1.25 -> 0.6
    assert O.pearson([1, 2, 3, 4], [2, 1, 4, 3]) == pytest.approx(0.6, abs=1e-15)
    # slots without a prediction are left out
    assert O.pearson([NEG, 1, 2, 3, NEG], [5.0, 1, 3, 2, -4.0]) == pytest.approx(0.5, abs=1e-15)
    assert O.pearson([1, 1, 1], [1, 2, 3]) == 0.0
    assert O.pearson([NEG, 2.0], [1.0, 2.0]) == 0.0


@pytest.mark.parametrize("n,k", [(10, 3), (10, 6), (130, 64), (200, 150)])
def test_recall_closed_forms(n, k):
    a = np.arange(n, dtype=np.float64)
    assert O.topk_recall(a, a, k) == 1.0
    assert O.topk_recall(2.0 * a + 1.0, a, k) == 1.0           # any increasing map
    assert O.topk_recall(-a, a, k) == max(0, 2 * k - n) / k     # reversed ranking
    assert O.topk_recall(np.full(n, NEG), a, k) == max(0, 2 * k - n) / k   # ties -> low slots


def test_random_ranking_recall_is_k_over_n():
    # every ranking of the predictor equally likely: mean recall = k / n exactly
    n, k = 6, 2
    actual = np.array([3.0, 9.0, 1.0, 7.0, 5.0, 2.0])
    rec = [O.topk_recall(np.array(p, dtype=np.float64), actual, k)
           for p in itertools.permutations(range(n))]
    assert Fraction(sum(Fraction(r).limit_denominator(100) for r in rec), len(rec)) == Fraction(k, n)
