"""Pins of the oracle's selection-fidelity functions: the online miss
estimate (exploration hits scaled by skipped / explored blocks), Pearson
correlation and top-k recall of slot predictors (v1 Table 1).

The hit ratio is checked by brute force over every exploration draw of tiny
cases (its mean over all equally likely draws must equal the true miss); the
weighted-threshold estimate against blocks whose skipped twins repeat the
explored scores (where it must equal the true miss exactly) and hand-walked
cases; Pearson and recall against hand-computed values, closed forms and
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


def _scores_of(scores, top):
    return np.array([scores[p] if p >= 0 else 0.0 for p in top])


@pytest.mark.parametrize("n_blocks,pred,n_exp,k,seed", [
    (6, [0, 3], 2, 40, 1), (7, [1], 3, 100, 2), (8, [0, 2, 5], 1, 64, 3), (5, [], 2, 200, 4)])
def test_hit_ratio_is_unbiased_over_all_draws(n_blocks, pred, n_exp, k, seed):
    """The upper-bound ratio, fed the all-keep top-k itself, is the plain
    ratio estimator: its mean over every equally likely exploration draw is
    the mean true miss.  Fed the sparse round's own top-k it can only grow,
    and the weighted-threshold estimate never exceeds it."""
    q, scores, full = _case(n_blocks, k, seed)
    U = [j for j in range(n_blocks) if j not in pred]
    total = Fraction(0)
    trues = []
    for E in itertools.combinations(U, n_exp):
        flags = np.zeros(n_blocks, dtype=np.uint8)
        flags[pred] = 1
        flags[list(E)] = 2
        trues.append(O.miss_rate(full, flags))
        _, ub = O.estimate_miss(full, _scores_of(scores, full), flags, q, k)
        assert 0.0 <= ub < 1.0                        # no clamp in these cases
        total += Fraction(ub)
        kept = np.nonzero(flags)[0]
        row = scores[(kept[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)]
        sparse = O.topk_positions(row, kept, q, k)
        est, ub_sparse = O.estimate_miss(sparse, _scores_of(scores, sparse), flags, q, k)
        assert ub_sparse >= ub and est <= ub_sparse
        assert 0.0 <= est
    draws = len(trues)
    true_u = float(np.isin(full // 64, U).sum()) / k                # all of U skipped
    assert math.isclose(float(total / draws), true_u * (len(U) - n_exp) / len(U),
                        rel_tol=1e-6, abs_tol=1e-7)
    assert math.isclose(float(total / draws), float(np.mean(trues)), rel_tol=1e-6, abs_tol=1e-7)


@pytest.mark.parametrize("c_e_true", [0, 5, 30, 64])
def test_threshold_estimate_exact_on_mirrored_blocks(c_e_true):
    """Skipped blocks that repeat the explored blocks' scores exactly: the
    explored sample is then a perfect picture of U, the weighted walk stops
    exactly at the all-keep threshold, and the estimate is the true miss."""
    rng = np.random.default_rng(c_e_true)
    # blocks 0..2 predicted, 3..4 explored, 5..6 skipped twins of 3..4
    vals_e = rng.permutation(np.arange(1000, 1128, dtype=np.float64))     # 128 explored slots
    vals_p = rng.permutation(np.arange(0, 192, dtype=np.float64)) * 10.0 - 500.0
    scores = np.concatenate([vals_p, vals_e, vals_e + 0.0])
    q = 7 * 64 - 1
    flags = np.array([1, 1, 1, 2, 2, 0, 0], dtype=np.uint8)
    # k: the all-keep top-k takes the top c_e_true explored values, their twins,
    # and the predicted slots above the next explored value
    e_sorted = np.sort(vals_e)[::-1]
    thr = e_sorted[c_e_true - 1] if c_e_true else 1e9
    nxt = e_sorted[c_e_true] if c_e_true < 128 else -1e9
    n_p = int(((vals_p > nxt) & (vals_p >= min(thr, 1e9))).sum()) if c_e_true else 0
    k = n_p + 2 * c_e_true
    if k == 0:
        k = 1
        n_p = 1
    full = O.topk_positions(scores, np.arange(7), q, k)
    true_miss = O.miss_rate(full, flags)
    kept = np.array([0, 1, 2, 3, 4])
    row = scores[(kept[:, None] * 64 + np.arange(64)[None, :]).reshape(-1)]
    sparse = O.topk_positions(row, kept, q, k)
    est, ub = O.estimate_miss(sparse, _scores_of(scores, sparse), flags, q, k)
    assert est == np.float32(true_miss)
    assert ub >= est


def test_estimate_special_cases():
    q, scores, full = _case(4, 64, 9)
    sc = _scores_of(scores, full)
    all_kept = np.array([1, 2, 1, 1], dtype=np.uint8)
    assert O.estimate_miss(full, sc, all_kept, q, 64) == (0.0, 0.0)      # nothing skipped
    no_expl = np.array([1, 0, 1, 0], dtype=np.uint8)
    assert O.estimate_miss(full, sc, no_expl, q, 64) == (-1.0, -1.0)     # no estimate
    # one explored block holding the whole top-k, three skipped: each explored
    # slot stands for |U| / |E| = 4, so the walk stops after 16 of them:
    # 16 * 3 / 64; the hit ratio 64 * 3 / 64 clamps to 1
    flags = np.array([2, 0, 0, 0], dtype=np.uint8)
    top = np.arange(64)
    assert O.estimate_miss(top, np.arange(64.0), flags, q, 64) == (0.75, 1.0)
    # h = 16 of k = 64 in the one explored block (|U| = 3, |E| = 1), 2 skipped
    flags = np.array([1, 2, 0, 0], dtype=np.uint8)
    top = np.concatenate([np.arange(48), 64 + np.arange(16)])
    # the explored slots score highest: the walk passes c explored slots with
    # weight 3 until 3c >= 64 -> c = 22 > 16, so it takes all 16 and stops
    # inside the predicted ones: estimate = upper = 16 * 2 / (1 * 64)
    sc = np.concatenate([np.zeros(48), 100.0 + np.arange(16)])
    assert O.estimate_miss(top, sc, flags, q, 64) == (0.5, 0.5)
    # the explored slots score lowest: the predicted 48 (weight 1) and then
    # c explored (weight 3): 48 + 3c >= 64 -> c = 6: 6 * 2 / 64
    sc = np.concatenate([100.0 + np.arange(48), np.zeros(16)])
    assert O.estimate_miss(top, sc, flags, q, 64) == (np.float32(12 / 64), 0.5)
    # positions past the row's query and -1 padding are ignored; k_r = q + 1
    q2 = 64 + 9
    flags = np.array([1, 2], dtype=np.uint8)
    assert O.estimate_miss(np.array([64, 65, 200, -1]), np.ones(4), flags, q2, 4096) == (0.0, 0.0)


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
