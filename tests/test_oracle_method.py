"""Pins of the oracle's method steps: brute force on tiny inputs, closed forms,
invariants and special cases that reduce to textbook routines.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import spin_oracle as O

NEG = float("-inf")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_state(rng, n, ninf=0.2, ties=True):
    x = np.abs(rng.standard_normal(n)) * 10
    if ties:
        idx = rng.integers(0, n, max(1, n // 10))
        x[idx] = x[idx[0]]
    x[rng.random(n) < ninf] = NEG
    return x


# --------------------------------------------------------------- a2: z, max-pool
@pytest.mark.parametrize("qpos", [0, 1, 63, 64, 65, 127, 200, 511])
def test_block_scores_brute_force(qpos):
    rng = np.random.default_rng(qpos)
    V, D = _rand_state(rng, 600), _rand_state(rng, 600)
    S = O.block_scores(V, D, qpos)
    n = (qpos + 64) // 64
    assert len(S) == n
    for j in range(n):
        best = NEG
        for i in range(64 * j, 64 * j + 64):
            if i > qpos:
                continue
            zi = V[i] if V[i] > D[qpos - i] else D[qpos - i]
            if zi > best:
                best = zi
        assert S[j] == best


# ------------------------------------------------------------------ a3: budget
def test_budget_closed_form_exhaustive_small():
    for n in range(1, 400):
        for keep in range(0, 10001, 37):
            for gam in (0, 500, 1000, 2500):
                kb, ne, p = O.budget(keep, n, gam)
                assert kb == math.ceil(Fraction(keep, 10000) * n)
                assert ne == math.floor(Fraction(gam, 10000) * kb)
                assert p == kb - ne


def test_budget_counts_large_vectorised():
    n = np.arange(1, 9001, dtype=np.int64)[:, None]
    keep = np.arange(0, 10001, dtype=np.int64)[None, :]
    kb = (keep * n + 9999) // 10000
    # exact ceil: kb is the least integer with kb * 10000 >= keep * n
    assert np.all(kb * 10000 >= keep * n)
    assert np.all((kb - 1) * 10000 < keep * n)
    # spot-check against the oracle's function
    for (ni, ki) in [(150, 8200), (8192, 5000), (8192, 6000), (4096, 5000), (152, 6000)]:
        assert O.budget(ki, ni, 0)[0] == kb[ni - 1, ki]
    assert O.budget(5000, 8192, 500) == (4096, 204, 3892)
    assert O.budget(6000, 8192, 500) == (4916, 245, 4671)
    assert O.budget(6000, 64, 500) == (39, 1, 38)


# -------------------------------------------------------- a4/a5: select, explore
def _rank_select(S, P):
    """Block j is predicted iff fewer than P blocks beat it (greater, or equal and lower j)."""
    n = len(S)
    out = np.zeros(n, dtype=bool)
    for j in range(n):
        beat = sum(1 for k in range(n) if S[k] > S[j] or (S[k] == S[j] and k < j))
        out[j] = beat < P
    return out


@pytest.mark.parametrize("seed", range(5))
def test_selection_and_exploration_brute_force(seed):
    rng = np.random.default_rng(seed)
    qpos = int(rng.integers(300, 1300))
    V, D = _rand_state(rng, 1400), _rand_state(rng, 1400)
    keep, gam = int(rng.integers(1000, 9000)), int(rng.choice([0, 500, 1000, 2000]))
    sd, layer, step, rid = 77, 2, 5, 1000 + seed
    n = (qpos + 64) // 64
    kb, ne, p = O.budget(keep, n, gam)
    keys = O.explore_keys(n, sd, layer, step, rid)
    pred, expl = O.predict_row(V, D, qpos, keep, gam, keys, False)
    S = O.block_scores(V, D, qpos)
    if kb >= n:
        assert pred.all()
        return
    assert np.array_equal(pred, _rank_select(S, p))
    assert expl.sum() == ne and not (pred & expl).any()
    # explored = the ne non-predicted blocks with the smallest Philox words
    cand = [j for j in range(n) if not pred[j]]
    beat = {j: sum(1 for k in cand if keys[k] < keys[j] or (keys[k] == keys[j] and k < j)) for j in cand}
    assert sorted(j for j in cand if beat[j] < ne) == list(np.nonzero(expl)[0])
    assert (pred | expl).sum() == kb


def test_exploration_zero_share_and_all_keep_cases():
    rng = np.random.default_rng(3)
    V, D = _rand_state(rng, 2000), _rand_state(rng, 2000)
    kept, flags = O.predict_blocks(V, D, 1500, 1, 6000, 0, 1, 0, 4, 9)
    kb, ne, p = O.budget(6000, 24, 0)
    assert len(kept) == kb and ne == 0 and np.all(flags[kept] == 1)
    # s = 0, warm-up, and K_b >= N are all-keep
    for args in [(10000, 500, 4), (6000, 500, 0)]:
        kept, flags = O.predict_blocks(V, D, 1500, 1, args[0], args[1], 1, 0, args[2], 9)
        assert np.array_equal(kept, np.arange(24)) and np.all(flags == 1)
    kept, _ = O.predict_blocks(V, D, 10, 1, 100, 500, 1, 0, 4, 9)   # N = 1, K_b = 1
    assert np.array_equal(kept, [0])


def test_exploration_is_uniform_over_seeds():
    """Each eligible block is drawn with probability n_exp / |eligible| (chi-square)."""
    n, ne = 40, 3
    pred = np.zeros(n, dtype=bool)
    pred[::3] = True                                   # 14 predicted, 26 eligible
    elig = np.nonzero(~pred)[0]
    counts = np.zeros(n)
    trials = 4000
    for s in range(trials):
        keys = O.explore_keys(n, s, 0, 0, 0)
        counts[O.explored_blocks(pred, ne, keys)] += 1
    assert counts[pred].sum() == 0
    exp = trials * ne / len(elig)
    chi2 = ((counts[elig] - exp) ** 2 / exp).sum()
    assert chi2 < 60.0                                 # dof 25: p ~ 1e-4


def test_mtp_union_contains_each_row_and_r1_is_single_row():
    rng = np.random.default_rng(11)
    V, D = _rand_state(rng, 3000), _rand_state(rng, 3000)
    qpos, R, keep, gam = 1023 - 1, 4, 5000, 1000                # rows cross a block edge
    kept, flags = O.predict_blocks(V, D, qpos, R, keep, gam, 5, 1, 3, 77)
    n_last = (qpos + R - 1 + 64) // 64
    keys = O.explore_keys(n_last, 5, 1, 3, 77)
    union = np.zeros(n_last, dtype=bool)
    for r in range(R):
        pr, ex = O.predict_row(V, D, qpos + r, keep, gam, keys, False)
        m = pr | ex
        assert set(np.nonzero(m)[0]) <= set(kept.tolist())
        kb, _, _ = O.budget(keep, (qpos + r + 64) // 64, gam)
        assert m.sum() == kb
        union[: len(m)] |= m
    assert np.array_equal(np.nonzero(union)[0], kept)
    k1, f1 = O.predict_blocks(V, D, qpos, 1, keep, gam, 5, 1, 3, 77)
    pr, ex = O.predict_row(V, D, qpos, keep, gam, keys[: (qpos + 64) // 64], False)
    assert np.array_equal(k1, np.nonzero(pr | ex)[0])
    assert np.array_equal(f1[pr], np.ones(pr.sum())) and np.all(f1[ex] == 2)


# ------------------------------------------------------------------ a7: indexer
def test_indexer_matches_einsum_and_single_head_special_case():
    rng = np.random.default_rng(5)
    R, H, d, pages = 2, 8, 16, 12
    qv = rng.standard_normal((R, H, d))
    wv = rng.uniform(0.5, 1.5, (R, H))
    kv = rng.standard_normal((pages, 64, d))
    sc = rng.uniform(0.1, 2.0, pages)
    table = rng.permutation(pages)
    kept = np.array([0, 2, 3, 7, 9])
    qpos = 9 * 64 + 20
    out = O.indexer_scores(qv, wv, kv, sc, table, kept, qpos)
    for r in range(R):
        for k, j in enumerate(kept):
            p = table[j]
            ref = sc[p] * np.einsum("h,ht->t", wv[r], np.maximum(np.einsum("hd,td->ht", qv[r], kv[p]), 0))
            slot = 64 * j + np.arange(64)
            ref = np.where(slot <= qpos + r, ref, NEG)
            assert np.allclose(out[r, k * 64:(k + 1) * 64], ref, rtol=1e-12, atol=0)
    # one head, w = 1, scale 1: plain ReLU(q . k)
    out1 = O.indexer_scores(qv[:1, :1], np.ones((1, 1)), kv, np.ones(pages), np.arange(pages), [4], 10 ** 6)
    assert np.allclose(out1[0], np.maximum(kv[4] @ qv[0, 0], 0), rtol=1e-12)


# -------------------------------------------------------------------- a8: top-k
def test_topk_rank_definition_with_ties_and_padding():
    rng = np.random.default_rng(8)
    kept = np.array([1, 4, 5, 9])
    scores = np.round(rng.random(256) * 8) / 8              # many ties
    qpos = 9 * 64 + 30
    for k in (1, 10, 100, 230, 300):
        got = O.topk_positions(scores, kept, qpos, k)
        slot = (kept[:, None] * 64 + np.arange(64)).reshape(-1)
        valid = slot <= qpos
        sv, ss = slot[valid], scores[valid]
        chosen = []
        for a in range(len(sv)):
            beat = sum(1 for b in range(len(sv)) if ss[b] > ss[a] or (ss[b] == ss[a] and sv[b] < sv[a]))
            if beat < k:
                chosen.append(sv[a])
        exp = np.full(k, -1)
        exp[: len(chosen)] = sorted(chosen)
        assert np.array_equal(got, exp)


def test_zero_sparsity_selection_equals_full_indexer_topk():
    """At s = 0 the pipeline's top-k equals the top-k of the indexer over all slots."""
    rng = np.random.default_rng(21)
    H, d, qpos, K = 4, 8, 64 * 9 + 17, 50
    nb = (qpos + 64) // 64
    kv = rng.standard_normal((nb, 64, d))
    qv, wv = rng.standard_normal((1, H, d)), rng.uniform(0.5, 1.5, (1, H))
    st = O.RequestState(1024, request_id=3)
    st.step = 5                                             # past warm-up
    st.V[: qpos] = _rand_state(rng, qpos, ninf=0)
    out = O.decode_round(st, qpos, 1, 10000, 500, 1, 0, qv, wv, kv, np.ones(nb),
                         np.arange(nb), K, 0.9)
    full = []
    for i in range(qpos + 1):
        s = sum(wv[0, h] * max(0.0, float(qv[0, h] @ kv[i // 64, i % 64])) for h in range(H))
        full.append((-s, i))
    assert np.array_equal(out["topk"][0], sorted(i for _, i in sorted(full)[:K]))


# ---------------------------------------------------------------- a9/a10: EMA
def test_ema_closed_form_and_special_cases():
    rng = np.random.default_rng(2)
    alpha = 0.9
    a, b = O.ema_weights(alpha)
    obs = rng.standard_normal(12) * 5
    x = np.array([NEG])
    for s in obs:
        x = O.ema_observe(x, s, a, b)
    n = len(obs)
    closed = a ** (n - 1) * obs[0] + b * sum(a ** (n - k) * obs[k - 1] for k in range(2, n + 1))
    assert math.isclose(x[0], closed, rel_tol=1e-12)
    # constant observations are a fixed point; alpha = 0 keeps the last one (prev-iter)
    c = np.array([3.25])
    assert O.ema_observe(c, 3.25, a, b)[0] == pytest.approx(3.25, rel=1e-12)
    a0, b0 = O.ema_weights(0.0)
    y = np.array([NEG])
    for s in obs:
        y = O.ema_observe(y, s, a0, b0)
    assert y[0] == obs[-1]


def test_update_touches_only_observed_slots_and_offsets():
    rng = np.random.default_rng(4)
    V, D = _rand_state(rng, 2048), _rand_state(rng, 2048)
    V0, D0 = V.copy(), D.copy()
    kept = np.array([0, 3, 7, 12])
    qpos = 12 * 64 + 40
    scores = rng.random((1, len(kept) * 64))
    O.ema_update(V, D, scores, kept, qpos, 0, 0.9)
    slot = (kept[:, None] * 64 + np.arange(64)).reshape(-1)
    seen = slot[slot <= qpos]
    unseen_v = np.setdiff1d(np.arange(2048), seen)
    unseen_d = np.setdiff1d(np.arange(2048), qpos - seen)
    assert np.array_equal(V[unseen_v], V0[unseen_v]) and np.array_equal(D[unseen_d], D0[unseen_d])
    a, b = O.ema_weights(0.9)
    k = 3 * 64 + 5                                          # slot 3*64+5 is in kept block 3
    i = 3 * 64 + 5
    exp = scores[0, 64 + 5] if V0[i] == NEG else a * V0[i] + b * scores[0, 64 + 5]
    assert V[i] == exp
    assert k == i


def test_replay_reductions():
    rng = np.random.default_rng(6)
    kept = np.array([2, 3, 5, 6])
    qpos, R = 6 * 64 + 61, 4                                # rows cross into block 7? no: stay in 6
    scores = rng.random((R, len(kept) * 64))
    base_V, base_D = _rand_state(rng, 1024), _rand_state(rng, 1024)
    # a = 0 equals a row-0 single-row update
    V1, D1 = base_V.copy(), base_D.copy()
    O.ema_update(V1, D1, scores, kept, qpos, 0, 0.9)
    V2, D2 = base_V.copy(), base_D.copy()
    O.ema_update(V2, D2, scores[:1], kept, qpos, 0, 0.9)
    assert np.array_equal(V1, V2) and np.array_equal(D1, D2)
    # a = R-1 equals R single-row updates at positions qpos, qpos+1, ...
    V3, D3 = base_V.copy(), base_D.copy()
    O.ema_update(V3, D3, scores, kept, qpos, R - 1, 0.9)
    V4, D4 = base_V.copy(), base_D.copy()
    for r in range(R):
        O.ema_update(V4, D4, scores[r:r + 1], kept, qpos + r, 0, 0.9)
    assert np.array_equal(V3, V4) and np.array_equal(D3, D4)
    # offsets beyond qpos are reached only by later rows (slot 128 at row 3: offset qpos+3-128)
    assert D3[qpos + 3 - 128] != base_D[qpos + 3 - 128] or base_D[qpos + 3 - 128] == NEG


# ------------------------------------------------------------- a11: miss, budgets
def test_miss_zero_at_zero_sparsity_and_random_mask_expectation():
    rng = np.random.default_rng(9)
    nb, K = 200, 400
    scores = rng.random(nb * 64)
    full = O.topk_positions(scores, np.arange(nb), nb * 64 - 1, K)
    assert O.miss_rate(full, np.ones(nb, dtype=np.uint8)) == 0.0
    kb = 80
    ms = []
    for _ in range(300):
        flags = np.zeros(nb, dtype=np.uint8)
        flags[rng.choice(nb, kb, replace=False)] = 1
        ms.append(O.miss_rate(full, flags))
    assert abs((1 - np.mean(ms)) - kb / nb) < 0.01           # recall of a random block mask ~ K_b/N


def test_random_baseline_recall_matches_table1():
    """A random top-K predictor has recall ~K/N; the page prints 0.203 and 0.022 (K = 2048)."""
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "table1_random_baseline.txt"))
            if ln.strip() and not ln.startswith("#")]
    rng = np.random.default_rng(10)
    K = 2048
    for name, n, pearson, recall in rows:
        n = int(n)
        scores = rng.random(n)
        true = set(np.argsort(-scores, kind="stable")[:K].tolist())
        rec = np.mean([len(true & set(rng.choice(n, K, replace=False).tolist())) / K for _ in range(20)])
        assert abs(rec - K / n) < 0.01
        assert abs(K / n - float(recall)) / float(recall) < 0.05


def test_table6_gains_are_ratios_of_printed_values():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "table6_serving.txt"))
            if ln.strip() and not ln.startswith("#")]
    base_tps, base_itl = float(rows[0][1]), float(rows[0][3])
    for r in rows[1:]:
        assert round(100 * (float(r[1]) / base_tps - 1), 1) == float(r[2])
        assert round(100 * (1 - float(r[3]) / base_itl), 1) == float(r[4])


def test_allocate_budgets_invariants():
    for L, mean in [(4, 5000), (6, 6000), (3, 7000)]:
        rng = np.random.default_rng(L)
        m = rng.random(L) * 0.3
        out = O.allocate_budgets(m, mean)
        assert out.sum() == L * mean
        assert np.all(out >= mean // 2) and np.all(out <= 10000)
        order = np.argsort(m)
        assert np.all(np.diff(out[order]) >= -1)            # monotone in miss (up to rounding)
    assert np.array_equal(O.allocate_budgets([0.1] * 4, 5000), [5000] * 4)
    out = O.allocate_budgets([0.0, 0.0, 0.0, 1.0], 5000)       # clamps: one layer saturates
    assert out[3] == 10000 and out[:3].sum() == 10000 and np.all(out[:3] >= 2500)


def _largest_remainder(exact):
    """Integer basis points from exact Fractions: floors, then +1 to the
    largest remainders (ties to the lower layer) until the total is whole."""
    base = [int(math.floor(x)) for x in exact]
    rem = int(sum(exact)) - sum(base)
    order = sorted(range(len(exact)), key=lambda l: (-(exact[l] - base[l]), l))
    for l in order[:rem]:
        base[l] += 1
    return base


@pytest.mark.parametrize("L,mean,seed", [(2, 5000, 1), (4, 6000, 2), (7, 5500, 3), (12, 7000, 4)])
def test_allocate_budgets_unclamped_closed_form(L, mean, seed):
    """Without clamping the rule is keep_l = L * mean * w_l / sum(w), w_l = m_l + 1e-3:
    computed exactly in rationals, then rounded by largest remainder."""
    rng = np.random.default_rng(seed)
    m = 0.05 + rng.random(L) * 0.05                  # near-equal: no layer reaches a clamp
    w = [Fraction(float(x)) + Fraction(1, 1000) for x in m]
    exact = [Fraction(L * mean) * wl / sum(w) for wl in w]
    assert all(Fraction(mean, 2) < x < 10000 for x in exact)
    assert list(O.allocate_budgets(m, mean)) == _largest_remainder(exact)


def test_allocate_budgets_clamped_closed_forms():
    # the cap binds: the high-miss layer takes 10000, the other the rest of 2 * mean
    assert list(O.allocate_budgets([0.0, 0.9], 7000)) == [4000, 10000]
    # the floor binds: the low-miss layer keeps mean / 2, the other the rest
    assert list(O.allocate_budgets([0.0, 0.9], 6000)) == [3000, 9000]
    # three layers, one capped: the other two share 3 * mean - 10000 in proportion
    m = [0.10, 0.12, 0.95]
    out = O.allocate_budgets(m, 6500)
    w = [Fraction(0.10) + Fraction(1, 1000), Fraction(0.12) + Fraction(1, 1000)]
    rest = Fraction(3 * 6500 - 10000)
    assert out[2] == 10000
    assert list(out[:2]) == _largest_remainder([rest * w[0] / sum(w), rest * w[1] / sum(w)])


def _convex_curve(rng, G):
    """A non-increasing curve, convex in the grid index, with distinct steps."""
    drops = np.sort(rng.random(G - 1))[::-1] * rng.uniform(0.05, 0.3)
    return np.concatenate([[drops.sum()], drops.sum() - np.cumsum(drops)])


@pytest.mark.parametrize("L,G,seed", [(2, 3, 1), (2, 5, 2), (3, 4, 3), (3, 5, 4), (4, 4, 5)])
def test_allocate_budgets_curve_is_least_summed_miss_on_convex_curves(L, G, seed):
    """Brute force over every grid assignment within the total: on curves convex
    in the keep (equal grid steps) marginal allocation reaches the least sum."""
    import itertools
    rng = np.random.default_rng(seed)
    grid = [2500 + 1250 * i for i in range(G)]
    for trial in range(30):
        curve = np.stack([_convex_curve(rng, G) for _ in range(L)])
        mean = grid[int(rng.integers(0, G))]
        out = O.allocate_budgets_curve(curve, grid, mean)
        best = min(sum(curve[l, c[l]] for l in range(L))
                   for c in itertools.product(range(G), repeat=L)
                   if sum(grid[i] for i in c) <= L * mean)
        got = sum(curve[l, grid.index(int(out[l]))] for l in range(L))
        assert got == pytest.approx(best, abs=1e-12)
        assert out.sum() == L * mean                     # equal steps: the total is spent


def test_allocate_budgets_curve_closed_forms():
    grid = [2500, 5000, 7500, 10000]
    # identical curves: every layer stays at the mean
    flat = [[0.4, 0.2, 0.1, 0.0]] * 3
    assert list(O.allocate_budgets_curve(flat, grid, 5000)) == [5000] * 3
    # a layer whose miss does not move gives its steps to one that falls steeply
    curve = [[0.05, 0.05, 0.05, 0.05], [0.6, 0.3, 0.1, 0.0]]
    assert list(O.allocate_budgets_curve(curve, grid, 5000)) == [2500, 7500]
    assert list(O.allocate_budgets_curve(curve, grid, 6250)) == [2500, 10000]
    # equal gains go to the lower layer first
    tie = [[0.5, 0.25, 0.0, 0.0], [0.5, 0.25, 0.0, 0.0]]
    assert list(O.allocate_budgets_curve(tie, grid, 6250)) == [7500, 5000]
    # uneven grid: the gain is per basis point of the step
    g2 = [4000, 5000, 8000]
    c2 = [[0.30, 0.20, 0.10], [0.30, 0.26, 0.00]]      # 1e-4/bp, then 3.3e-5/bp; 4e-5/bp, then 8.7e-5/bp
    assert list(O.allocate_budgets_curve(c2, g2, 5000)) == [5000, 5000]
    assert list(O.allocate_budgets_curve(c2, g2, 6500)) == [5000, 8000]
    # the mean at the lowest grid point: nothing to hand out
    assert list(O.allocate_budgets_curve(curve, grid, 2500)) == [2500, 2500]


def test_allocate_budgets_curve_invariants():
    rng = np.random.default_rng(11)
    grid = [2000, 3000, 4500, 5000, 7000, 10000]
    for trial in range(200):
        L = int(rng.integers(1, 9))
        curve = rng.random((L, len(grid)))              # not monotone, not convex
        mean = int(rng.integers(2000, 10001))
        out = O.allocate_budgets_curve(curve, grid, mean)
        assert all(int(k) in grid for k in out)
        assert out.sum() <= L * mean
        room = L * mean - out.sum()
        for l in range(L):                              # no further step fits
            i = grid.index(int(out[l]))
            assert i + 1 == len(grid) or grid[i + 1] - grid[i] > room
