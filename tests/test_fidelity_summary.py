"""Host-side aggregation of the selection-fidelity runs (mean / p99 miss over
eligible rows, v1 Table 5 caption; realized block sparsity), on hand-built
miss arrays whose answers are known in closed form."""
import numpy as np

import bench


def _case(T=101, L=2, B=3, R=2, keep=5000, q0=64 * 100):
    miss = np.zeros((T, L, B, R), dtype=np.float32)
    kept = np.full((T, L, B), 50, dtype=np.int64)
    keeps = np.full((T, L), keep, dtype=np.int64)
    qpos = np.full((T, B), q0, dtype=np.int64)
    return miss, kept, keeps, qpos


def test_warmup_rounds_are_not_eligible():
    miss, kept, keeps, qpos = _case()
    miss[0] = 1.0                                  # warm-up round: everything missed
    s = bench._fidelity_summary(miss, kept, keeps, qpos, 2, warmup=1)
    assert s["eligible_rows"] == 100 * 2 * 3 * 2
    assert s["mean_miss"] == 0.0 and s["p99_miss"] == 0.0 and s["p99_pooled"] == 0.0


def test_p99_is_per_trace_then_averaged():
    miss, kept, keeps, qpos = _case(R=1)
    # trace (layer 0, request 0): one row of 100 eligible rows has miss 1
    miss[7, 0, 0, 0] = 1.0
    s = bench._fidelity_summary(miss, kept, keeps, qpos, 1, warmup=1)
    # the linear p99 of 99 zeros and a one sits at 0.99 * 99 = 98.01: 0.01
    assert np.isclose(s["per_layer"][0]["p99_miss"], 0.01 / 3)
    assert np.isclose(s["p99_miss"], 0.01 / 6)      # 6 traces, one of them at 0.01
    assert np.isclose(s["mean_miss"], 1.0 / 600)
    # pooled over 600 rows, one of them 1: position 0.99 * 599 = 593.01 -> 0
    assert s["p99_pooled"] == 0.0
    assert s["per_layer"][1]["mean_miss"] == 0.0


def test_rows_without_sparsity_are_not_eligible():
    miss, kept, keeps, qpos = _case()
    keeps[:, 1] = 10000                            # layer 1 keeps everything
    miss[:, 1] = 0.5
    s = bench._fidelity_summary(miss, kept, keeps, qpos, 2, warmup=1)
    assert s["eligible_rows"] == 100 * 1 * 3 * 2
    assert s["per_layer"][1]["mean_miss"] is None
    assert s["mean_miss"] == 0.0


def test_realized_sparsity_counts_blocks_to_the_last_row():
    miss, kept, keeps, qpos = _case(T=5, R=2, q0=64 * 99 + 63)   # row 1 opens block 100
    kept[:] = 40
    kept[0] = 101                                  # warm-up round, not counted
    s = bench._fidelity_summary(miss, kept, keeps, qpos, 2, warmup=1)
    assert np.isclose(s["realized_sparsity"], 1.0 - 40.0 / 101.0)
    s = bench._fidelity_summary(miss, kept, keeps, qpos, 2, warmup=1, first_round=3)
    assert np.isclose(s["realized_sparsity"], 1.0 - 40.0 / 101.0)
    assert s["eligible_rows"] == 2 * 2 * 3 * 2


def test_online_estimates_are_reported_beside_the_miss():
    miss, kept, keeps, qpos = _case(T=11, R=1)
    rng = np.random.default_rng(3)
    miss[:] = rng.random(miss.shape)
    est = np.stack([miss, np.minimum(1.0, 2.0 * miss)], axis=-1)   # estimate exact, bound 2x
    est[5, 0, 0, 0] = -1.0                                         # one row without an estimate
    s = bench._fidelity_summary(miss, kept, keeps, qpos, 1, warmup=1, est=est)
    assert s["online_rows_without_estimate"] == 1
    keep = np.ones(miss[1:].shape, dtype=bool)
    keep[4, 0, 0, 0] = False
    assert np.isclose(s["online_mean_miss"], miss[1:][keep].mean())
    assert np.isclose(s["online_upper_mean_miss"], np.minimum(1.0, 2.0 * miss[1:][keep]).mean())
    assert np.isclose(s["online_row_pearson"], 1.0)
    assert s["online_upper_row_pearson"] < 1.0
    assert np.isclose(s["per_layer"][1]["online_mean_miss"], s["per_layer"][1]["mean_miss"])
