"""GPU parity of the selection-fidelity calls against the oracle: the slot
predictions z = max(V, D) (bit-exact), the online miss estimate from the
exploration blocks (bit-exact: an integer weighted walk, fp64 ratios rounded
to fp32), and predictor quality (Pearson within 1e-10, top-k recall exact).
Inputs are drawn on the host; every expected value comes from the oracle."""
import numpy as np
import pytest
import torch

import predictive_kv_block_amd as spin
from oracle import spin_oracle as O
from tests.spin_harness import NEG, Rig, nblocks, np_
from workload import random_state

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("R,blocks", [(1, 40), (4, 40), (2, 3000)])
def test_slot_scores_exact(gpu_lib, R, blocks):
    B, ctx = 3, 64 * blocks
    mb = nblocks(ctx - 1)
    cfg = spin.make_config(2, B, ctx, 256, max_rows=R)
    rig = Rig(cfg, B, R, mb)
    rig.reset([5, 6, 7])
    qpos = np.array([ctx - R, 64 * (blocks // 2) + 17, 0], dtype=np.int64)
    states = []
    for b in range(B):
        V = np_(random_state(ctx, 0.2, seed=30 + b)).astype(np.float64)
        D = np_(random_state(ctx, 0.2, seed=40 + b)).astype(np.float64)
        V[qpos[b] + 1:] = NEG
        rig.inject(1, b, V.astype(np.float32), D.astype(np.float32), 3)
        states.append((V, D))
    rig.set_qpos(qpos)
    _say("slot scores", R, blocks)
    z = torch.full((B, R, mb * 64), 7.0, device=DEV)
    spin.spin_slot_scores(rig.h, 1, rig.batch, z)
    torch.cuda.synchronize()
    zz = np_(z)
    for b in range(B):
        V, D = states[b]
        for r in range(R):
            q = int(qpos[b]) + r
            assert np.array_equal(zz[b, r, : q + 1], O.slot_scores(V, D, q)), (b, r)
            assert np.all(zz[b, r, q + 1:] == NEG), (b, r)
    assert rig.state.error() == 0


def _est_inputs(rng, B, R, mb, qpos, K, p_skip, p_expl, bias, grid):
    """Flags, ascending kept lists, kept-layout scores and each row's sparse
    top-k (taken by the oracle over the kept slots, then shuffled, with an
    ignored entry past the row's position where there is room)."""
    flags = np.zeros((B, mb), dtype=np.uint8)
    kept = np.full((B, mb), -1, dtype=np.int32)
    cnt = np.zeros(B, dtype=np.int32)
    scores = np.zeros((B, R, mb * 64), dtype=np.float32)
    topk = np.full((B, R, K), -1, dtype=np.int32)
    for b in range(B):
        n = nblocks(int(qpos[b]) + R - 1)
        u = rng.random(n)
        flags[b, :n] = np.where(u < p_skip, 0, np.where(u < p_skip + p_expl, 2, 1))
        flags[b, n:] = rng.integers(0, 3, mb - n)        # past the rows: never read
        kl = np.nonzero(flags[b, :n])[0]
        kept[b, : len(kl)] = kl
        cnt[b] = len(kl)
        boost = np.repeat(np.where(flags[b, kl] == 2, bias, 0.0), 64)
        for r in range(R):
            q = int(qpos[b]) + r
            v = rng.normal(size=len(kl) * 64) + boost
            if grid:
                v = np.round(v * grid) / grid                      # many equal scores
            scores[b, r, : len(v)] = v
            t = O.topk_positions(scores[b, r, : len(v)].astype(np.float64), kl, q, K)
            if (t < 0).any():
                t[np.nonzero(t < 0)[0][0]] = q + 1                 # ignored: past the row
            topk[b, r] = rng.permutation(t)
    return flags, kept, cnt, scores, topk


def _score_at(scores_row, kl, p):
    j = int(np.searchsorted(kl, p // 64))
    return float(scores_row[j * 64 + p % 64])


@pytest.mark.parametrize("R,mb,K,p_skip,p_expl,bias,grid", [
    (1, 200, 256, 0.5, 0.05, 0.0, 0), (4, 200, 2048, 0.5, 0.1, 0.5, 4), (2, 8192, 2048, 0.5, 0.05, 0.0, 0),
    (1, 64, 4096, 0.3, 0.2, 3.0, 0),        # explored slots on top: clamps for some rows
    (3, 300, 1024, 0.6, 0.1, -1.0, 2),      # explored slots low, heavy ties
    (2, 50, 256, 0.0, 0.1, 0.0, 0),         # nothing skipped: 0
    (2, 50, 256, 0.5, 0.0, 0.0, 0)])        # nothing explored: -1
def test_estimate_miss_exact(gpu_lib, R, mb, K, p_skip, p_expl, bias, grid):
    rng = np.random.default_rng(mb + K + R)
    B = 4
    qpos = np.array([64 * mb - R, 64 * (mb // 3) + 5, 63, 0], dtype=np.int64)
    flags, kept, cnt, scores, topk = _est_inputs(rng, B, R, mb, qpos, K, p_skip, p_expl, bias,
                                                 grid)
    qd = torch.as_tensor(qpos.astype(np.int32), device=DEV)
    slot = torch.arange(B, dtype=torch.int32, device=DEV)
    bt = spin.make_batch(slot, qd, R, mb)
    est = torch.full((B, R, 2), 5.0, device=DEV)
    _say("estimate miss", R, mb, K, p_skip, p_expl, bias, grid)
    spin.spin_estimate_miss(bt, K, torch.as_tensor(scores, device=DEV),
                            torch.as_tensor(kept, device=DEV), torch.as_tensor(cnt, device=DEV),
                            torch.as_tensor(topk, device=DEV), torch.as_tensor(flags, device=DEV),
                            est)
    torch.cuda.synchronize()
    got = np_(est)
    for b in range(B):
        kl = kept[b, : cnt[b]].astype(np.int64)
        for r in range(R):
            q = int(qpos[b]) + r
            t = topk[b, r]
            ts = [_score_at(scores[b, r], kl, int(p)) if 0 <= p <= q else 0.0 for p in t]
            want = O.estimate_miss(t, ts, flags[b], q, K)
            assert (np.float32(want[0]), np.float32(want[1])) == (got[b, r, 0], got[b, r, 1]), \
                (b, r, want, got[b, r])


def test_estimate_miss_bad_position_is_nan(gpu_lib):
    mb, R = 10, 2
    qd = torch.tensor([64 * mb - 1, -3], dtype=torch.int32, device=DEV)   # row 1 needs block 10
    bt = spin.make_batch(torch.zeros(2, dtype=torch.int32, device=DEV), qd, R, mb)
    est = torch.zeros(2, R, 2, device=DEV)
    spin.spin_estimate_miss(bt, 64, torch.zeros(2, R, mb * 64, device=DEV),
                            torch.zeros(2, mb, dtype=torch.int32, device=DEV),
                            torch.zeros(2, dtype=torch.int32, device=DEV),
                            torch.full((2, R, 64), -1, dtype=torch.int32, device=DEV),
                            torch.zeros(2, mb, dtype=torch.uint8, device=DEV), est)
    torch.cuda.synchronize()
    assert np.all(np.isnan(np_(est)))


def _pred_actual(rng, B, R, n, qpos, hole):
    actual = rng.normal(size=(B, R, n)).astype(np.float32)
    pred = (0.7 * actual + 0.5 * rng.normal(size=(B, R, n))).astype(np.float32)
    pred[rng.random(size=pred.shape) < hole] = NEG
    actual[rng.random(size=actual.shape) < hole / 4] = NEG
    for b in range(B):
        for r in range(R):
            q = int(qpos[b]) + r
            pred[b, r, q + 1:] = rng.normal(size=n - q - 1)           # past q: never read
            actual[b, r, q + 1:] = 1e30
    return pred, actual


@pytest.mark.parametrize("R,mb,K,hole", [(1, 100, 256, 0.1), (2, 300, 2048, 0.3),
                                          (1, 8192, 2048, 0.05), (4, 40, 4096, 0.0)])
def test_predictor_fidelity(gpu_lib, R, mb, K, hole):
    rng = np.random.default_rng(mb * 7 + R)
    B, n = 3, mb * 64
    qpos = np.array([n - R, n // 2 + 3, 0], dtype=np.int64)
    pred, actual = _pred_actual(rng, B, R, n, qpos, hole)
    qd = torch.as_tensor(qpos.astype(np.int32), device=DEV)
    bt = spin.make_batch(torch.arange(B, dtype=torch.int32, device=DEV), qd, R, mb)
    pd, ad = torch.as_tensor(pred, device=DEV), torch.as_tensor(actual, device=DEV)
    # both top-k lists from the GPU top-k over every block up to the row's last
    kept = torch.arange(mb, dtype=torch.int32, device=DEV)[None, :].repeat(B, 1).contiguous()
    cnt = torch.as_tensor([nblocks(int(q) + R - 1) for q in qpos], dtype=torch.int32, device=DEV)
    ws = torch.empty(max(256, spin.spin_topk_workspace_bytes(bt, K)), dtype=torch.uint8, device=DEV)
    tp = torch.empty(B, R, K, dtype=torch.int32, device=DEV)
    ta = torch.empty_like(tp)
    _say("predictor fidelity", R, mb, K, hole)
    spin.spin_topk_scores(bt, K, pd, kept, cnt, tp, ws)
    spin.spin_topk_scores(bt, K, ad, kept, cnt, ta, ws)
    out = torch.full((B, R, 2), 9.0, dtype=torch.float64, device=DEV)
    spin.spin_predictor_fidelity(bt, K, pd, ad, tp, ta, out)
    torch.cuda.synchronize()
    got = np_(out)
    for b in range(B):
        for r in range(R):
            q = int(qpos[b]) + r
            p64 = pred[b, r, : q + 1].astype(np.float64)
            a64 = actual[b, r, : q + 1].astype(np.float64)
            assert abs(got[b, r, 0] - O.pearson(p64, a64)) <= 1e-10, (b, r)
            assert got[b, r, 1] == O.topk_recall(p64, a64, K), (b, r)
