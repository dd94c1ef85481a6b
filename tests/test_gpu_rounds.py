"""Whole SPIN rounds on the GPU against the oracle.

Free-running: the GPU and the oracle each evolve their own state from the same
generated inputs.  Each round compares kept blocks (exact, or a tie at the
selection threshold within tolerance), indexer scores, top-k (tie-aware) and
the EMA state.  After a tolerated tie the two trajectories legitimately part:
the oracle's state, rounded to fp32, is then written into that GPU slot and
the comparison goes on from the next round.

Lockstep: before every round the oracle's state is rounded to fp32 on both
sides, so the predictor starts from identical values and its block selection
must match exactly in every round.

Data only ever flows oracle -> GPU; the oracle never takes a value from the
GPU.
"""
import dataclasses

import numpy as np
import pytest
import torch

import predictive_kv_block_amd as spin
from oracle import spin_oracle as O
from tests.spin_harness import (NEG, Rig, assert_scores_close, assert_topk_tie_aware, nblocks,
                                np_, oracle_fp8_operands, predicted_sets_tie_only, score_mag,
                                score_tol, sync_from_oracle)
from workload import WORKLOADS, acceptances, make_pool, make_queries, positions

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


def _state_close(g, r, scale, what):
    fin = np.isfinite(r)
    assert np.array_equal(fin, np.isfinite(g)), f"{what}: observed sets differ"
    tol = np.maximum(1e-3 * np.abs(r[fin]), 1e-5 * scale)
    err = np.abs(g[fin] - r[fin])
    assert np.all(err <= tol), f"{what}: worst {err.max():.3e}"


def _predicted_sets_tie_only(ost_before, q, R, keep_bp, explore_bp, gpu_flags, ref_flags):
    """True if every predicted-set difference sits within tolerance of a row's threshold."""
    return predicted_sets_tie_only(ost_before, q, R, keep_bp, explore_bp,
                                   np.nonzero(gpu_flags == 1)[0].tolist(),
                                   np.nonzero(ref_flags == 1)[0].tolist())


# ---------------------------------------------------------------- tiny 4K
def test_tiny4k_trajectory_with_oracle_scores(gpu_lib):
    """fp32 4096-token workload: the GPU runs predict, top-k and update on the
    oracle's fp64 scores rounded to fp32 (its indexer is fp8-only)."""
    wl = WORKLOADS["tiny-4k"]
    pool = make_pool(wl, 0, device="cpu")
    kv = np_(pool.key_f32).astype(np.float64)
    table = np_(pool.block_table[0])
    ones = np.ones(kv.shape[0])
    keep_bp = 10000 - wl.sparsity_bp[0]
    cfg = spin.make_config(1, 1, wl.ctx, wl.topk, heads=wl.heads, head_dim=wl.head_dim,
                           explore_bp=wl.explore_bp, alpha=wl.alpha)
    rig = Rig(cfg, 1, 1, wl.blocks)
    rig.reset([7])
    ost = O.RequestState(wl.ctx, request_id=7)
    qp = np_(positions(wl))[:, 0]
    compared = ties = 0
    for t in range(wl.steps):
        q = int(qp[t])
        qf, w = make_queries(wl, pool, 0, t, [q])
        qv, wv = np_(qf[0]).astype(np.float64), np_(w[0]).astype(np.float64)
        before = ost.copy()
        kb = keep_bp
        ref = O.decode_round(ost, q, 1, kb, wl.explore_bp, cfg.seed, 0, qv, wv, kv, ones, table,
                             wl.topk, wl.alpha)
        rig.set_qpos([q])
        spin.spin_predict_blocks(rig.h, 0, rig.batch, kb, rig.kept, rig.kept_count, rig.flags)
        torch.cuda.synchronize()
        gk = rig.kept_list(0)
        if not np.array_equal(gk, ref["kept"]):
            assert _predicted_sets_tie_only(before, q, 1, kb, wl.explore_bp,
                                            np_(rig.flags[0])[: len(ref["flags"])], ref["flags"]), \
                f"round {t}: kept blocks differ beyond a threshold tie"
            _say("tolerated threshold tie: round", t, "-> oracle state synced")
            sync_from_oracle(rig, 0, 0, ost)
            ties += 1
            continue
        sc = np.full((1, 1, wl.blocks * 64), NEG, dtype=np.float32)
        sc[0, 0, : len(gk) * 64] = ref["scores"][0].astype(np.float32)
        rig.scores.copy_(torch.as_tensor(sc))
        spin.spin_topk_scores(rig.batch, wl.topk, rig.scores, rig.kept, rig.kept_count, rig.topk,
                              rig.topk_ws)
        spin.spin_update(rig.h, 0, rig.batch, rig.scores, rig.kept, rig.kept_count)
        torch.cuda.synchronize()
        s32 = {int(x): float(v) for x, v in zip(
            (gk[:, None] * 64 + np.arange(64)).reshape(-1), sc[0, 0, : len(gk) * 64])}
        assert_topk_tie_aware(np_(rig.topk[0, 0]), ref["topk"][0], lambda x: s32[x],
                              lambda x: 1e-6 * abs(s32[x]) + 1e-9, f"round {t}")
        gV, gD, _, gstep = rig.read_state(0, 0)
        scale = np.abs(ref["scores"][np.isfinite(ref["scores"])]).max()
        _state_close(gV, ost.V, scale, f"V round {t}")
        _state_close(gD, ost.D, scale, f"D round {t}")
        assert gstep == ost.step
        compared += 1
    _say("tiny4k rounds compared", compared, "ties", ties)
    assert compared + ties == wl.steps and compared >= 21


# ------------------------------------------------------- 9.7K fp8 indexer
def _run_rounds(wl, keep_bps, n_rounds, B=None, layer=0, check_state=True, lockstep=False):
    """Returns (rounds compared in full, tolerated ties)."""
    B = B or wl.batch
    wl = dataclasses.replace(wl, batch=B)
    pool = make_pool(wl, layer, device=DEV)
    kv = O.e4m3fn_decode(np_(pool.key_codes))
    scv = np_(pool.key_scale).astype(np.float64)
    tables = np_(pool.block_table)
    cfg = spin.make_config(layer + 1, B, wl.ctx, wl.topk, explore_bp=wl.explore_bp, alpha=wl.alpha)
    rig = Rig(cfg, B, 1, wl.blocks)
    rids = [500 + b for b in range(B)]
    rig.reset(rids)
    osts = [O.RequestState(wl.ctx, request_id=rids[b]) for b in range(B)]
    qp = np_(positions(wl))
    compared = ties = 0
    for t in range(n_rounds):
        kb = keep_bps[t % len(keep_bps)] if t > 0 else 10000
        q = qp[t]
        qb, w = make_queries(wl, pool, layer, t, q, device=DEV)
        rig.set_qpos(q)
        if lockstep and t > 0:
            for b in range(B):
                sync_from_oracle(rig, layer, b, osts[b], lockstep=True)
        spin.spin_predict_blocks(rig.h, layer, rig.batch, kb, rig.kept, rig.kept_count, rig.flags)
        spin.spin_indexer_topk(rig.h, rig.batch, qb, w, pool.key_codes, pool.key_scale,
                               pool.block_table, rig.kept, rig.kept_count, rig.scores, rig.topk)
        torch.cuda.synchronize()
        g_scores = np_(rig.scores)
        g_topk = np_(rig.topk)
        spin.spin_update(rig.h, layer, rig.batch, rig.scores, rig.kept, rig.kept_count)
        torch.cuda.synchronize()
        for b in range(B):
            qv, wv, _, _ = oracle_fp8_operands(qb[b], w[b])
            before = osts[b].copy()
            ref = O.decode_round(osts[b], int(q[b]), 1, kb, wl.explore_bp, cfg.seed, layer, qv,
                                 wv, kv, scv, tables[b], wl.topk, wl.alpha)
            gk = rig.kept_list(b)
            gflags = np_(rig.flags[b])[: len(ref["flags"])]
            if not (np.array_equal(gk, ref["kept"]) and np.array_equal(gflags, ref["flags"])):
                assert not lockstep, f"round {t} b{b}: kept blocks differ from identical states"
                assert _predicted_sets_tie_only(before, int(q[b]), 1, kb, wl.explore_bp,
                                                np_(rig.flags[b])[: len(ref["flags"])],
                                                ref["flags"]), f"round {t} b{b}: kept differ"
                _say("tolerated threshold tie: round", t, "request", b, "-> oracle state synced")
                sync_from_oracle(rig, layer, b, osts[b])
                ties += 1
                continue
            n = len(gk) * 64
            mag = score_mag(qv, wv, kv, scv, tables[b], gk)
            assert_scores_close(g_scores[b, :, :n], ref["scores"], mag, f"round {t} b{b}")
            slots = (gk[:, None] * 64 + np.arange(64)).reshape(-1)
            rs = dict(zip(slots.tolist(), ref["scores"][0].tolist()))
            mg = dict(zip(slots.tolist(), mag[0].tolist()))
            assert_topk_tie_aware(g_topk[b, 0], ref["topk"][0], lambda x: rs[x],
                                  lambda x: score_tol(rs[x], mg[x]), f"round {t} b{b}")
            if check_state:
                gV, gD, gVB, gstep = rig.read_state(layer, b)
                scale = float(np.max(mag))
                _state_close(gV, osts[b].V, scale, f"V round {t} b{b}")
                _state_close(gD, osts[b].D, scale, f"D round {t} b{b}")
                assert gstep == osts[b].step
            compared += 1
    assert rig.state.error() == 0
    return compared, ties


def test_ctx9k_trajectory(gpu_lib):
    wl = WORKLOADS["ctx9k-b1"]
    _say("ctx9k-b1 rounds at 20/30/40/50%")
    n, ties = _run_rounds(wl, [8000, 7000, 6000, 5000], 12)
    assert n + ties == 12 and n >= 8


def test_ctx9k_trajectory_lockstep(gpu_lib):
    wl = WORKLOADS["ctx9k-b1"]
    _say("ctx9k-b1 lockstep rounds at 20/30/40/50%")
    n, ties = _run_rounds(wl, [8000, 7000, 6000, 5000], 16, lockstep=True)
    assert n == 16 and ties == 0


def test_ctx94k_trajectory_two_requests(gpu_lib):
    wl = WORKLOADS["ctx94k-b8"]
    _say("ctx94k two requests, 50%")
    n, ties = _run_rounds(wl, [5000], 6, B=2)
    assert n + ties == 12 and n >= 8


def test_ctx94k_lockstep_three_requests(gpu_lib):
    wl = WORKLOADS["ctx94k-b8"]
    _say("ctx94k three requests lockstep, 30/50%")
    n, ties = _run_rounds(wl, [3000, 5000], 6, B=3, lockstep=True)
    assert n == 18 and ties == 0


def test_determinism_bit_identical(gpu_lib):
    wl = dataclasses.replace(WORKLOADS["ctx9k-b1"], batch=2)
    pool = make_pool(wl, 0, device=DEV)
    outs = []
    for rep in range(2):
        cfg = spin.make_config(1, 2, wl.ctx, wl.topk, explore_bp=wl.explore_bp, alpha=wl.alpha)
        rig = Rig(cfg, 2, 1, wl.blocks)
        rig.reset([1, 2])
        qp = np_(positions(wl))
        rec = []
        for t in range(5):
            qb, w = make_queries(wl, pool, 0, t, qp[t], device=DEV)
            rig.set_qpos(qp[t])
            kb = 10000 if t == 0 else 6000
            spin.spin_predict_blocks(rig.h, 0, rig.batch, kb, rig.kept, rig.kept_count, rig.flags)
            spin.spin_indexer_topk(rig.h, rig.batch, qb, w, pool.key_codes, pool.key_scale,
                                   pool.block_table, rig.kept, rig.kept_count, rig.scores, rig.topk)
            spin.spin_update(rig.h, 0, rig.batch, rig.scores, rig.kept, rig.kept_count)
            torch.cuda.synchronize()
            rec.append((np_(rig.kept).copy(), np_(rig.scores).copy(), np_(rig.topk).copy()))
        rec.append((np_(rig.state.V()).copy(), np_(rig.state.D()).copy(), np_(rig.state.VB()).copy()))
        outs.append(rec)
    for a, b in zip(outs[0], outs[1]):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


# --------------------------------------------------------------------- MTP
def _mtp_rounds(lockstep):
    """4 query rows, 2 layers with their own keys and state, prefix-valid
    replay.  Returns (request-layer rounds compared in full, tolerated ties)."""
    base = WORKLOADS["mtp-ctx256k-b32"]
    wl = dataclasses.replace(base, batch=3, ctx=64 * 260, layers=2, steps=6)
    acc = np_(acceptances(wl))
    qp = np_(positions(wl, torch.as_tensor(acc)))
    cfg = spin.make_config(wl.layers, wl.batch, wl.ctx, wl.topk, max_rows=wl.rows,
                           explore_bp=wl.explore_bp, alpha=wl.alpha)
    rig = Rig(cfg, wl.batch, wl.rows, wl.blocks)
    rids = [900 + b for b in range(wl.batch)]
    rig.reset(rids)
    pools = [make_pool(wl, l, device=DEV) for l in range(wl.layers)]
    kvs = [O.e4m3fn_decode(np_(p.key_codes)) for p in pools]
    scs = [np_(p.key_scale).astype(np.float64) for p in pools]
    osts = [[O.RequestState(wl.ctx, request_id=rids[b]) for b in range(wl.batch)]
            for _ in range(wl.layers)]
    compared = ties = 0
    keep = [10000, 5000, 4500, 6000, 5000, 5000]
    for t in range(wl.steps):
        rig.set_qpos(qp[t])
        a_dev = torch.as_tensor(acc[t].astype(np.int32), device=DEV)
        for layer in range(wl.layers):
            pool = pools[layer]
            if lockstep and t > 0:
                for b in range(wl.batch):
                    sync_from_oracle(rig, layer, b, osts[layer][b], lockstep=True)
            qb, w = make_queries(wl, pool, layer, t, qp[t], device=DEV)
            kb = keep[t]
            spin.spin_predict_blocks(rig.h, layer, rig.batch, kb, rig.kept, rig.kept_count, rig.flags)
            spin.spin_indexer_topk(rig.h, rig.batch, qb, w, pool.key_codes, pool.key_scale,
                                   pool.block_table, rig.kept, rig.kept_count, rig.scores, rig.topk)
            torch.cuda.synchronize()
            g_scores, g_topk = np_(rig.scores), np_(rig.topk)
            spin.spin_mtp_replay(rig.h, layer, rig.batch, a_dev, rig.scores, rig.kept, rig.kept_count)
            torch.cuda.synchronize()
            tables = np_(pool.block_table)
            for b in range(wl.batch):
                qv, wv, _, _ = oracle_fp8_operands(qb[b], w[b])
                before = osts[layer][b].copy()
                ref = O.decode_round(osts[layer][b], int(qp[t, b]), wl.rows, kb, wl.explore_bp,
                                     cfg.seed, layer, qv, wv, kvs[layer], scs[layer], tables[b],
                                     wl.topk, wl.alpha, accepted=int(acc[t, b]))
                gk = rig.kept_list(b)
                gflags = np_(rig.flags[b])[: len(ref["flags"])]
                if not (np.array_equal(gk, ref["kept"]) and np.array_equal(gflags, ref["flags"])):
                    assert not lockstep, f"t{t} l{layer} b{b}: kept differ from identical states"
                    assert _predicted_sets_tie_only(before, int(qp[t, b]), wl.rows, kb,
                                                    wl.explore_bp, np_(rig.flags[b])[: len(ref["flags"])],
                                                    ref["flags"]), f"t{t} l{layer} b{b}: kept differ"
                    _say("tolerated threshold tie", t, layer, b, "-> oracle state synced")
                    sync_from_oracle(rig, layer, b, osts[layer][b])
                    ties += 1
                    continue
                n = len(gk) * 64
                mag = score_mag(qv, wv, kvs[layer], scs[layer], tables[b], gk)
                assert_scores_close(g_scores[b, :, :n], ref["scores"], mag, f"t{t} l{layer} b{b}")
                slots = (gk[:, None] * 64 + np.arange(64)).reshape(-1)
                for r in range(wl.rows):
                    rs = dict(zip(slots.tolist(), ref["scores"][r].tolist()))
                    mg = dict(zip(slots.tolist(), mag[r].tolist()))
                    assert_topk_tie_aware(g_topk[b, r], ref["topk"][r], lambda x: rs[x],
                                          lambda x: score_tol(rs[x], mg[x]), f"t{t} l{layer} b{b} r{r}")
                gV, gD, _, gstep = rig.read_state(layer, b)
                scale = float(np.max(mag))
                _state_close(gV, osts[layer][b].V, scale, f"V t{t} l{layer} b{b}")
                _state_close(gD, osts[layer][b].D, scale, f"D t{t} l{layer} b{b}")
                assert gstep == osts[layer][b].step
                compared += 1
    assert rig.state.error() == 0
    _say("mtp rounds compared", compared, "ties", ties)
    return compared, ties


def test_mtp_union_and_replay_rounds(gpu_lib):
    n, ties = _mtp_rounds(lockstep=False)
    assert n + ties == 36 and n >= 24


def test_mtp_union_and_replay_lockstep(gpu_lib):
    n, ties = _mtp_rounds(lockstep=True)
    assert n == 36 and ties == 0


# ------------------------------------------------------ start of a sequence
@pytest.mark.parametrize("R", [1, 4])
def test_sequence_start_lockstep(gpu_lib, R):
    """The first positions of a sequence, in lockstep with the oracle: a
    one-slot context, a first block with one slot left, a full first block,
    the first two-block context (the first real selection), and with four
    rows, rows that cross the first block boundary.  Every round runs the
    whole path (quantise, predict, indexer, top-k with fewer valid slots than
    K, update or prefix-valid replay)."""
    base = WORKLOADS["ctx9k-b1"] if R == 1 else WORKLOADS["mtp-ctx256k-b32"]
    starts = [0, 1, 62, 63, 64, 126] if R == 1 else [0, 1, 58, 60, 61, 62]
    steps = 5
    wl = dataclasses.replace(base, batch=len(starts), ctx=64 * 4, layers=1, steps=steps,
                             heavy=(4,))
    acc = (np.random.default_rng(3).integers(0, R, size=(steps, wl.batch))
           if R > 1 else np.zeros((steps, wl.batch), dtype=np.int64))
    qp = np.zeros((steps, wl.batch), dtype=np.int64)
    qp[0] = starts
    for t in range(1, steps):
        qp[t] = qp[t - 1] + acc[t - 1] + 1
    assert int((qp[-1] + R - 1).max()) < wl.ctx
    cfg = spin.make_config(1, wl.batch, wl.ctx, wl.topk, max_rows=R, explore_bp=wl.explore_bp,
                           alpha=wl.alpha)
    rig = Rig(cfg, wl.batch, R, wl.blocks)
    rids = [700 + b for b in range(wl.batch)]
    rig.reset(rids)
    pool = make_pool(wl, 0, device=DEV)
    kv = O.e4m3fn_decode(np_(pool.key_codes))
    scv = np_(pool.key_scale).astype(np.float64)
    tables = np_(pool.block_table)
    osts = [O.RequestState(wl.ctx, request_id=rids[b]) for b in range(wl.batch)]
    keep = [10000, 5000, 3000, 6000, 5000]
    for t in range(steps):
        _say("sequence start R", R, "round", t, "positions", qp[t].tolist())
        rig.set_qpos(qp[t])
        if t > 0:
            for b in range(wl.batch):
                sync_from_oracle(rig, 0, b, osts[b], lockstep=True)
        qb, w = make_queries(wl, pool, 0, t, qp[t].tolist(), device=DEV)
        spin.spin_predict_blocks(rig.h, 0, rig.batch, keep[t], rig.kept, rig.kept_count,
                                 rig.flags)
        spin.spin_indexer_topk(rig.h, rig.batch, qb, w, pool.key_codes, pool.key_scale,
                               pool.block_table, rig.kept, rig.kept_count, rig.scores, rig.topk)
        torch.cuda.synchronize()
        g_scores, g_topk = np_(rig.scores), np_(rig.topk)
        if R == 1:
            spin.spin_update(rig.h, 0, rig.batch, rig.scores, rig.kept, rig.kept_count)
        else:
            spin.spin_mtp_replay(rig.h, 0, rig.batch,
                                 torch.as_tensor(acc[t].astype(np.int32), device=DEV),
                                 rig.scores, rig.kept, rig.kept_count)
        torch.cuda.synchronize()
        for b in range(wl.batch):
            q = int(qp[t, b])
            qv, wv, _, _ = oracle_fp8_operands(qb[b], w[b])
            ref = O.decode_round(osts[b], q, R, keep[t], wl.explore_bp, cfg.seed, 0, qv, wv, kv,
                                 scv, tables[b], wl.topk, wl.alpha, accepted=int(acc[t, b]))
            gk = rig.kept_list(b)
            assert np.array_equal(gk, ref["kept"]), f"t{t} b{b}: kept blocks"
            assert np.array_equal(np_(rig.flags[b])[: len(ref["flags"])], ref["flags"]), \
                f"t{t} b{b}: flags"
            n = len(gk) * 64
            mag = score_mag(qv, wv, kv, scv, tables[b], gk)
            assert_scores_close(g_scores[b, :, :n], ref["scores"], mag, f"t{t} b{b}")
            slots = (gk[:, None] * 64 + np.arange(64)).reshape(-1)
            for r in range(R):
                valid = int(np.sum(slots <= q + r))
                assert valid < wl.topk                      # fewer valid slots than K
                assert np.all(g_topk[b, r, valid:] == -1), f"t{t} b{b} r{r}: padding"
                rs = dict(zip(slots.tolist(), ref["scores"][r].tolist()))
                mg = dict(zip(slots.tolist(), mag[r].tolist()))
                assert_topk_tie_aware(g_topk[b, r], ref["topk"][r], lambda x: rs[x],
                                      lambda x: score_tol(rs[x], mg[x]), f"t{t} b{b} r{r}")
            gV, gD, _, gstep = rig.read_state(0, b)
            scale = float(np.max(mag))
            _state_close(gV, osts[b].V, scale, f"V t{t} b{b}")
            _state_close(gD, osts[b].D, scale, f"D t{t} b{b}")
            assert gstep == osts[b].step
    assert rig.state.error() == 0
