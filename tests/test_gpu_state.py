"""State checkpoint / resume and mid-trajectory slot reset (the state buffer
is the whole SPIN state: a byte copy restored later, or into another buffer,
replays bit for bit; restarting one request leaves every other one alone)."""
import dataclasses

import numpy as np
import pytest
import torch

import predictive_kv_block_amd as spin
from oracle import spin_oracle as O
from tests.spin_harness import np_, oracle_fp8_operands, predicted_sets_tie_only
from workload import WORKLOADS, make_pool, make_queries, positions

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


class _Run:
    """One state buffer plus the per-call buffers of a batch of B requests."""

    def __init__(self, wl, B, layers=1, st=None):
        self.wl, self.B = wl, B
        nb = wl.blocks
        self.cfg = spin.make_config(layers, B, wl.ctx, wl.topk, explore_bp=wl.explore_bp,
                                    alpha=wl.alpha)
        self.st = st or spin.SpinState(self.cfg)
        self.slot = torch.arange(B, dtype=torch.int32, device=DEV)
        self.qpos = torch.zeros(B, dtype=torch.int32, device=DEV)
        self.batch = spin.make_batch(self.slot, self.qpos, 1, nb)
        self.kept = torch.zeros(B, nb, dtype=torch.int32, device=DEV)
        self.cnt = torch.zeros(B, dtype=torch.int32, device=DEV)
        self.flags = torch.zeros(B, nb, dtype=torch.uint8, device=DEV)
        self.scores = torch.zeros(B, 1, nb * 64, device=DEV)
        self.topk = torch.zeros(B, 1, wl.topk, dtype=torch.int32, device=DEV)

    def round(self, pool, layer, t, q, keep_bp):
        """predict -> quantise + index + top-k -> update; returns the outputs."""
        self.qpos.copy_(torch.as_tensor(np.asarray(q, dtype=np.int32)))
        qb, w = make_queries(self.wl, pool, layer, t, q, device=DEV)
        h = self.st.handle
        spin.spin_predict_blocks(h, layer, self.batch, keep_bp, self.kept, self.cnt, self.flags)
        spin.spin_indexer_topk(h, self.batch, qb, w, pool.key_codes, pool.key_scale,
                               pool.block_table, self.kept, self.cnt, self.scores, self.topk)
        spin.spin_update(h, layer, self.batch, self.scores, self.kept, self.cnt)
        torch.cuda.synchronize()
        cnt = np_(self.cnt).copy()
        out = {"cnt": cnt, "topk": np_(self.topk).copy(), "flags": np_(self.flags).copy()}
        out["kept"] = [np_(self.kept[b, : cnt[b]]).copy() for b in range(self.B)]
        out["scores"] = [np_(self.scores[b, 0, : cnt[b] * 64]).copy() for b in range(self.B)]
        return out, (qb, w)

    def state_regions(self):
        s = self.st
        return {"V": np_(s.V()).copy(), "D": np_(s.D()).copy(), "VB": np_(s.VB()).copy(),
                "step": np_(s.step()).copy()}


def _bits_equal(x, y):
    x, y = np.ascontiguousarray(x), np.ascontiguousarray(y)
    return x.shape == y.shape and np.array_equal(x.view(np.uint8), y.view(np.uint8))


def _same(a, b, what):
    for k in a:
        if isinstance(a[k], list):
            for i, (x, y) in enumerate(zip(a[k], b[k])):
                assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{what}: {k}[{i}]"
        else:
            assert np.array_equal(np.asarray(a[k]).view(np.uint8),
                                  np.asarray(b[k]).view(np.uint8)), f"{what}: {k}"


def test_checkpoint_restore_replays_bit_identical(gpu_lib):
    wl = dataclasses.replace(WORKLOADS["ctx9k-b1"], batch=3)
    pool = make_pool(wl, 0, device=DEV)
    qp = np_(positions(wl))
    keeps = [10000, 6000, 5000, 7000, 5000, 6000]
    run = _Run(wl, 3)
    spin.spin_reset_slots(run.st.handle, run.slot,
                          torch.tensor([11, 12, 13], dtype=torch.int64, device=DEV))
    for t in range(3):
        run.round(pool, 0, t, qp[t], keeps[t])
    _say("checkpoint after round 2")
    ckpt = run.st.mem.clone()
    first = [run.round(pool, 0, t, qp[t], keeps[t])[0] for t in range(3, 6)]
    end_state = run.state_regions()
    end_bytes = run.st.mem.clone()

    _say("restore into the same buffer")
    run.st.mem.copy_(ckpt)
    torch.cuda.synchronize()
    again = [run.round(pool, 0, t, qp[t], keeps[t])[0] for t in range(3, 6)]
    for t, (a, b) in enumerate(zip(first, again)):
        _same(a, b, f"same buffer, round {t + 3}")
    _same(end_state, run.state_regions(), "same buffer, final state")
    assert torch.equal(end_bytes, run.st.mem)

    _say("restore into a second buffer bound by its own handle")
    other = _Run(wl, 3)
    other.st.mem.copy_(ckpt)
    torch.cuda.synchronize()
    moved = [other.round(pool, 0, t, qp[t], keeps[t])[0] for t in range(3, 6)]
    for t, (a, b) in enumerate(zip(first, moved)):
        _same(a, b, f"second buffer, round {t + 3}")
    _same(end_state, other.state_regions(), "second buffer, final state")
    assert run.st.error() == 0 and other.st.error() == 0


def test_reset_one_slot_mid_trajectory(gpu_lib):
    wl = dataclasses.replace(WORKLOADS["ctx9k-b1"], batch=4)
    layers = 2
    pools = [make_pool(wl, l, device=DEV) for l in range(layers)]
    qp = np_(positions(wl))
    keeps = [10000, 5000, 6000, 5000, 5000, 7000]
    rids = torch.tensor([21, 22, 23, 24], dtype=torch.int64, device=DEV)
    ref_run, run = _Run(wl, 4, layers), _Run(wl, 4, layers)
    for r in (ref_run, run):
        spin.spin_reset_slots(r.st.handle, r.slot, rids)
    for t in range(3):
        for l in range(layers):
            a, _ = ref_run.round(pools[l], l, t, qp[t], keeps[t])
            b, _ = run.round(pools[l], l, t, qp[t], keeps[t])
            _same(a, b, f"before the reset, round {t} layer {l}")

    reset_slot, new_rid = 2, 777
    before = run.state_regions()
    _say("reset slot", reset_slot, "before round 3")
    spin.spin_reset_slots(run.st.handle, torch.tensor([reset_slot], dtype=torch.int32, device=DEV),
                          torch.tensor([new_rid], dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    after = run.state_regions()
    others = [s for s in range(4) if s != reset_slot]
    for k in ("V", "D", "VB", "step"):
        assert _bits_equal(after[k][:, others], before[k][:, others]), k
    assert np.all(after["V"][:, reset_slot] == -np.inf) and np.all(after["D"][:, reset_slot] == -np.inf)
    assert np.all(after["VB"][:, reset_slot] == -np.inf) and np.all(after["step"][:, reset_slot] == 0)
    rid_region = run.st.region("request_id", torch.int64, (4,))
    assert int(rid_region[reset_slot]) == new_rid

    # The restarted request against a fresh oracle state with its new id; the
    # others bit-identical to the run without the reset.
    kv = [O.e4m3fn_decode(np_(p.key_codes)) for p in pools]
    sc = [np_(p.key_scale).astype(np.float64) for p in pools]
    ost = [O.RequestState(wl.ctx, request_id=new_rid) for _ in range(layers)]
    before_ost = [None] * layers
    live = [True] * layers
    for t in range(3, 6):
        for l in range(layers):
            a, _ = ref_run.round(pools[l], l, t, qp[t], keeps[t])
            b, (qb, w) = run.round(pools[l], l, t, qp[t], keeps[t])
            for s in others:
                for k in ("kept", "scores"):
                    assert np.array_equal(a[k][s], b[k][s]), (t, l, s, k)
                assert np.array_equal(a["topk"][s], b["topk"][s]), (t, l, s)
                assert np.array_equal(a["flags"][s], b["flags"][s]), (t, l, s)
            qv, wv, _, _ = oracle_fp8_operands(qb[reset_slot], w[reset_slot])
            before_ost[l] = ost[l].copy()
            ref = O.decode_round(ost[l], int(qp[t, reset_slot]), 1, keeps[t], wl.explore_bp,
                                 run.cfg.seed, l, qv, wv, kv[l], sc[l],
                                 np_(pools[l].block_table[reset_slot]), wl.topk, wl.alpha)
            if t == 3:
                # its first round after the reset is the all-keep warm-up
                n_blocks = int(qp[t, reset_slot]) // 64 + 1
                assert b["cnt"][reset_slot] == n_blocks and len(ref["kept"]) == n_blocks
                assert np.array_equal(b["kept"][reset_slot], ref["kept"]), (t, l)
            elif t == 4 and live[l]:
                # the first sparse round: exact, or an fp32-vs-fp64 tie at the
                # predicted-set threshold (then this layer's comparison stops)
                if not np.array_equal(b["kept"][reset_slot], ref["kept"]):
                    assert predicted_sets_tie_only(
                        before_ost[l], int(qp[t, reset_slot]), 1, keeps[t], wl.explore_bp,
                        np.nonzero(b["flags"][reset_slot] == 1)[0].tolist(),
                        np.nonzero(ref["flags"] == 1)[0].tolist()), (t, l)
                    live[l] = False
        st_a, st_b = ref_run.state_regions(), run.state_regions()
        for k in ("V", "D", "VB", "step"):
            assert _bits_equal(st_a[k][:, others], st_b[k][:, others]), (t, k)
        assert np.all(st_b["step"][:, reset_slot] == t - 2)
    assert run.st.error() == 0 and ref_run.st.error() == 0
