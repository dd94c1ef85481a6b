"""The benchmark's two round schedules (the EMA update beside the top-k on a
second stream behind the library's gate, the streams taking turns from round
to round; or the update behind the top-k on one stream; in both, two sets of
round outputs and one position row per round) against the same calls issued
one after another on one stream: every output and the whole state must be
bit-identical, round after round, with a host synchronisation after every
round and without any (the rounds' outputs then copied on the stream).  A
missing dependency between the streams or between rounds would show up here
as a difference.  Also: spin_topk_update equals spin_topk_scores followed by
spin_update / spin_mtp_replay, bit for bit."""
import dataclasses

import numpy as np
import pytest
import torch

import bench
import predictive_kv_block_amd as spin
from tests.spin_harness import np_
from workload import WORKLOADS, acceptances, make_queries, positions

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _serial_round(st, b, pool, q, w, keep_bp):
    spin.spin_predict_blocks(st.handle, 0, b["batch"], keep_bp, b["kept"], b["cnt"], b["flags"])
    spin.spin_quantize_q(st.handle, b["batch"], q, w)
    spin.spin_indexer_scores(st.handle, b["batch"], pool.key_codes, pool.key_scale,
                             pool.block_table, b["kept"], b["cnt"], b["scores"], b["pq"])
    spin.spin_topk_scores(b["batch"], st.cfg.topk, b["scores"], b["kept"], b["cnt"], b["topk"],
                          b["topk_ws"], b["pq"])
    spin.spin_update(st.handle, 0, b["batch"], b["scores"], b["kept"], b["cnt"])


_KEYS = ("kept", "cnt", "flags", "scores", "pq", "topk")


def _snapshot_dev(st, b):
    """Copies of a round's outputs and the state, enqueued on the current stream."""
    d = {k: b[k].clone() for k in _KEYS}
    d.update(V=st.V().clone(), D=st.D().clone(), VB=st.VB().clone(), step=st.step().clone())
    return d


def _host(d):
    return {k: np_(v).copy() for k, v in d.items()}


def _masked_scores(s, cnt):
    """Scores past each request's kept count are never written: blank them."""
    out = s.copy()
    for b, c in enumerate(cnt):
        out[b, :, int(c) * 64:] = 0.0
    return out


def _same(a, b, t):
    assert np.array_equal(a["cnt"], b["cnt"]), t
    for bi, c in enumerate(a["cnt"]):          # entries past the count are not written
        assert np.array_equal(a["kept"][bi, : int(c)], b["kept"][bi, : int(c)]), (t, "kept", bi)
    for k in ("flags", "topk", "V", "D", "VB", "step"):
        assert np.array_equal(a[k], b[k]), (t, k)
    assert np.array_equal(_masked_scores(a["scores"], a["cnt"]),
                          _masked_scores(b["scores"], b["cnt"])), (t, "scores")
    for bi, c in enumerate(a["cnt"]):
        assert np.array_equal(a["pq"][bi, :, : int(c)], b["pq"][bi, :, : int(c)]), (t, "pq")


def test_benchmark_round_equals_serial(gpu_lib):
    wl = dataclasses.replace(WORKLOADS["ctx94k-b8"], steps=6)
    qp = np_(positions(wl))
    runs = {}
    modes = ("serial", "beside-synced", "beside-unsynced", "behind-synced", "behind-unsynced")
    for mode in modes:
        print("[case] stream plan", mode, flush=True)
        spin_, pool, cfg, st, bufs, _ = bench._setup(wl, DEV)
        streams = (torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV))
        qs = [make_queries(wl, pool, 0, t, qp[t].tolist(), device=DEV) for t in range(wl.steps)]
        qpos = torch.as_tensor(qp.astype(np.int32), device=DEV).contiguous()
        batches = [spin.make_batch(bufs["slot"], qpos[t], wl.rows, wl.blocks)
                   for t in range(wl.steps)]
        torch.cuda.synchronize()
        snaps = []
        tail = mode.split("-")[0]
        for t in range(wl.steps):
            keep = 10000 if t == 0 else 5000
            if mode == "serial":
                bufs["qpos"].copy_(qpos[t])
                _serial_round(st, bufs, pool, qs[t][0], qs[t][1], keep)
                out = bufs
            else:
                out = bench._round(spin, st, bufs, pool, batches[t], qs[t][0], qs[t][1], keep,
                                   streams, t, tail=tail)
            if mode.endswith("unsynced"):
                # on the stream the next round's chain runs on, once the
                # round's top-k and update are both done
                main = streams[t % 2] if tail == "beside" else streams[0]
                nxt = streams[(t + 1) % 2] if tail == "beside" else streams[0]
                done = torch.cuda.Event()
                done.record(main)
                nxt.wait_event(done)
                with torch.cuda.stream(nxt):
                    snaps.append(_snapshot_dev(st, out))
            else:
                torch.cuda.synchronize()
                snaps.append(_host(_snapshot_dev(st, out)))
        torch.cuda.synchronize()
        if mode.endswith("unsynced"):
            snaps = [_host(d) for d in snaps]
        assert st.error() == 0
        runs[mode] = snaps
    for mode in modes[1:]:
        for t, (a, b) in enumerate(zip(runs["serial"], runs[mode])):
            _same(a, b, (mode, t))


@pytest.mark.parametrize("R", [1, 4])
def test_topk_update_equals_separate_calls(gpu_lib, R):
    base = WORKLOADS["ctx94k-b8"] if R == 1 else WORKLOADS["mtp-ctx256k-b32"]
    wl = dataclasses.replace(base, batch=3, ctx=64 * 300, steps=4, layers=1)
    acc = np_(acceptances(wl)) if R > 1 else None
    qp = np_(positions(wl, torch.as_tensor(acc) if acc is not None else None))
    outs = {}
    side = torch.cuda.Stream(device=DEV)
    for mode in ("separate", "one stream", "two streams"):
        print("[case] tail", mode, "R", R, flush=True)
        spin_, pool, cfg, st, bufs, _ = bench._setup(wl, DEV)
        outs[mode] = []
        for t in range(wl.steps):
            keep = 10000 if t == 0 else 5000
            bufs["qpos"].copy_(torch.as_tensor(qp[t].astype(np.int32), device=DEV))
            q, w = make_queries(wl, pool, 0, t, qp[t].tolist(), device=DEV)
            a_dev = (torch.as_tensor(acc[t].astype(np.int32), device=DEV) if acc is not None
                     else None)
            spin.spin_predict_blocks(st.handle, 0, bufs["batch"], keep, bufs["kept"], bufs["cnt"],
                                     bufs["flags"])
            spin.spin_quantize_q(st.handle, bufs["batch"], q, w)
            spin.spin_indexer_scores(st.handle, bufs["batch"], pool.key_codes, pool.key_scale,
                                     pool.block_table, bufs["kept"], bufs["cnt"], bufs["scores"],
                                     bufs["pq"])
            if mode == "separate":
                spin.spin_topk_scores(bufs["batch"], cfg.topk, bufs["scores"], bufs["kept"],
                                      bufs["cnt"], bufs["topk"], bufs["topk_ws"], bufs["pq"])
                if a_dev is None:
                    spin.spin_update(st.handle, 0, bufs["batch"], bufs["scores"], bufs["kept"],
                                     bufs["cnt"])
                else:
                    spin.spin_mtp_replay(st.handle, 0, bufs["batch"], a_dev, bufs["scores"],
                                         bufs["kept"], bufs["cnt"])
            else:
                spin.spin_topk_update(st.handle, 0, bufs["batch"], bufs["scores"], bufs["pq"],
                                      bufs["kept"], bufs["cnt"], bufs["topk"], a_dev,
                                      update_stream=side if mode == "two streams" else None)
            torch.cuda.synchronize()
            outs[mode].append((np_(bufs["topk"]).copy(), np_(st.V()).copy(), np_(st.D()).copy(),
                               np_(st.VB()).copy(), np_(st.step()).copy()))
        assert st.error() == 0
        if mode == "two streams":
            # every gated top-k workgroup was counted: B * R per round
            gate = int(st.region("tail_gate", torch.int64, (1,)).item())
            assert gate == wl.steps * wl.batch * R
    for mode in ("one stream", "two streams"):
        for t, (x, y) in enumerate(zip(outs["separate"], outs[mode])):
            for i, name in enumerate(("topk", "V", "D", "VB", "step")):
                assert np.array_equal(x[i], y[i]), (R, mode, t, name)
