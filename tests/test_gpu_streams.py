"""The benchmark's overlapped round (quantiser beside the predictor, EMA update
beside the top-k on a second stream, a spin before the update) against the same
calls issued one after another on one stream: every output and the whole
state must be bit-identical, round after round.  A missing dependency between
the two streams would show up here as a difference."""
import dataclasses

import numpy as np
import pytest
import torch

import bench
import predictive_kv_block_amd as spin
from tests.spin_harness import np_
from workload import WORKLOADS, make_queries, positions

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


def _snapshot(st, b):
    n = np_(b["cnt"]).copy()
    return dict(kept=np_(b["kept"]).copy(), cnt=n, flags=np_(b["flags"]).copy(),
                scores=np_(b["scores"]).copy(), pq=np_(b["pq"]).copy(),
                topk=np_(b["topk"]).copy(), V=np_(st.V()).copy(), D=np_(st.D()).copy(),
                VB=np_(st.VB()).copy(), step=np_(st.step()).copy())


def _masked_scores(s, cnt):
    """Scores past each request's kept count are never written: blank them."""
    out = s.copy()
    for b, c in enumerate(cnt):
        out[b, :, int(c) * 64:] = 0.0
    return out


def test_overlapped_round_equals_serial(gpu_lib):
    wl = dataclasses.replace(WORKLOADS["ctx94k-b8"], steps=6)
    qp = np_(positions(wl))
    runs = []
    for mode in ("serial", "overlapped"):
        print("[case] stream plan", mode, flush=True)
        spin_, pool, cfg, st, bufs, _ = bench._setup(wl, DEV)
        side = torch.cuda.Stream(device=DEV)
        bench.SPACER_CYCLES = 4000
        done = None
        snaps = []
        for t in range(wl.steps):
            keep = 10000 if t == 0 else 5000
            bufs["qpos"].copy_(torch.as_tensor(qp[t].astype(np.int32), device=DEV))
            qb, w = make_queries(wl, pool, 0, t, qp[t].tolist(), device=DEV)
            if mode == "serial":
                _serial_round(st, bufs, pool, qb, w, keep)
            else:
                done = bench._round(spin, st, bufs, pool, qb, w, keep, side, done)
            torch.cuda.synchronize()
            snaps.append(_snapshot(st, bufs))
        assert st.error() == 0
        runs.append(snaps)
        bench.SPACER_CYCLES = 0
    for t, (a, b) in enumerate(zip(*runs)):
        assert np.array_equal(a["cnt"], b["cnt"]), t
        for k in ("kept", "flags", "topk", "V", "D", "VB", "step"):
            assert np.array_equal(a[k], b[k]), (t, k)
        assert np.array_equal(_masked_scores(a["scores"], a["cnt"]),
                              _masked_scores(b["scores"], b["cnt"])), (t, "scores")
        for bi, c in enumerate(a["cnt"]):
            assert np.array_equal(a["pq"][bi, :, : int(c)], b["pq"][bi, :, : int(c)]), (t, "pq")
