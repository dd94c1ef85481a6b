"""SPIN decode-round benchmark on one MI355X.

One step = one whole SPIN round for one layer over the batch: predict blocks
(z = max(V, D), block max-pool, budget + Philox exploration), quantise the
queries, run the fp8 gather-indexer on the kept pages, take the per-row
top-k, and update the EMAs from the observed slots.  The default workload is
the serving-shaped round: batch 96, 524288-token context (8192 pages of 64 per
request) in a shuffled paged fp8 pool, 64 indexer heads x 128, top-k 2048, at
50% target block sparsity with 5% exploration.

Prints one JSON line.  `value` = indexer-scored KV tokens per second over the
whole step (kept pages x 64 tokens / step time), inputs resident in HBM.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_DENSE_PEAK_TFLOPS = 5000.0 # MI355X dense fp8 MFMA
BF16_DENSE_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20         # MI355X Infinity Cache (last-level, memory side)
PAGE_BYTES = 64 * 128          # fp8 keys of one 64-token page
# Algorithmic bytes the indexer kernel moves per kept page and row: the page's
# keys, its scale, its block-table entry, its kept-list entry, 64 fp32 scores
# and the page's four quarter maxima per row.
IDX_BYTES_PER_PAGE = PAGE_BYTES + 4 + 4 + 4
IDX_SCORE_BYTES_PER_PAGE_ROW = 64 * 4 + 16      # scores + the page's quarter maxima


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_indexer_ctx512k-b96_hbm_traffic.md")
INDEXER_BUILD_FILES = ["predictive_kv_block_amd/csrc/spin_indexer.hip",
                       "predictive_kv_block_amd/csrc/spin_device.h",
                       "predictive_kv_block_amd/csrc/spin_internal.h"]


def indexer_build_digest():
    """SHA-256 over what the indexer kernel is compiled from: its source, the
    headers it includes from the package, and the compiler flags."""
    import hashlib

    from predictive_kv_block_amd.build import FLAGS

    h = hashlib.sha256()
    for f in INDEXER_BUILD_FILES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(a for a in FLAGS if not a.startswith("/")).encode())
    return h.hexdigest()


def _measured_traffic(workload, sparsity_bp):
    """HBM bytes per indexer launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, or None when that summary is for another workload or
    the indexer has been rebuilt from different sources since."""
    import re

    if workload != "ctx512k-b96" or sparsity_bp != 5000 or not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    t = re.search(r"^traffic_bytes_per_launch = (\d+)$", text, re.M)
    d = re.search(r"^indexer_build_sha256 = ([0-9a-f]{64})$", text, re.M)
    if not t or not d:
        return None
    return int(t.group(1)) if indexer_build_digest() == d.group(1) else None


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ctx512k-b96")
    ap.add_argument("--sparsity-bp", type=int, default=5000)
    ap.add_argument("--sweep", default="0,4000", help="extra sparsities (bp) timed for scaling")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-requests", type=int, default=64)
    ap.add_argument("--pools", type=int, default=1,
                    help="independently drawn key pools, round t reading pool t mod N, so that "
                         "a small workload's keys do not stay in the 256 MB Infinity Cache")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter scaling)")
    ap.add_argument("--fidelity", choices=("ablation", "budgets", "predictors"), default=None,
                    help="selection-fidelity run instead of the timing: MTP mask/update "
                         "policies over target sparsities, per-layer budgets, or slot "
                         "predictor quality (Pearson, top-k recall)")
    ap.add_argument("--fid-targets", default=",".join(str(t) for t in FID_TARGETS))
    ap.add_argument("--ceilings", action="store_true",
                    help="measure the HBM rates of a streaming read, a copy and a page gather")
    ap.add_argument("--attention", action="store_true",
                    help="time the sparse core attention over a real round's top-k instead")
    return ap.parse_args()


def _setup(wl, device):
    import torch

    import predictive_kv_block_amd as spin
    from workload import make_pool, make_queries

    spin.load()
    pool = make_pool(wl, 0, device=device)
    B, nb = wl.batch, wl.blocks
    cfg = spin.make_config(1, B, wl.ctx, wl.topk, max_rows=wl.rows, explore_bp=wl.explore_bp,
                           alpha=wl.alpha)
    st = spin.SpinState(cfg, device=device)
    slot = torch.arange(B, dtype=torch.int32, device=device)
    spin.spin_reset_slots(st.handle, slot, torch.arange(B, dtype=torch.int64, device=device) + 1000)
    qpos = torch.zeros(B, dtype=torch.int32, device=device)

    def outputs():
        return dict(kept=torch.zeros(B, nb, dtype=torch.int32, device=device),
                    cnt=torch.zeros(B, dtype=torch.int32, device=device),
                    flags=torch.zeros(B, nb, dtype=torch.uint8, device=device),
                    scores=torch.empty(B, wl.rows, nb * 64, dtype=torch.float32, device=device),
                    pq=torch.empty(B, wl.rows, nb, 4, dtype=torch.float32, device=device),
                    topk=torch.empty(B, wl.rows, wl.topk, dtype=torch.int32, device=device))

    # two sets of round outputs: round t writes set t % 2 while round t - 1's
    # top-k and update may still read the other (set 0 also under the plain keys)
    sets = [outputs(), outputs()]
    bufs = dict(slot=slot, qpos=qpos, batch=spin.make_batch(slot, qpos, wl.rows, nb), sets=sets,
                **sets[0])
    bufs["topk_ws"] = torch.empty(max(256, spin.spin_topk_workspace_bytes(bufs["batch"], wl.topk)),
                                  dtype=torch.uint8, device=device)
    return spin, pool, cfg, st, bufs, make_queries


def _round(spin, st, bufs, pool, batch, q, w, keep_bp, streams, t, ev=None, accepted=None,
           tail="beside", start=True):
    """Round t of a run, enqueued without host waits; returns its output set.

    The round's chain (quantise, predict, indexer, top-k, EMA update, then the
    next round's chain) runs without a wait between streams: a wait, like any
    event, is a packet between two kernels, and costs the chain several µs
    where consecutive kernels follow each other directly.  Round t writes
    output set t % 2 (kept list, counts, flags, scores, quarter maxima,
    top-k), so it needs nothing from round t - 1 but the state, and reads its
    positions through its own `batch` (a spin_batch over that round's row of
    positions, written before the run).
    tail="beside": the two streams take turns.  Round t's chain up to the
    top-k runs on streams[t % 2]; its update runs on the other stream beside
    the top-k, behind the library's gate (spin_topk_update: it opens once
    every top-k workgroup has started), and round t + 1's chain follows that
    update on its stream.
    tail="behind": everything on streams[0], the update after the top-k.
    `ev` = 8 timing events (0 at the start, 5-6 around the quantiser, 1 after
    the predictor, 2-3 around the indexer, 4 after the top-k, 7 after the
    update), or None; `start` = False leaves event 0 to the caller (the
    previous round's event 7 marks the same point).  `accepted` (int32 [B],
    device): MTP acceptances, whose prefix-valid replay replaces the
    single-row update.
    """
    beside = tail == "beside"
    main = streams[t % 2] if beside else streams[0]
    side = streams[(t + 1) % 2] if beside else main
    ev = ev or [None] * 8
    rec = lambda e, s: e.record(s) if e is not None else None
    o = bufs["sets"][t % 2]
    if start:
        rec(ev[0], main)
    rec(ev[5], main)
    spin.spin_quantize_q(st.handle, batch, q, w, stream=main)
    rec(ev[6], main)
    spin.spin_predict_blocks(st.handle, 0, batch, keep_bp, o["kept"], o["cnt"], o["flags"],
                             stream=main)
    rec(ev[1], main)
    rec(ev[2], main)
    spin.spin_indexer_scores(st.handle, batch, pool.key_codes, pool.key_scale, pool.block_table,
                             o["kept"], o["cnt"], o["scores"], o["pq"], stream=main)
    rec(ev[3], main)
    if beside:
        spin.spin_topk_update(st.handle, 0, batch, o["scores"], o["pq"], o["kept"], o["cnt"],
                              o["topk"], accepted, stream=main, update_stream=side)
        rec(ev[4], main)
    else:
        spin.spin_topk_scores(batch, st.cfg.topk, o["scores"], o["kept"], o["cnt"], o["topk"],
                              None, o["pq"], stream=main)
        rec(ev[4], main)
        if accepted is None:
            spin.spin_update(st.handle, 0, batch, o["scores"], o["kept"], o["cnt"], stream=main)
        else:
            spin.spin_mtp_replay(st.handle, 0, batch, accepted, o["scores"], o["kept"], o["cnt"],
                                 stream=main)
    rec(ev[7], side)
    return o


# timing passes: (name, tail, events recorded per round)
PASSES = (("plain", "beside", ()), ("lean", "beside", (0, 4, 7)),
          ("behind", "behind", (0, 4, 7)), ("detailed", "beside", tuple(range(8))))


def _run_gpu(wl, keep_bps, steps, warmup, device, n_pools=1):
    """Per keep and per timing pass of PASSES, `warmup` untimed rounds then
    `steps` timed rounds, all from the same state reset and inputs:
      plain     the round with the update beside the top-k on a second
                stream, behind the library's gate, the streams taking turns,
                with no event inside the timed rounds (an event between two
                kernels delays the second): value and ms_per_step, from the
                wall clock.
      lean      the same round with 3 events per round (its start, the
                top-k's end, the update's end): the predict + index + top-k
                latency and the whole step.
      behind    the round on one stream, the update behind the top-k (3
                events): the same figures without the overlap.
      detailed  the lean round with events around every stage (8 per round):
                the stage times, the sweep's indexer times and the roofline.
    Before the first timed pass, untimed cycles of the run's rounds in the
    lean schedule (at least 100 ms of them) settle the part: the first pass
    after the inputs are drawn ran 1-10% slower than the same pass repeated.
    Returns {keep: {pass name: {...}}}."""
    import torch

    from workload import acceptances, make_pool, positions

    spin, pool, cfg, st, bufs, make_queries = _setup(wl, device)
    # pool i is drawn as layer i's pool would be: same pattern, its own keys
    pools = [pool] + [make_pool(wl, i, device=device) for i in range(1, n_pools)]
    T = warmup + steps
    if wl.rows == 1:
        qpos_all = (torch.arange(T, dtype=torch.int64) + (wl.ctx - T))[:, None].repeat(1, wl.batch)
        acc_all = None
    else:
        # MTP: each request advances by its accepted drafts + 1 per round, and
        # the round's EMA update is the prefix-valid replay of those rows
        if T > wl.steps:
            raise SystemExit(f"{wl.name} has {wl.steps} rounds; asked for {T}")
        acc = acceptances(wl)
        qpos_all = positions(wl, acc)[:T]
        acc_all = acc[:T].to(torch.int32).to(device)
    qs = [make_queries(wl, pools[t % n_pools], 0, t, qpos_all[t].tolist(), device=device)
          for t in range(T)]
    qpos_all = qpos_all.to(torch.int32).to(device).contiguous()
    # one batch per round, over that round's row of positions
    batches = [spin.make_batch(bufs["slot"], qpos_all[t], wl.rows, wl.blocks) for t in range(T)]
    torch.cuda.synchronize()
    results = {}
    streams = (torch.cuda.Stream(device=device), torch.cuda.Stream(device=device))  # default priority
    acc_of = (lambda t: acc_all[t]) if acc_all is not None else (lambda t: None)
    spin.spin_reset_slots(st.handle, bufs["slot"],
                          torch.arange(wl.batch, dtype=torch.int64, device=device) + 1000)
    torch.cuda.synchronize()
    # untimed: settles the part before the first pass (cycles of the run's
    # rounds for at least 100 ms)
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < 0.1:
        for t in range(T):
            _round(spin, st, bufs, pools[t % n_pools], batches[t], qs[t][0], qs[t][1],
                   keep_bps[0], streams, t, accepted=acc_of(t), tail=PASSES[0][1])
        torch.cuda.synchronize()
    for keep_bp in keep_bps:
        results[keep_bp] = {}
        for name, tail, recorded in PASSES:
            spin.spin_reset_slots(st.handle, bufs["slot"],
                                  torch.arange(wl.batch, dtype=torch.int64, device=device) + 1000)
            torch.cuda.synchronize()
            for t in range(warmup):
                _round(spin, st, bufs, pools[t % n_pools], batches[t], qs[t][0], qs[t][1], keep_bp,
                       streams, t, accepted=acc_of(t), tail=tail)
            torch.cuda.synchronize()
            evs = []
            for i in range(steps):
                e = [None] * 8
                for k in recorded:
                    e[k] = torch.cuda.Event(enable_timing=True)
                if i > 0 and recorded:
                    e[0] = evs[-1][7]     # the previous update's end starts this round
                evs.append(e)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                t = warmup + i
                q, w = qs[t]
                last = _round(spin, st, bufs, pools[t % n_pools], batches[t], q, w, keep_bp,
                              streams, t, evs[i], accepted=acc_of(t), tail=tail, start=i == 0)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            per = {"step": [e[0].elapsed_time(e[7]) * 1e3 for e in evs]} if recorded else {}
            if 4 in recorded:
                # critical path to the top-k: quantise, predict, indexer, top-k
                per["to_topk"] = [e[0].elapsed_time(e[4]) * 1e3 for e in evs]
            if 4 in recorded:
                # a round ends when both the top-k and the update are done
                per["step"] = [max(e[0].elapsed_time(e[4]), e[0].elapsed_time(e[7])) * 1e3
                               for e in evs]
            if name == "detailed":
                per["quantize"] = [e[5].elapsed_time(e[6]) * 1e3 for e in evs]
                per["predict"] = [e[6].elapsed_time(e[1]) * 1e3 for e in evs]
                per["indexer"] = [e[2].elapsed_time(e[3]) * 1e3 for e in evs]
                per["topk"] = [e[3].elapsed_time(e[4]) * 1e3 for e in evs]
                # the update: from the top-k's end (behind it) or the indexer's
                # end (beside it) to its own
                u0 = 4 if tail == "behind" else 3
                per["update"] = [e[u0].elapsed_time(e[7]) * 1e3 for e in evs]
            kept_pages = int(last["cnt"].sum().item())
            if st.error() != 0:
                raise RuntimeError(f"device error word {st.error()}")
            results[keep_bp][name] = dict(wall_s=wall, per_us=per, kept_pages=kept_pages,
                                          blocks=wl.batch * wl.blocks)
    return results


def _median(x):
    s = sorted(x)
    return s[len(s) // 2]


def _pct(x, p):
    """p-th percentile (nearest rank) of a list."""
    s = sorted(x)
    return s[min(len(s) - 1, max(0, int(round(p / 100.0 * (len(s) - 1)))))]


def _cpu_worker(args):
    """One oracle process of the CPU baseline: `n` request-rounds of a
    one-request slice of the workload (same shapes), single-threaded BLAS."""
    wl_name, keep_bp, first, n = args
    import numpy as np

    from oracle import spin_oracle as O
    from workload import WORKLOADS, make_pool, make_queries, random_state
    import dataclasses
    wl = WORKLOADS[wl_name]
    wl1 = dataclasses.replace(wl, batch=1)
    pool = make_pool(wl1, 0, device="cpu")
    kv = O.e4m3fn_decode(pool.key_codes.numpy())
    scv = pool.key_scale.numpy().astype(np.float64)
    table = pool.block_table[0].numpy()
    q = wl.ctx - wl.rows
    qb, w = make_queries(wl1, pool, 0, 5, [q], device="cpu")
    qv, wv, _, _ = O.fp8_query_operands(qb[0].float().numpy(), w[0].numpy())
    tokens = 0
    elapsed = 0.0
    for r in range(first, first + n):
        st = O.RequestState(wl.ctx, request_id=1000 + r)
        st.V[:] = random_state(wl.ctx, 0.0, seed=r).double().numpy()
        st.D[:] = random_state(wl.ctx, 0.0, seed=r + 77).double().numpy()
        st.step = 5
        t0 = time.perf_counter()
        out = O.decode_round(st, q, wl.rows, keep_bp, wl.explore_bp, 0x5350494E, 0, qv, wv, kv, scv,
                             table, wl.topk, wl.alpha)
        elapsed += time.perf_counter() - t0
        tokens += len(out["kept"]) * 64
    return tokens, elapsed


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baseline(wl, keep_bp, n_req, max_procs=16):
    """Time the oracle on a bounded sample of the workload: n_req
    request-rounds spread over one single-threaded oracle process per core of
    this process's CPU share (at most max_procs, the share a one-GPU job
    gets).  Each process times only its decode rounds; the rate is the total
    kept tokens over the longest process's timed seconds."""
    import multiprocessing as mp

    visible = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    procs = max(1, min(visible, max_procs, n_req))
    per = [n_req // procs + (1 if i < n_req % procs else 0) for i in range(procs)]
    jobs, first = [], 0
    for n in per:
        jobs.append((wl.name, keep_bp, first, n))
        first += n
    env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in env:
        os.environ[k] = "1"                 # inherited by the spawned oracle processes
    try:
        # spawned interpreters (not forks of this process, which may hold the GPU)
        with mp.get_context("spawn").Pool(procs) as pool:
            res = pool.map(_cpu_worker, jobs)
    finally:
        for k, v in env.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    tokens = sum(t for t, _ in res)
    slowest = max(e for _, e in res)
    cpu_s = sum(e for _, e in res)
    return {"value": tokens / slowest, "unit": "tokens/s", "cores": procs, "kind": "oracle",
            "sample": (f"{n_req} requests x 1 round of {wl.name} at {keep_bp} bp keep over "
                       f"{procs} single-threaded oracle processes ({tokens} kept tokens, "
                       f"{cpu_s:.1f} CPU-s, slowest process {slowest:.1f} s): predict + fp64 "
                       f"indexer + top-k + EMA update"),
            "s_per_request_round": cpu_s / n_req, "nproc": os.cpu_count(), "cpus_visible": visible,
            "cpu_model": _cpu_model()}


# ------------------------------------------------------------ selection fidelity
# Mean / p99 miss over eligible rows (v1, Table 5 caption) for the MTP policies
# of v1 Figure 2 and Table 7, and the per-layer budgets of the v3 abstract.
# Every round of every layer runs a shadow all-keep indexer + top-k beside the
# sparse round; spin_measure_miss compares that top-k with the round's block
# flags.  All R verification rows of a round count as decode rows.

FID_TARGETS = (2000, 3000, 4000, 5000)
FID_POLICIES = (("union", "prefix"), ("union", "row0"), ("row0", "prefix"), ("row0", "row0"))


def _fidelity_inputs(wl, device):
    """Per-layer pools, acceptances, positions and every round's queries."""
    from workload import acceptances, make_pool, make_queries, positions

    pools = [make_pool(wl, l, device=device) for l in range(wl.layers)]
    acc = acceptances(wl)
    qpos = positions(wl, acc)
    qs = [[make_queries(wl, pools[l], l, t, qpos[t].tolist(), device=device)
           for t in range(wl.steps)] for l in range(wl.layers)]
    return pools, acc, qpos, qs


def _fidelity_trace(wl, inputs, device, mask, update, keep_of, rounds=None):
    """Run `rounds` MTP rounds over every layer under one policy.

    mask: "union" (row-local union) or "row0" (row 0's mask for every row);
    update: "prefix" (prefix-valid replay) or "row0" (row 0's scores only).
    keep_of(t, layer, miss_so_far, est_so_far) -> keep_bp of that layer in
    round t, given the measured miss [t, L, B, R] and the online estimates
    [t, L, B, R, 2] of the earlier rounds.
    Returns miss [T, L, B, R], kept block counts [T, L, B], the keep_bp used
    [T, L], and the online estimates [T, L, B, R, 2] of each row's miss from
    its exploration blocks and the sparse round's own top-k
    (spin_estimate_miss: the weighted-threshold estimate and the hit-ratio
    upper bound; -1 where nothing was explored).
    """
    import numpy as np
    import torch

    import predictive_kv_block_amd as spin

    pools, acc, qpos_all, qs = inputs
    T = rounds or wl.steps
    L, B, R, nb, K = wl.layers, wl.batch, wl.rows, wl.blocks, wl.topk
    policy = spin.SPIN_MASK_ROW0 if mask == "row0" else 0
    cfg = spin.make_config(L, B, wl.ctx, K, max_rows=R, explore_bp=wl.explore_bp,
                           alpha=wl.alpha, policy=policy)
    st = spin.SpinState(cfg, device=device)
    slot = torch.arange(B, dtype=torch.int32, device=device)
    spin.spin_reset_slots(st.handle, slot, torch.arange(B, dtype=torch.int64, device=device) + 1000)
    qpos = torch.zeros(B, dtype=torch.int32, device=device)
    batch = spin.make_batch(slot, qpos, R, nb)
    i32 = dict(dtype=torch.int32, device=device)
    kept, cnt = torch.zeros(B, nb, **i32), torch.zeros(B, **i32)
    flags = torch.zeros(B, nb, dtype=torch.uint8, device=device)
    scores = torch.empty(B, R, nb * 64, dtype=torch.float32, device=device)
    pq = torch.empty(B, R, nb, 4, dtype=torch.float32, device=device)
    kept_all = torch.arange(nb, **i32)[None, :].repeat(B, 1).contiguous()
    cnt_all = torch.zeros(B, **i32)
    scores_all = torch.empty_like(scores)
    pq_all = torch.empty_like(pq)
    topk_all = torch.empty(B, R, K, **i32)
    topk_sp = torch.empty(B, R, K, **i32)
    est_dev = torch.zeros(L, B, R, 2, dtype=torch.float32, device=device)
    miss_dev = torch.zeros(L, B, R, dtype=torch.float32, device=device)
    cnt_dev = torch.zeros(L, B, **i32)
    acc_dev = acc.to(torch.int32).to(device)
    miss = np.zeros((T, L, B, R), dtype=np.float32)
    est = np.zeros((T, L, B, R, 2), dtype=np.float32)
    kept_n = np.zeros((T, L, B), dtype=np.int64)
    keeps = np.zeros((T, L), dtype=np.int64)
    for t in range(T):
        qpos.copy_(qpos_all[t].to(torch.int32))
        cnt_all.copy_((qpos + (R - 1)) // 64 + 1)
        for l in range(L):
            keep = int(keep_of(t, l, miss[:t], est[:t]))
            keeps[t, l] = keep
            q, w = qs[l][t]
            pool = pools[l]
            spin.spin_predict_blocks(st.handle, l, batch, keep, kept, cnt, flags)
            spin.spin_quantize_q(st.handle, batch, q, w)
            spin.spin_indexer_scores(st.handle, batch, pool.key_codes, pool.key_scale,
                                     pool.block_table, kept_all, cnt_all, scores_all, pq_all)
            spin.spin_topk_scores(batch, K, scores_all, kept_all, cnt_all, topk_all, None, pq_all)
            spin.spin_measure_miss(batch, K, topk_all, flags, miss_dev[l])
            spin.spin_indexer_scores(st.handle, batch, pool.key_codes, pool.key_scale,
                                     pool.block_table, kept, cnt, scores, pq)
            spin.spin_topk_scores(batch, K, scores, kept, cnt, topk_sp, None, pq)
            spin.spin_estimate_miss(batch, K, scores, kept, cnt, topk_sp, flags, est_dev[l])
            if update == "prefix":
                spin.spin_mtp_replay(st.handle, l, batch, acc_dev[t], scores, kept, cnt)
            else:
                spin.spin_update(st.handle, l, batch, scores, kept, cnt)
            cnt_dev[l].copy_(cnt)
        miss[t] = miss_dev.cpu().numpy()
        est[t] = est_dev.cpu().numpy()
        kept_n[t] = cnt_dev.cpu().numpy()
    if st.error() != 0:
        raise RuntimeError(f"device error word {st.error()}")
    return miss, kept_n, keeps, est


def _fidelity_summary(miss, kept_n, keeps, qpos, rows, warmup, first_round=0, est=None):
    """Mean and p99 miss over eligible rows, and the realized block sparsity.

    A row (round t, layer l, request b, row r) is eligible when the round is
    past warm-up (t >= warmup) and sparse for that row (its kept budget
    ceil(keep * n / 10000) is below its block count n).  p99 is taken per
    (layer, request) over that trace's eligible rows (linear interpolation),
    then averaged, as in the pages' per-layer, per-trace p99; `p99_pooled` is
    the p99 of all eligible rows together.  Realized sparsity = 1 - kept
    blocks / blocks up to the round's last row, over the eligible rounds.
    With `est` (online estimates, -1 = none), the mean estimate over the
    eligible rows that have one is reported beside the measured mean miss,
    per layer and overall, with the rows' Pearson correlation to the miss.
    """
    import numpy as np

    miss = np.asarray(miss, dtype=np.float64)
    T, L, B, R = miss.shape
    qpos = np.asarray(qpos[:T], dtype=np.int64)                    # [T, B]
    n_row = (qpos[:, :, None] + np.arange(R)[None, None, :]) // 64 + 1   # [T, B, R]
    kb = (keeps[:, :, None, None] * n_row[:, None, :, :] + 9999) // 10000  # [T, L, B, R]
    t_ok = (np.arange(T) >= max(warmup, first_round))[:, None, None, None]
    elig = t_ok & (kb < n_row[:, None, :, :])
    per_trace = []
    per_layer = []
    for l in range(L):
        lm = []
        for b in range(B):
            x = miss[:, l, b, :][elig[:, l, b, :]]
            if len(x):
                per_trace.append(np.percentile(x, 99))
                lm.append(x)
        xl = np.concatenate(lm) if lm else np.zeros(0)
        rec = {"mean_miss": float(xl.mean()) if len(xl) else None,
               "p99_miss": float(np.mean([np.percentile(x, 99) for x in lm])) if lm else None}
        if est is not None:
            el = np.asarray(est, dtype=np.float64)[:, l][elig[:, l]]      # [rows, 2]
            el = el[el[:, 0] >= 0]
            rec["online_mean_miss"] = float(el[:, 0].mean()) if len(el) else None
            rec["online_upper_mean_miss"] = float(el[:, 1].mean()) if len(el) else None
        per_layer.append(rec)
    allx = miss[elig]
    rt = np.arange(T) >= max(warmup, first_round)
    n_last = n_row[:, :, R - 1]                                     # [T, B]
    tot = float(n_last[rt].sum()) * L
    online = {}
    if est is not None:
        e2 = np.asarray(est, dtype=np.float64)[elig]                      # [rows, 2]
        has = e2[:, 0] >= 0
        e, u, m = e2[has, 0], e2[has, 1], allx[has]
        corr = lambda a: (float(np.corrcoef(a, m)[0, 1])
                          if len(a) > 1 and a.std() > 0 and m.std() > 0 else None)
        online = {"online_mean_miss": float(e.mean()) if len(e) else None,
                  "online_upper_mean_miss": float(u.mean()) if len(u) else None,
                  "online_rows_without_estimate": int((~has).sum()),
                  "online_row_pearson": corr(e), "online_upper_row_pearson": corr(u)}
    return {**online, "eligible_rows": int(elig.sum()),
            "mean_miss": float(allx.mean()) if len(allx) else None,
            "p99_miss": float(np.mean(per_trace)) if per_trace else None,
            "p99_pooled": float(np.percentile(allx, 99)) if len(allx) else None,
            "realized_sparsity": 1.0 - float(kept_n[rt].sum()) / tot if tot else None,
            "per_layer": per_layer}


def _fidelity_predictors(wl, device, keeps):
    """Table 1 of the v1 listing on a single-row workload: Pearson correlation
    and top-k recall of slot predictors against the all-keep indexer, averaged
    over requests and rounds 1..T-1.

    Predictors: SPIN's z = max(V, D) from the state before the round (the
    state itself runs SPIN rounds at each keep in `keeps`, observing only the
    kept slots), prev-iter (the previous round's all-keep scores; the new
    slots have none), and random (uniform values; expected recall K / N).
    """
    import numpy as np
    import torch

    import predictive_kv_block_amd as spin
    from workload import make_pool, make_queries, positions

    pool = make_pool(wl, 0, device=device)
    B, nb, K, T = wl.batch, wl.blocks, wl.topk, wl.steps
    qpos_all = positions(wl)
    qs = [make_queries(wl, pool, 0, t, qpos_all[t].tolist(), device=device) for t in range(T)]
    i32 = dict(dtype=torch.int32, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    slot = torch.arange(B, **i32)
    qpos = torch.zeros(B, **i32)
    batch = spin.make_batch(slot, qpos, 1, nb)
    kept, cnt = torch.zeros(B, nb, **i32), torch.zeros(B, **i32)
    flags = torch.zeros(B, nb, dtype=torch.uint8, device=device)
    scores, actual = torch.empty(B, 1, nb * 64, **f32), torch.empty(B, 1, nb * 64, **f32)
    pq, pq_all = torch.empty(B, 1, nb, 4, **f32), torch.empty(B, 1, nb, 4, **f32)
    kept_all = torch.arange(nb, **i32)[None, :].repeat(B, 1).contiguous()
    cnt_all = torch.zeros(B, **i32)
    z, prev, rnd = (torch.empty(B, 1, nb * 64, **f32) for _ in range(3))
    ta, tp = torch.empty(B, 1, K, **i32), torch.empty(B, 1, K, **i32)
    ws = torch.empty(max(256, spin.spin_topk_workspace_bytes(batch, K)), dtype=torch.uint8,
                     device=device)
    out = torch.empty(B, 1, 2, dtype=torch.float64, device=device)
    slots = torch.arange(nb * 64, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed + 17)
    res = []
    for keep in keeps:
        cfg = spin.make_config(1, B, wl.ctx, K, explore_bp=wl.explore_bp, alpha=wl.alpha)
        st = spin.SpinState(cfg, device=device)
        spin.spin_reset_slots(st.handle, slot, torch.arange(B, dtype=torch.int64,
                                                            device=device) + 1000)
        sums = {n: np.zeros(2) for n in ("spin", "prev_iter", "random")}
        rows = 0
        n_tok = 0
        for t in range(T):
            qpos.copy_(qpos_all[t].to(torch.int32))
            cnt_all.copy_(qpos // 64 + 1)
            q, w = qs[t]
            spin.spin_slot_scores(st.handle, 0, batch, z)
            spin.spin_predict_blocks(st.handle, 0, batch, keep, kept, cnt, flags)
            spin.spin_quantize_q(st.handle, batch, q, w)
            spin.spin_indexer_scores(st.handle, batch, pool.key_codes, pool.key_scale,
                                     pool.block_table, kept_all, cnt_all, actual, pq_all)
            spin.spin_topk_scores(batch, K, actual, kept_all, cnt_all, ta, None, pq_all)
            spin.spin_indexer_scores(st.handle, batch, pool.key_codes, pool.key_scale,
                                     pool.block_table, kept, cnt, scores, pq)
            spin.spin_update(st.handle, 0, batch, scores, kept, cnt)
            if t >= 1:
                torch.rand(B, 1, nb * 64, generator=gen, device=device, out=rnd)
                for name, p in (("spin", z), ("prev_iter", prev), ("random", rnd)):
                    spin.spin_topk_scores(batch, K, p, kept_all, cnt_all, tp, ws)
                    spin.spin_predictor_fidelity(batch, K, p, actual, tp, ta, out)
                    sums[name] += out[:, 0, :].sum(dim=0).cpu().numpy()
                rows += B
                n_tok += int((qpos + 1).sum())
            # prev-iter for the next round: these scores, none for later slots
            torch.where(slots[None, None, :] <= qpos[:, None, None].long(), actual,
                        torch.full_like(actual, float("-inf")), out=prev)
        if st.error() != 0:
            raise RuntimeError(f"device error word {st.error()}")
        rec = {"fidelity": "predictors", "workload": wl.name, "keep_bp": keep,
               "rounds": T - 1, "rows": rows, "topk": K, "k_over_n": K * rows / n_tok}
        for name, v in sums.items():
            rec[name] = {"pearson": float(v[0] / rows), "topk_recall": float(v[1] / rows)}
        print(json.dumps(rec), flush=True)
        res.append(rec)
    return res


def _fidelity(mode, wl, device, targets):
    import numpy as np

    import predictive_kv_block_amd as spin

    spin.load()
    if mode == "predictors":
        return _fidelity_predictors(wl, device, [10000 - t for t in targets])
    t0 = time.perf_counter()
    inputs = _fidelity_inputs(wl, device)
    qpos = inputs[2].numpy()
    print(f"[fidelity] {wl.name}: inputs drawn in {time.perf_counter() - t0:.1f} s",
          file=sys.stderr, flush=True)
    warm = 1                                   # the config's warm-up rounds
    out = []
    if mode == "ablation":
        for tgt in targets:
            for mask, upd in FID_POLICIES:
                miss, kept_n, keeps, est = _fidelity_trace(wl, inputs, device, mask, upd,
                                                           lambda t, l, m, e, k=10000 - tgt: k)
                s = _fidelity_summary(miss, kept_n, keeps, qpos, wl.rows, warm, est=est)
                rec = {"fidelity": "mtp_policy", "workload": wl.name, "target_sparsity_bp": tgt,
                       "mask": mask, "update": upd, **s}
                print(json.dumps(rec), flush=True)
                out.append(rec)
        return out
    # per-layer budgets: W calibration rounds at the uniform mean keep, then
    # spin_allocate_budgets from each layer's mean miss over those rounds,
    # measured with the shadow all-keep indexer or estimated online from the
    # exploration blocks alone
    W = 8
    mean_keep = 10000 - targets[-1]
    uni = _fidelity_trace(wl, inputs, device, "union", "prefix", lambda t, l, m, e: mean_keep)
    runs = [("uniform", uni, None)]
    for source in ("shadow", "online"):
        plan = {}

        def keep_of(t, l, m, e, plan=plan, source=source):
            if t < W:
                return mean_keep
            if "keep" not in plan:
                if source == "online":
                    m = np.where(e[..., 0] >= 0, e[..., 0], 0.0)
                s = _fidelity_summary(m, np.ones((t, wl.layers, wl.batch)),
                                      np.full((t, wl.layers), mean_keep), qpos, wl.rows, warm)
                plan["calib_miss"] = [p["mean_miss"] for p in s["per_layer"]]
                plan["keep"] = spin.spin_allocate_budgets(plan["calib_miss"], mean_keep)
            return plan["keep"][l]

        runs.append((f"per_layer_{source}",
                     _fidelity_trace(wl, inputs, device, "union", "prefix", keep_of), plan))
    # the same v3 passage read through each layer's miss curve: W calibration
    # rounds at every keep of a grid (each grid keep on its own fresh state, the
    # mean's from the uniform run), then spin_allocate_budgets_curve
    step = max(mean_keep // 4, 1)
    grid = sorted({min(10000, mean_keep // 2 + i * step) for i in range(10000 // step + 3)})
    curve = np.zeros((wl.layers, len(grid)))
    for gi, g in enumerate(grid):
        if g == 10000:
            continue                  # every block kept: nothing can be missed
        m = uni[0][:W] if g == mean_keep else _fidelity_trace(
            wl, inputs, device, "union", "prefix", lambda t, l, m, e, g=g: g, rounds=W)[0]
        s = _fidelity_summary(m, np.ones((W, wl.layers, wl.batch)), np.full((W, wl.layers), g),
                              qpos, wl.rows, warm)
        curve[:, gi] = [p["mean_miss"] or 0.0 for p in s["per_layer"]]
        print(f"[fidelity] calibration at keep {g}: per-layer mean miss "
              f"{[round(float(x), 4) for x in curve[:, gi]]}", file=sys.stderr, flush=True)
    cplan = {"calib_grid_bp": grid, "calib_miss_curve": curve.tolist(),
             "keep": spin.spin_allocate_budgets_curve(curve.tolist(), grid, mean_keep)}
    runs.append(("per_layer_curve", _fidelity_trace(
        wl, inputs, device, "union", "prefix",
        lambda t, l, m, e: mean_keep if t < W else cplan["keep"][l]), cplan))
    for name, (miss, kept_n, keeps, est), plan in runs:
        s = _fidelity_summary(miss, kept_n, keeps, qpos, wl.rows, warm, first_round=W, est=est)
        rec = {"fidelity": "layer_budgets", "workload": wl.name, "mean_keep_bp": mean_keep,
               "calibration_rounds": W, "budgets": name,
               "keep_bp": [int(k) for k in keeps[-1]], **s}
        if plan and "calib_miss" in plan:
            rec["calibration_mean_miss"] = plan["calib_miss"]
        if plan and "calib_miss_curve" in plan:
            rec["calibration_grid_bp"] = plan["calib_grid_bp"]
            rec["calibration_miss_curve"] = plan["calib_miss_curve"]
        print(json.dumps(rec), flush=True)
        out.append(rec)
    return out


def _attention_bench(wl, device, steps, warmup, keep_bp):
    """Time the sparse core attention over the top-k of a real round.

    Two rounds (the all-keep warm-up, then one at keep_bp) produce each
    row's top-k from the indexer; a latent cache of the workload's full size
    (pool pages x 64 tokens x 576 bf16) and bf16 queries for 128 heads are
    drawn on the device; the attention over that top-k is then launched
    `steps` times between HIP events on the current stream.
    """
    import torch

    spin, pool, cfg, st, bufs, make_queries = _setup(wl, device)
    from workload import positions

    streams = (torch.cuda.Stream(device=device), torch.cuda.Stream(device=device))
    qp = positions(wl)[:2].to(device=device, dtype=torch.int32).contiguous()
    batches = [spin.make_batch(bufs["slot"], qp[t], wl.rows, wl.blocks) for t in range(2)]
    qws = [make_queries(wl, pool, 0, t, qp[t].tolist(), device=device) for t in range(2)]
    torch.cuda.synchronize()
    for t, keep in enumerate((10000, keep_bp)):
        out = _round(spin, st, bufs, pool, batches[t], qws[t][0], qws[t][1], keep, streams, t)
    batch, topk = batches[1], out["topk"]
    torch.cuda.synchronize()
    H, D, DV = 128, 576, 512
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed + 31)
    kv = torch.empty(wl.pool_pages, 64, D, dtype=torch.bfloat16, device=device)
    for i in range(0, wl.pool_pages, 8192):
        kv[i:i + 8192].copy_(torch.randn(min(8192, wl.pool_pages - i), 64, D, device=device,
                                         generator=g))
    qa = torch.randn(wl.batch, wl.rows, H, D, device=device, generator=g).to(torch.bfloat16)
    n = spin.spin_attention_workspace_bytes(batch, wl.topk)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    out = torch.empty(wl.batch, wl.rows, H, DV, dtype=torch.bfloat16, device=device)
    lse = torch.empty(wl.batch, wl.rows, H, device=device)
    scale = 1.0 / 192 ** 0.5
    args = (batch, wl.topk, topk, qa, kv, pool.block_table, scale, out, lse, ws)
    for _ in range(warmup):
        spin.spin_sparse_attention(*args)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        spin.spin_sparse_attention(*args)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    tok = int((topk >= 0).sum())
    rows = wl.batch * wl.rows
    byts = tok * D * 2 + rows * (H * D * 2 + H * DV * 2 + H * 4 + wl.topk * 4)
    flops = 2 * H * tok * (D + DV)
    return {"workload": wl.name, "rows": rows, "topk": wl.topk, "attended_tokens": tok,
            "us_per_launch": round(us, 2), "workspace_bytes": n,
            "algorithmic_bytes": byts, "flops": flops,
            "hbm": {"achieved_GBps": round(byts / us / 1e3, 1), "peak": HBM_PEAK_GBS,
                    "frac": round(byts / us / 1e3 / HBM_PEAK_GBS, 4)},
            "mfma_bf16": {"achieved_TFLOPs": round(flops / us / 1e6, 1),
                          "peak": BF16_DENSE_PEAK_TFLOPS,
                          "frac": round(flops / us / 1e6 / BF16_DENSE_PEAK_TFLOPS, 4)}}


def _ceilings(device, reps=10):
    """HBM rates this part reaches with plain torch kernels: streaming reads
    of 4 GiB (a sum, row sums, and a matrix-vector product), a device copy
    (2 GiB read + 2 GiB written), and a gather of random 8 KB pages into a
    fresh output (the indexer's read pattern, with a write stream beside
    it).  GB/s of bytes moved."""
    import torch

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    out = {}
    x = torch.ones(1 << 30, dtype=torch.float32, device=device)           # 4 GiB
    m = x.view(1 << 17, 1 << 13)
    v = torch.ones(1 << 13, dtype=torch.float32, device=device)
    reads = {"sum": lambda: x.sum(), "row_sums": lambda: m.sum(dim=1), "gemv": lambda: m @ v}
    out["read_GBps"] = {k: round(x.numel() * 4 / timed(f) / 1e9, 1) for k, f in reads.items()}
    del x, m, v
    a = torch.ones(1 << 29, dtype=torch.float32, device=device)           # 2 GiB
    b = torch.empty_like(a)
    out["copy_GBps"] = round(2 * a.numel() * 4 / timed(lambda: b.copy_(a)) / 1e9, 1)
    del a, b
    pages = torch.ones(786432, 2048, dtype=torch.float32, device=device)  # 6 GiB of 8 KB pages
    g = torch.Generator(device=device)
    g.manual_seed(7)
    idx = torch.randperm(pages.shape[0], generator=g, device=device)[:393216]
    t = timed(lambda: pages.index_select(0, idx))
    out["page_gather_GBps"] = round(2 * idx.numel() * 8192 / t / 1e9, 1)
    out["page_gather_read_GBps"] = round(idx.numel() * 8192 / t / 1e9, 1)
    return out


def _copy_calibration(device):
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def main():
    a = _args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the SPIN path shards by request with no exchange).", file=sys.stderr)
        sys.exit(2)
    import torch
    from workload import WORKLOADS

    wl = WORKLOADS[a.workload]
    device = "cuda:0"
    torch.cuda.set_device(0)
    if a.fidelity:
        _fidelity(a.fidelity, wl, device, [int(x) for x in a.fid_targets.split(",")])
        return
    if a.ceilings:
        print(json.dumps({"hbm_ceilings": _ceilings(device)}), flush=True)
        return
    if a.attention:
        print(json.dumps({"attention": _attention_bench(wl, device, a.steps, a.warmup,
                                                        10000 - a.sparsity_bp)}), flush=True)
        return
    keep_main = 10000 - a.sparsity_bp
    sweep = [10000 - int(s) for s in a.sweep.split(",") if s.strip() != ""]
    keeps = [keep_main] + [k for k in sweep if k != keep_main]
    if a.copy_calibration:
        _copy_calibration(device)
    both = _run_gpu(wl, keeps, a.steps, a.warmup, device, max(1, a.pools))
    res = {k: v["detailed"] for k, v in both.items()}    # per-stage times
    plain = both[keep_main]["plain"]                     # the round: wall clock only
    lean = both[keep_main]["lean"]                       # the round: latency, step
    beh = both[keep_main]["behind"]                      # the update behind the top-k

    main_r = res[keep_main]
    per = main_r["per_us"]
    step_us = lean["per_us"]["step"]
    pit = lean["per_us"]["to_topk"]
    ms_per_step = plain["wall_s"] * 1e3 / a.steps
    tokens_per_step = plain["kept_pages"] * 64
    value = tokens_per_step / (ms_per_step / 1e3)
    idx_us = sum(per["indexer"]) / a.steps
    idx_flops = main_r["kept_pages"] * 64 * wl.rows * wl.heads * wl.head_dim * 2
    idx_bytes = main_r["kept_pages"] * (IDX_BYTES_PER_PAGE + wl.rows * IDX_SCORE_BYTES_PER_PAGE_ROW)
    achieved = idx_bytes / (idx_us * 1e-6) / 1e9
    key_ws = max(1, a.pools) * wl.pool_pages * (64 * wl.head_dim + 4)
    sweep_out = {}
    for k, r in res.items():
        iu = sum(r["per_us"]["indexer"]) / a.steps
        sweep_out[str(10000 - k)] = {
            "kept_share": r["kept_pages"] / r["blocks"],
            "indexer_us": round(iu, 2),
            "step_us_median": round(_median(both[k]["lean"]["per_us"]["step"]), 2),
        }
    if "0" in sweep_out:
        base = sweep_out["0"]["indexer_us"]
        for s in sweep_out.values():
            s["indexer_time_ratio_vs_allkeep"] = round(s["indexer_us"] / base, 4)
    cpu = None
    if not a.no_cpu_baseline:
        cpu = _cpu_baseline(wl, keep_main, a.cpu_requests)
    out = {
        "metric": "indexer-scored KV tokens/s + per-step predict+index+topk us at 512K ctx, B=96",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 x fp8-e4m3 -> fp32 (indexer); fp32 (EMA)",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "ctx": wl.ctx, "pages_per_request": wl.blocks,
                   "heads": wl.heads, "head_dim": wl.head_dim, "topk": wl.topk,
                   "target_sparsity_bp": a.sparsity_bp, "explore_bp": wl.explore_bp,
                   "rows": wl.rows, "block_table": "shuffled" if wl.shuffle else "identity",
                   "key_pools": max(1, a.pools)},
        # the keys the indexer can touch over the run; at or under the 256 MB
        # Infinity Cache the indexer's figures are cache-resident, not HBM rates
        "key_working_set_bytes": key_ws,
        "cache_resident": key_ws <= MALL_BYTES,
        "indexer_tokens_per_s": tokens_per_step / (idx_us * 1e-6),
        "indexer_row_tokens_per_s": wl.rows * tokens_per_step / (idx_us * 1e-6),
        "indexer_roofline_tokens_per_s": HBM_PEAK_GBS * 1e9 / (
            IDX_BYTES_PER_PAGE / 64 + wl.rows * IDX_SCORE_BYTES_PER_PAGE_ROW / 64),
        "per_step_us": {
            # lean pass: the update beside the top-k, 3 events per round
            "lean_pass_ms_per_step": round(lean["wall_s"] * 1e3 / a.steps, 4),
            "predict_index_topk_median": round(_median(pit), 2),
            "predict_index_topk_p10": round(_pct(pit, 10), 2),
            "predict_index_topk_p90": round(_pct(pit, 90), 2),
            "whole_step_median": round(_median(step_us), 2),
            "update_median": round(_median(per["update"]), 2),
            **{f"{n}_mean": round(sum(v) / len(v), 2) for n, v in per.items()
               if n not in ("step", "to_topk")},
            "schedule": "two streams taking turns: quantise, predict, indexer and top-k on "
                        "one, the EMA update beside the top-k on the other behind the library's "
                        "gate (spin_topk_update), the next round's chain after that update on "
                        "its stream; two sets of round outputs, so that no round waits on "
                        "another stream",
            # the same rounds on one stream, the update behind the top-k
            "behind_pass": {
                "ms_per_step": round(beh["wall_s"] * 1e3 / a.steps, 4),
                "whole_step_median": round(_median(beh["per_us"]["step"]), 2),
                "predict_index_topk_median": round(_median(beh["per_us"]["to_topk"]), 2),
            },
            # every stage bracketed by events (8 per round): the stage means,
            # the sweep's indexer times and the roofline
            "detailed_pass": {
                "ms_per_step": round(main_r["wall_s"] * 1e3 / a.steps, 4),
                "predict_index_topk_median": round(_median(per["to_topk"]), 2),
                "whole_step_median": round(_median(per["step"]), 2),
            },
        },
        "realized_block_sparsity": 1.0 - main_r["kept_pages"] / main_r["blocks"],
        "roofline": {"bound": "hbm", "kernel": "k_indexer", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": _measured_traffic(wl.name, a.sparsity_bp),
                     "bytes_per_launch": idx_bytes},
        "indexer_mfma": {"dtype": "fp8 e4m3", "flops_per_launch": idx_flops,
                         "achieved_tflops": round(idx_flops / (idx_us * 1e-6) / 1e12, 1),
                         "peak_tflops": FP8_DENSE_PEAK_TFLOPS,
                         "frac": round(idx_flops / (idx_us * 1e-6) / 1e12 / FP8_DENSE_PEAK_TFLOPS, 4)},
        "sweep": sweep_out,
        "cpu_baseline": cpu,
        "context": "pages' serving run: 4720 -> 5421 output TPS (+14.9% at 50% sparsity, 8x B300, "
                   "TP8/EP8, end-to-end vLLM) -- another system, context only",
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
