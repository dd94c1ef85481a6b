"""Kernel-level parity of the HIP path against the oracle, through the C ABI.

Every input comes from the seeded generator (or plain numpy/torch draws in the
test); every expected value from oracle/.  Bars: q8 codes/exponents, masks,
counts, exploration and top-k over identical scores bit-exact; indexer scores
and EMA state within max(1e-3 |ref|, 1e-5 mag) (fp32 accumulation).
"""
import numpy as np
import pytest
import torch

import predictive_kv_block_amd as spin
from oracle import spin_oracle as O
from tests.spin_harness import (NEG, Rig, assert_scores_close, assert_topk_tie_aware,
                                nblocks, np_, oracle_fp8_operands, score_mag, score_tol)
from workload import random_state

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


# --------------------------------------------------------------- quantiser
def test_quantize_codes_and_exponents_bit_exact(gpu_lib):
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    vals = bits.view(torch.bfloat16)
    vals = vals[torch.isfinite(vals.float())]
    mag_order = torch.argsort(vals.float().abs())
    n_heads = 8 * 2 * 64
    need = n_heads * 128
    rng = np.random.default_rng(0)
    # layout 1: heads of similar magnitude (every value meets a nearby exponent);
    # layout 2: random heads (small values under a large exponent round to 0)
    lay1 = vals[mag_order].repeat(need // len(vals) + 1)[:need]
    lay2 = vals[torch.as_tensor(rng.integers(0, len(vals), need))]
    for name, q in (("sorted", lay1), ("random", lay2)):
        q = q.view(8, 2, 64, 128).contiguous().to(DEV)
        q[0, 0, 5] = 0                                              # an all-zero head
        w = torch.rand(8, 2, 64, device=DEV) + 0.5
        cfg = spin.make_config(1, 8, 4096, 64, max_rows=2)
        rig = Rig(cfg, 8, 2, 64)
        _say("quantize", name)
        spin.spin_quantize_q(rig.h, rig.batch, q, w)
        torch.cuda.synchronize()
        lay = rig.state.layout
        q8 = np_(rig.state.region("q8", torch.uint8, (8, 2, 64, 128)))
        qe = np_(rig.state.region("qexp", torch.int32, (8, 2, 64)))
        wq = np_(rig.state.region("wq", torch.float32, (8, 2, 64)))
        qv, wv, codes, e = oracle_fp8_operands(q, w)
        assert np.array_equal(qe, e), name
        assert np.array_equal(q8, codes), f"{name}: {np.sum(q8 != codes)} codes differ"
        # w * 2^e is exact in fp32 except where it lands below the normal range
        # (heads of subnormal-sized bf16 values only)
        sane = e > -100
        assert np.array_equal(wq[sane], wv[sane].astype(np.float32)), name
        assert lay["q8"] > 0


# ------------------------------------------------------------------ indexer
def _rand_pool(rng, pages, d=128):
    k = torch.randn(pages, 64, d, generator=torch.Generator().manual_seed(int(rng.integers(1 << 30))))
    amax = k.abs().amax(dim=(1, 2))
    sc = amax / 448.0
    codes = (k / sc[:, None, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, sc.float()


@pytest.mark.parametrize("R", [1, 2, 3, 4])
def test_indexer_scores_parity(gpu_lib, R):
    rng = np.random.default_rng(R)
    B, mb, pages = 3, 40, 150
    codes, sc = _rand_pool(rng, pages)
    table = np.stack([rng.permutation(pages)[:mb] for _ in range(B)]).astype(np.int32)
    qpos = np.array([64 * 37 + 20, 64 * 12 + 63, 64 * 39 - R], dtype=np.int64)
    kept = []
    for b in range(B):
        n = nblocks(qpos[b] + R - 1)
        sel = np.sort(rng.choice(n, size=max(1, n // 2), replace=False))
        sel = np.union1d(sel, [n - 1])                            # ragged last block
        kept.append(sel)
    kept[2] = kept[2][:0]                                        # a request with nothing kept
    q = (torch.randn(B, R, 64, 128) * 2).to(torch.bfloat16)
    w = torch.rand(B, R, 64) + 0.5
    cfg = spin.make_config(1, B, 64 * mb, 2048, max_rows=R)
    rig = Rig(cfg, B, R, mb)
    rig.set_qpos(qpos)
    kt = np.full((B, mb), -1, dtype=np.int32)
    for b in range(B):
        kt[b, : len(kept[b])] = kept[b]
    rig.kept.copy_(torch.as_tensor(kt))
    rig.kept_count.copy_(torch.as_tensor([len(k) for k in kept], dtype=torch.int32))
    rig.scores.fill_(12345.0)
    pq = torch.full((B, R, mb, 4), 777.0, device=DEV)
    _say("indexer R", R)
    spin.spin_quantize_q(rig.h, rig.batch, q.to(DEV), w.to(DEV))
    spin.spin_indexer_scores(rig.h, rig.batch, codes.to(DEV), sc.to(DEV),
                             torch.as_tensor(table).to(DEV), rig.kept, rig.kept_count, rig.scores,
                             pq)
    torch.cuda.synchronize()
    gpq = np_(pq)
    kv = O.e4m3fn_decode(np_(codes))
    scv = np_(sc).astype(np.float64)
    got = np_(rig.scores)
    for b in range(B):
        qv, wv, _, _ = oracle_fp8_operands(q[b], w[b])
        ref = O.indexer_scores(qv, wv, kv, scv, table[b], kept[b], int(qpos[b]))
        mag = score_mag(qv, wv, kv, scv, table[b], kept[b])
        n = len(kept[b]) * 64
        assert_scores_close(got[b, :, :n], ref, mag, f"b{b}")
        assert np.all(got[b, :, n:] == 12345.0)                  # nothing written past kept
        # quarter maxima: exactly the max of each 16-slot quarter of the GPU's own scores
        nk = len(kept[b])
        if nk:
            own = got[b, :, :n].reshape(R, nk, 4, 16).max(axis=3)
            assert np.array_equal(gpq[b, :, :nk], own)
        assert np.all(gpq[b, :, nk:] == 777.0)
    assert rig.state.error() == 0


@pytest.mark.parametrize("R", [1, 4])
def test_indexer_balanced_split_many_short_rows(gpu_lib, R):
    """The indexer splits the batch's kept pages, row after row, into equal
    workgroup shares: with 150 rows (three 64-row walk chunks), kept counts
    from 0 to the maximum and most rows shorter than a share, shares start and
    end inside rows and span many rows; every row must still match the oracle
    and nothing past its kept count may be written."""
    rng = np.random.default_rng(100 + R)
    B, mb, pages = 150, 24, 400
    codes, sc = _rand_pool(rng, pages)
    table = np.stack([rng.permutation(pages)[:mb] for _ in range(B)]).astype(np.int32)
    qpos = rng.integers(64 * 4, 64 * mb - R, size=B).astype(np.int64)
    kept = []
    for b in range(B):
        n = nblocks(qpos[b] + R - 1)
        size = [0, 1, 2, 3, n][b % 5] if b % 7 else int(rng.integers(0, n + 1))
        kept.append(np.sort(rng.choice(n, size=min(size, n), replace=False)))
    q = (torch.randn(B, R, 64, 128) * 2).to(torch.bfloat16)
    w = torch.rand(B, R, 64) + 0.5
    cfg = spin.make_config(1, B, 64 * mb, 2048, max_rows=R)
    rig = Rig(cfg, B, R, mb)
    rig.set_qpos(qpos)
    kt = np.full((B, mb), -1, dtype=np.int32)
    for b in range(B):
        kt[b, : len(kept[b])] = kept[b]
    rig.kept.copy_(torch.as_tensor(kt))
    rig.kept_count.copy_(torch.as_tensor([len(k) for k in kept], dtype=torch.int32))
    rig.scores.fill_(12345.0)
    pq = torch.full((B, R, mb, 4), 777.0, device=DEV)
    _say("indexer balanced split R", R, "rows", B, "kept pages", sum(len(k) for k in kept))
    spin.spin_quantize_q(rig.h, rig.batch, q.to(DEV), w.to(DEV))
    spin.spin_indexer_scores(rig.h, rig.batch, codes.to(DEV), sc.to(DEV),
                             torch.as_tensor(table).to(DEV), rig.kept, rig.kept_count, rig.scores,
                             pq)
    torch.cuda.synchronize()
    gpq = np_(pq)
    kv = O.e4m3fn_decode(np_(codes))
    scv = np_(sc).astype(np.float64)
    got = np_(rig.scores)
    for b in range(B):
        nk = len(kept[b])
        n = nk * 64
        assert np.all(got[b, :, n:] == 12345.0), f"b{b}: written past the kept count"
        assert np.all(gpq[b, :, nk:] == 777.0), f"b{b}"
        if not nk:
            continue
        qv, wv, _, _ = oracle_fp8_operands(q[b], w[b])
        ref = O.indexer_scores(qv, wv, kv, scv, table[b], kept[b], int(qpos[b]))
        mag = score_mag(qv, wv, kv, scv, table[b], kept[b])
        assert_scores_close(got[b, :, :n], ref, mag, f"b{b}")
        own = got[b, :, :n].reshape(R, nk, 4, 16).max(axis=3)
        assert np.array_equal(gpq[b, :, :nk], own), f"b{b}"
    assert rig.state.error() == 0


# ------------------------------------------------------------------- top-k
TOPK_CASES = {
    # name: (rows R, max_blocks, K, pattern); "pm-" cases pass page quarter maxima
    "random": (2, 120, 512, "random"),
    "ties": (2, 120, 512, "ties"),
    "short": (2, 120, 512, "short"),
    "zeros": (2, 120, 512, "zeros"),
    "two-levels": (1, 2048, 2048, "random"),
    "three-levels-ties": (2, 8192, 2048, "ties"),
    "k-equals-chunk-quarter": (1, 1500, 4096, "random"),
    "pm-random": (1, 8192, 2048, "random"),
    "pm-clustered": (2, 8192, 2048, "clustered"),
    "pm-equal-maxima": (1, 4096, 2048, "plateau"),
    "pm-few-pages": (2, 1000, 2048, "random"),
    # fused kernel's own fallback: ties at t1, a row over 16384 kept pages, K = 4096
    # with running merges of up to 2K entries, and signed zeros
    "pm-ties": (2, 4096, 2048, "ties"),
    "pm-over-16k-pages": (1, 20000, 2048, "random"),
    "pm-k4096-chunks": (1, 3000, 4096, "random"),
    "pm-zeros": (2, 1200, 512, "zeros"),
    # as many kept pages as K (the MTP shape: only the quarter-maxima bound filters)
    "pm-pages-equal-k": (1, 3100, 2048, "random"),
    "pm-pages-quarter-k": (2, 800, 2048, "random"),
}


@pytest.mark.parametrize("case", list(TOPK_CASES))
def test_topk_exact_on_identical_scores(gpu_lib, case):
    R, mb, K, pattern = TOPK_CASES[case]
    rng = np.random.default_rng(list(TOPK_CASES).index(case))
    B = 3
    qpos = np.array([64 * (mb - 10) + 5, 64 * (mb - 20) + 63, 64 * 5 + 3], dtype=np.int64)
    kept = [np.sort(rng.choice(nblocks(q + R - 1), nblocks(q + R - 1) * 2 // 3, replace=False))
            for q in qpos]
    kept = [np.union1d(k, [nblocks(q + R - 1) - 1]) for k, q in zip(kept, qpos)]
    if pattern == "short":
        kept[0] = kept[0][:3]                                    # fewer candidates than K
    if case in ("two-levels", "pm-over-16k-pages"):
        kept[1] = np.arange(nblocks(qpos[1]))                    # a whole row kept
    sc = rng.random((B, R, mb * 64)).astype(np.float32)
    if pattern == "ties":
        sc = (np.round(sc * 16) / 16).astype(np.float32)
    if pattern == "zeros":
        sc[:] = 0.0
        sc[:, :, ::7] = -0.0
        sc[:, :, ::13] = 1.0
    if pattern == "clustered":                                   # every large score in 40 pages
        sc *= 0.5
        sc[:, :, 64 * 100: 64 * 140] += 10.0
    if pattern == "plateau":                                     # every page has the same maximum
        sc = np.minimum(sc, np.float32(0.75))
    qp = torch.as_tensor(qpos.astype(np.int32), device=DEV)
    bt = spin.make_batch(torch.zeros(B, dtype=torch.int32, device=DEV), qp, R, mb)
    kt = np.full((B, mb), -1, dtype=np.int32)
    for b in range(B):
        kt[b, : len(kept[b])] = kept[b]
    kept_d = torch.as_tensor(kt, device=DEV)
    cnt_d = torch.as_tensor([len(k) for k in kept], dtype=torch.int32, device=DEV)
    out = torch.zeros(B, R, K, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(256, spin.spin_topk_workspace_bytes(bt, K)), dtype=torch.uint8, device=DEV)
    ws.fill_(0xA5)                                               # stale contents must not matter
    pm = None
    if case.startswith("pm-"):
        # quarter maxima over each row's valid slots, in kept order (as the indexer writes them)
        pmh = np.full((B, R, mb, 4), -np.inf, dtype=np.float32)
        for b in range(B):
            for r in range(R):
                nk = len(kept[b])
                slot = (kept[b][:, None] * 64 + np.arange(64)).reshape(nk, 64)
                v = np.where(slot <= qpos[b] + r, sc[b, r, : nk * 64].reshape(nk, 64), -np.inf)
                pmh[b, r, :nk] = v.reshape(nk, 4, 16).max(axis=2)
        pm = torch.as_tensor(pmh, device=DEV)
    refs = {(b, r): O.topk_positions(sc[b, r, : len(kept[b]) * 64].astype(np.float64), kept[b],
                                     int(qpos[b]) + r, K) for b in range(B) for r in range(R)}
    # with quarter maxima: the collected path (rows spread over workgroups,
    # survivors in the workspace) and the one-workgroup-per-row path
    for workspace in ((ws, None) if pm is not None else (ws,)):
        _say("topk", case, "workspace" if workspace is not None else "no workspace")
        out.fill_(-7)
        spin.spin_topk_scores(bt, K, torch.as_tensor(sc, device=DEV), kept_d, cnt_d, out,
                              workspace, pm)
        torch.cuda.synchronize()
        got = np_(out)
        for b in range(B):
            for r in range(R):
                assert np.array_equal(got[b, r], refs[(b, r)]), (case, b, r, workspace is None)


# --------------------------------------------------------------- predictor
POOL_NAMES = {spin.SPIN_POOL_MAX: O.POOL_MAX, spin.SPIN_POOL_MEAN: O.POOL_MEAN,
              spin.SPIN_POOL_TOP4: O.POOL_TOP4}


@pytest.mark.parametrize("R,keep_bp,explore_bp,step,blocks,policy", [
    (1, 6000, 500, 3, 200, 0), (1, 5000, 0, 1, 200, 0), (1, 8000, 2500, 7, 200, 0),
    (4, 5000, 1000, 2, 200, 0), (4, 6000, 500, 0, 200, 0), (1, 10000, 500, 4, 200, 0),
    (1, 0, 500, 4, 200, 0), (2, 9990, 500, 5, 200, 0), (1, 5000, 10000, 3, 200, 0),
    # register-resident selection at 4, 8 and 16 blocks per thread
    (1, 5000, 500, 3, 12000, 0), (4, 6000, 1000, 2, 12000, 0), (1, 5000, 500, 3, 8192, 0),
    # the MTP shape: 4 rows over 4096 blocks, each row selected by its own workgroup
    (4, 5000, 1000, 2, 4096, 0),
    # past the register-resident limit (16384 blocks): the selection from global memory
    (1, 5000, 500, 3, 17000, 0), (4, 5000, 1000, 2, 17000, 0),
    # the pages' ablation variants: Mean / Top-4 pooling, row-0 mask
    (1, 6000, 500, 3, 200, spin.SPIN_POOL_MEAN), (1, 5000, 1000, 2, 200, spin.SPIN_POOL_TOP4),
    (4, 5000, 1000, 2, 200, spin.SPIN_MASK_ROW0),
    (4, 6000, 500, 3, 200, spin.SPIN_MASK_ROW0 | spin.SPIN_POOL_TOP4),
    (2, 5000, 500, 1, 12000, spin.SPIN_POOL_MEAN), (2, 5000, 500, 1, 17000, spin.SPIN_MASK_ROW0),
    # three verification rows (draft length 2)
    (3, 5000, 1000, 2, 200, 0), (3, 6000, 500, 3, 4096, 0), (3, 5000, 1000, 2, 300, spin.SPIN_MASK_ROW0)])
def test_predict_exact(gpu_lib, R, keep_bp, explore_bp, step, blocks, policy):
    _predict_case(R, keep_bp, explore_bp, step, blocks, policy, "random")


# score ties: V and D on four levels (block scores tie in long runs at the
# threshold), almost never observed (most block scores -inf), or never
# observed at all (every block score -inf, every key equal)
@pytest.mark.parametrize("R,blocks,kind", [
    (1, 200, "levels"), (1, 8192, "levels"), (1, 8192, "sparse"), (1, 8192, "empty"),
    (4, 4096, "levels"), (1, 17000, "levels"), (4, 17000, "sparse"), (2, 12000, "empty")])
def test_predict_exact_ties(gpu_lib, R, blocks, kind):
    _predict_case(R, 5000, 1000, 3, blocks, 0, kind)


def _states(kind, ctx, b):
    if kind == "random":
        V = np_(random_state(ctx, 0.15, seed=10 * b + 1)).astype(np.float64)
        D = np_(random_state(ctx, 0.15, seed=10 * b + 2)).astype(np.float64)
        return V, D
    rng = np.random.default_rng(77 + b)
    if kind == "levels":
        V = np.floor(np.abs(rng.standard_normal(ctx)) * 1.5).clip(0, 3)
        D = np.floor(np.abs(rng.standard_normal(ctx)) * 1.5).clip(0, 3)
        V[rng.random(ctx) < 0.1] = NEG
        D[rng.random(ctx) < 0.1] = NEG
    elif kind == "sparse":
        V = np.full(ctx, NEG)
        D = np.full(ctx, NEG)
        V[rng.integers(0, ctx, max(1, ctx // 20000))] = 2.0
        D[rng.integers(0, ctx, max(1, ctx // 20000))] = 1.0
    else:
        V = np.full(ctx, NEG)
        D = np.full(ctx, NEG)
    return V, D


def _predict_case(R, keep_bp, explore_bp, step, blocks, policy, kind):
    B, ctx = 4, 64 * blocks
    mb = nblocks(ctx - 1)
    qpos = np.array([ctx - R, 64 * (blocks * 3 // 4) + 63 - 1, 64 * 3 + 1, 40], dtype=np.int64)
    cfg = spin.make_config(2, B, ctx, 256, max_rows=R, explore_bp=explore_bp, seed=0xABCDEF,
                           policy=policy)
    pooling = POOL_NAMES[policy & 3]
    mask = O.MASK_ROW0 if policy & spin.SPIN_MASK_ROW0 else O.MASK_UNION
    rig = Rig(cfg, B, R, mb)
    rids = [1000 + 7 * b for b in range(B)]
    rig.reset(rids)
    layer = 1
    states = []
    for b in range(B):
        V, D = _states(kind, ctx, b)
        V[qpos[b] + 1:] = NEG
        rig.inject(layer, b, V.astype(np.float32), D.astype(np.float32), step)
        states.append((V.astype(np.float32).astype(np.float64), D.astype(np.float32).astype(np.float64)))
    rig.set_qpos(qpos)
    _say("predict", R, keep_bp, explore_bp, step, blocks, policy, kind)
    spin.spin_predict_blocks(rig.h, layer, rig.batch, keep_bp, rig.kept, rig.kept_count, rig.flags)
    torch.cuda.synchronize()
    for b in range(B):
        V, D = states[b]
        kept, flags = O.predict_blocks(V, D, int(qpos[b]), R, keep_bp, explore_bp, cfg.seed, layer,
                                       step, rids[b], cfg.warmup_steps, pooling, mask)
        gf = np_(rig.flags[b])
        assert np.all(gf[len(flags):] == 0)
        if pooling != O.POOL_MAX and not np.array_equal(gf[: len(flags)], flags):
            # fp32 sums on the GPU, fp64 in the oracle: only a tie at the
            # predicted-set threshold may differ
            rows = 1 if mask == O.MASK_ROW0 else R
            gp = set(np.nonzero(gf[: len(flags)] == 1)[0].tolist())
            rp = set(np.nonzero(flags == 1)[0].tolist())
            near = set()
            for r in range(rows):
                S = O.block_scores(V, D, int(qpos[b]) + r, pooling)
                _, _, p_ = O.budget(keep_bp, len(S), explore_bp)
                theta = np.sort(S)[::-1][p_ - 1]
                near |= set(np.nonzero(np.abs(S - theta) <= 1e-5 * abs(theta))[0].tolist())
            assert (gp ^ rp) <= near, (b, sorted(gp ^ rp))
            continue
        assert np.array_equal(rig.kept_list(b), kept), b
        assert np.array_equal(gf[: len(flags)], flags), b
    assert rig.state.error() == 0


# ------------------------------------------------------ update and replay
@pytest.mark.parametrize("R", [1, 2, 3, 4])
def test_update_and_replay_parity(gpu_lib, R):
    rng = np.random.default_rng(40 + R)
    B, ctx = 5, 64 * 60
    mb = nblocks(ctx - 1)
    cfg = spin.make_config(1, B, ctx, 256, max_rows=R, alpha=0.9)
    rig = Rig(cfg, B, R, mb)
    qpos = np.array([64 * 50 + 61, 64 * 50 + 63, 64 * 20, 64 * 55 + 2, 63], dtype=np.int64)
    qpos = np.minimum(qpos, ctx - R)
    acc = rng.integers(0, R, B).astype(np.int32)
    states, kept = [], []
    for b in range(B):
        V = np_(random_state(ctx, 0.3, seed=b + 100)).astype(np.float32).astype(np.float64)
        D = np_(random_state(ctx, 0.3, seed=b + 200)).astype(np.float32).astype(np.float64)
        V[qpos[b] + 1:] = NEG
        rig.inject(0, b, V, D, 3)
        n = nblocks(qpos[b] + R - 1)
        k = np.sort(rng.choice(n, size=max(1, (2 * n) // 3), replace=False))
        k = np.union1d(k, [n - 1])
        if b == 1:
            k = np.arange(n)                                     # every block kept
        kept.append(k)
        states.append((V, D))
    kt = np.full((B, mb), -1, dtype=np.int32)
    for b in range(B):
        kt[b, : len(kept[b])] = kept[b]
    rig.kept.copy_(torch.as_tensor(kt))
    rig.kept_count.copy_(torch.as_tensor([len(k) for k in kept], dtype=torch.int32))
    sc = (rng.random((B, R, mb * 64)) * 20).astype(np.float32)
    for b in range(B):
        slot = (kept[b][:, None] * 64 + np.arange(64)).reshape(-1)
        for r in range(R):
            row = sc[b, r, : len(slot)]
            row[slot > qpos[b] + r] = NEG
    rig.scores.copy_(torch.as_tensor(sc))
    rig.set_qpos(qpos)
    _say("update R", R, "accepted", acc.tolist())
    if R == 1:
        spin.spin_update(rig.h, 0, rig.batch, rig.scores, rig.kept, rig.kept_count)
        acc[:] = 0
    else:
        spin.spin_mtp_replay(rig.h, 0, rig.batch, torch.as_tensor(acc, device=DEV), rig.scores,
                             rig.kept, rig.kept_count)
    torch.cuda.synchronize()
    for b in range(B):
        V, D = states[b][0].copy(), states[b][1].copy()
        O.ema_update(V, D, sc[b, :, : len(kept[b]) * 64].astype(np.float64), kept[b], int(qpos[b]),
                     int(acc[b]), 0.9)
        gV, gD, gVB, gstep = rig.read_state(0, b)
        for name, g, r in (("V", gV, V), ("D", gD, D)):
            fin = np.isfinite(r)
            assert np.array_equal(fin, np.isfinite(g)), (name, b)
            tol = 1e-3 * np.abs(r[fin]) + 1e-6
            assert np.all(np.abs(g[fin] - r[fin]) <= tol), (name, b)
        # unobserved entries are bit-unchanged
        slot = (kept[b][:, None] * 64 + np.arange(64)).reshape(-1)
        obs_v = np.zeros(ctx, dtype=bool)
        obs_d = np.zeros(ctx, dtype=bool)
        for r in range(int(acc[b]) + 1):
            i = slot[slot <= qpos[b] + r]
            obs_v[i] = True
            obs_d[qpos[b] + r - i] = True
        assert np.array_equal(gV[~obs_v], states[b][0][~obs_v]), b
        assert np.array_equal(gD[~obs_d], states[b][1][~obs_d]), b
        vb = np.concatenate([gV, np.full(mb * 64 - len(gV), NEG)]).reshape(mb, 64).max(1)
        assert np.array_equal(gVB[kept[b]], vb[kept[b]]), b
        assert gstep == 4
    assert rig.state.error() == 0



@pytest.mark.parametrize("R", [2, 4])
def test_replay_every_acceptance_and_kept_pattern(gpu_lib, R):
    """Prefix-valid replay with every acceptance 0..R-1 against kept lists that
    put every neighbour case at every position of a wave's four entries:
    alternate blocks (each kept block's predecessor skipped, so its owner also
    takes the offsets just before it), runs of two and three, all blocks, and
    a random half; positions at, just past and just before block boundaries."""
    rng = np.random.default_rng(70 + R)
    B, ctx = 8, 64 * 48
    mb = nblocks(ctx - 1)
    cfg = spin.make_config(1, B, ctx, 256, max_rows=R, alpha=0.75)
    rig = Rig(cfg, B, R, mb)
    qpos = np.array([64 * 40, 64 * 40 + 1, 64 * 41 - 1, 64 * 41 - 2, 64 * 33 + 31,
                     64 * 44 + 7, 64 * 45 - R, 64 * 30 + 62], dtype=np.int64)
    qpos = np.minimum(qpos, ctx - R)
    acc = np.array([b % R for b in range(B)], dtype=np.int32)
    states, kept = [], []
    for b in range(B):
        V = np_(random_state(ctx, 0.3, seed=b + 300)).astype(np.float32).astype(np.float64)
        D = np_(random_state(ctx, 0.3, seed=b + 400)).astype(np.float32).astype(np.float64)
        V[qpos[b] + 1:] = NEG
        rig.inject(0, b, V, D, 2)
        n = nblocks(qpos[b] + R - 1)
        kind = b % 4
        if kind == 0:
            k = np.arange(0, n, 2)                               # alternate blocks
        elif kind == 1:
            k = np.array([j for j in range(n) if j % 5 in (0, 1, 3)])   # runs of 2 and 1
        elif kind == 2:
            k = np.arange(n)                                     # every block
        else:
            k = np.sort(rng.choice(n, size=max(1, n // 2), replace=False))
        k = np.union1d(k, [n - 1])
        kept.append(k)
        states.append((V, D))
    kt = np.full((B, mb), -1, dtype=np.int32)
    for b in range(B):
        kt[b, : len(kept[b])] = kept[b]
    rig.kept.copy_(torch.as_tensor(kt))
    rig.kept_count.copy_(torch.as_tensor([len(k) for k in kept], dtype=torch.int32))
    sc = (rng.random((B, R, mb * 64)) * 20).astype(np.float32)
    for b in range(B):
        slot = (kept[b][:, None] * 64 + np.arange(64)).reshape(-1)
        for r in range(R):
            row = sc[b, r, : len(slot)]
            row[slot > qpos[b] + r] = NEG
    rig.scores.copy_(torch.as_tensor(sc))
    rig.set_qpos(qpos)
    _say("replay R", R, "accepted", acc.tolist())
    spin.spin_mtp_replay(rig.h, 0, rig.batch, torch.as_tensor(acc, device=DEV), rig.scores,
                         rig.kept, rig.kept_count)
    torch.cuda.synchronize()
    for b in range(B):
        V, D = states[b][0].copy(), states[b][1].copy()
        O.ema_update(V, D, sc[b, :, : len(kept[b]) * 64].astype(np.float64), kept[b], int(qpos[b]),
                     int(acc[b]), 0.75)
        gV, gD, gVB, gstep = rig.read_state(0, b)
        for name, g, r in (("V", gV, V), ("D", gD, D)):
            fin = np.isfinite(r)
            assert np.array_equal(fin, np.isfinite(g)), (name, b)
            tol = 1e-3 * np.abs(r[fin]) + 1e-6
            assert np.all(np.abs(g[fin] - r[fin]) <= tol), (name, b)
        slot = (kept[b][:, None] * 64 + np.arange(64)).reshape(-1)
        obs_v = np.zeros(ctx, dtype=bool)
        obs_d = np.zeros(ctx, dtype=bool)
        for r in range(int(acc[b]) + 1):
            i = slot[slot <= qpos[b] + r]
            obs_v[i] = True
            obs_d[qpos[b] + r - i] = True
        assert np.array_equal(gV[~obs_v], states[b][0][~obs_v]), b
        assert np.array_equal(gD[~obs_d], states[b][1][~obs_d]), b
        vb = np.concatenate([gV, np.full(mb * 64 - len(gV), NEG)]).reshape(mb, 64).max(1)
        assert np.array_equal(gVB[kept[b]], vb[kept[b]]), b
        assert gstep == 3
    assert rig.state.error() == 0

def test_measure_miss_parity(gpu_lib):
    rng = np.random.default_rng(7)
    B, R, mb, K = 3, 2, 50, 300
    full = rng.integers(-1, mb * 64, (B, R, K)).astype(np.int32)
    flags = rng.integers(0, 3, (B, mb)).astype(np.uint8)
    bt = spin.make_batch(torch.zeros(B, dtype=torch.int32, device=DEV),
                         torch.zeros(B, dtype=torch.int32, device=DEV), R, mb)
    miss = torch.zeros(B, R, device=DEV)
    spin.spin_measure_miss(bt, K, torch.as_tensor(full, device=DEV),
                           torch.as_tensor(flags, device=DEV), miss)
    got = np_(miss)
    for b in range(B):
        for r in range(R):
            assert abs(got[b, r] - O.miss_rate(full[b, r], flags[b])) < 1e-6


def test_device_errors_flagged_with_per_row_selection(gpu_lib):
    """Four rows building their own masks take the per-row selection and the
    union kernel: a request with a bad slot or position is reported, gets no
    kept blocks and zero flags, and the other request is still selected (its
    first round keeps every block of its last row)."""
    R = 4
    cfg = spin.make_config(1, 2, 4096, 64, max_rows=R)
    rig = Rig(cfg, 2, R, 64)
    rig.reset([11, 12])
    rig.slot.copy_(torch.tensor([0, 7], dtype=torch.int32))        # slot 7 >= max_slots
    rig.set_qpos([100, 100])
    _say("predict R=4 with a bad slot")
    spin.spin_predict_blocks(rig.h, 0, rig.batch, 5000, rig.kept, rig.kept_count, rig.flags)
    torch.cuda.synchronize()
    assert rig.state.error() & spin.ERR_SLOT
    assert int(rig.kept_count[1]) == 0
    assert int(rig.flags[1].sum()) == 0
    assert int(rig.kept_count[0]) == nblocks(100 + R - 1)
    assert np.array_equal(np_(rig.kept[0, : nblocks(100 + R - 1)]), np.arange(nblocks(100 + R - 1)))
    rig.slot.copy_(torch.tensor([0, 1], dtype=torch.int32))
    rig.set_qpos([100, 4096 - 2])                                  # rows past max_ctx
    _say("predict R=4 with a bad position")
    spin.spin_predict_blocks(rig.h, 0, rig.batch, 5000, rig.kept, rig.kept_count, rig.flags)
    torch.cuda.synchronize()
    assert rig.state.error() & spin.ERR_QPOS
    assert int(rig.kept_count[1]) == 0
    assert int(rig.flags[1].sum()) == 0
    assert int(rig.kept_count[0]) == nblocks(100 + R - 1)


def test_device_errors_flagged_without_faults(gpu_lib):
    cfg = spin.make_config(1, 2, 4096, 64)
    rig = Rig(cfg, 2, 1, 64)
    rig.slot.copy_(torch.tensor([0, 7], dtype=torch.int32))        # slot 7 >= max_slots
    rig.set_qpos([100, 100])
    spin.spin_predict_blocks(rig.h, 0, rig.batch, 5000, rig.kept, rig.kept_count, rig.flags)
    torch.cuda.synchronize()
    assert rig.state.error() & spin.ERR_SLOT
    assert int(rig.kept_count[1]) == 0
    rig.slot.copy_(torch.tensor([0, 1], dtype=torch.int32))
    rig.set_qpos([100, 4096])                                      # past max_ctx
    spin.spin_predict_blocks(rig.h, 0, rig.batch, 5000, rig.kept, rig.kept_count, rig.flags)
    spin.spin_update(rig.h, 0, rig.batch, rig.scores, rig.kept, rig.kept_count)
    torch.cuda.synchronize()
    assert rig.state.error() & spin.ERR_QPOS
    assert int(rig.kept_count[1]) == 0


def test_device_errors_indexer_update_replay(gpu_lib):
    """Bad device-side values the host cannot check: a kept entry past
    max_blocks, a block-table entry past the pool, a kept count past
    max_blocks, an accepted count past the rows.  Each is flagged in the
    state's error word; the offending page, entry or request is skipped (its
    scores -inf, its state untouched) and everything else is computed as
    usual.  Every kernel checks these values before it reads through them."""
    rng = np.random.default_rng(21)
    B, mb, pages = 2, 8, 16
    codes, sc = _rand_pool(rng, pages)
    table = np.stack([rng.permutation(pages)[:mb] for _ in range(B)]).astype(np.int32)
    table[0, 2] = pages + 83                                    # past the pool
    qpos = np.array([64 * mb - 1, 64 * mb - 1], dtype=np.int64)
    cfg = spin.make_config(1, B, 64 * mb, 256, max_rows=2, alpha=0.9)
    rig = Rig(cfg, B, 1, mb)
    rig.reset([31, 32])
    rig.set_qpos(qpos)
    kt = np.full((B, mb), -1, dtype=np.int32)
    kt[0, :4] = [0, 1, mb + 1, 2]                               # entry 2 past max_blocks
    kt[1, :] = np.arange(mb)
    rig.kept.copy_(torch.as_tensor(kt))
    rig.kept_count.copy_(torch.as_tensor([4, 100], dtype=torch.int32))   # 100 > max_blocks
    q = (torch.randn(B, 1, 64, 128) * 2).to(torch.bfloat16)
    w = torch.rand(B, 1, 64) + 0.5
    _say("indexer with bad kept entries, a page past the pool, a count past max_blocks")
    spin.spin_quantize_q(rig.h, rig.batch, q.to(DEV), w.to(DEV))
    spin.spin_indexer_scores(rig.h, rig.batch, codes.to(DEV), sc.to(DEV),
                             torch.as_tensor(table).to(DEV), rig.kept, rig.kept_count, rig.scores)
    torch.cuda.synchronize()
    err = rig.state.error()
    assert err & spin.ERR_KEPT and err & spin.ERR_PAGE
    got = np_(rig.scores)
    kv = O.e4m3fn_decode(np_(codes))
    scv = np_(sc).astype(np.float64)
    for b, good in ((0, [(0, 0), (1, 1)]), (1, [(i, i) for i in range(mb)])):
        qv, wv, _, _ = oracle_fp8_operands(q[b], w[b])
        for pos, j in good:
            ref = O.indexer_scores(qv, wv, kv, scv, table[b], np.array([j]), int(qpos[b]))
            mag = score_mag(qv, wv, kv, scv, table[b], np.array([j]))
            assert_scores_close(got[b, :, 64 * pos: 64 * pos + 64], ref, mag, f"b{b} page {pos}")
    assert np.all(got[0, 0, 128:256] == -np.inf)                 # the two skipped pages

    # the update over the same lists: the bad entry is skipped and flagged,
    # the clamped count covers every block of request 1
    V0, D0 = [np_(x).copy() for x in (rig.state.V(), rig.state.D())]
    s_fin = np.where(np.isfinite(got), got, 0.0).astype(np.float32)
    rig.scores.copy_(torch.as_tensor(s_fin))
    rig.kept_count.copy_(torch.as_tensor([4, mb], dtype=torch.int32))
    _say("update with a bad kept entry")
    spin.spin_update(rig.h, 0, rig.batch, rig.scores, rig.kept, rig.kept_count)
    torch.cuda.synchronize()
    V1 = np_(rig.state.V())
    for j in (0, 1, 2):                                          # kept blocks observed
        assert np.all(np.isfinite(V1[0, 0, 64 * j: 64 * j + 64]))
    assert np.array_equal(V1[0, 0, 64 * 3: 64 * mb], V0[0, 0, 64 * 3: 64 * mb])   # untouched
    assert int(rig.state.step()[0, 0]) == 1 and int(rig.state.step()[0, 1]) == 1

    # a replay whose accepted count is past the rows: that request is skipped
    cfg2 = spin.make_config(1, B, 64 * mb, 256, max_rows=2, alpha=0.9)
    rig2 = Rig(cfg2, B, 2, mb)
    rig2.reset([41, 42])
    rig2.set_qpos([64 * 4, 64 * 4])
    kt2 = np.tile(np.arange(mb, dtype=np.int32), (B, 1))
    rig2.kept.copy_(torch.as_tensor(kt2))
    rig2.kept_count.copy_(torch.as_tensor([5, 5], dtype=torch.int32))
    rig2.scores.copy_(torch.as_tensor(rng.random((B, 2, mb * 64)).astype(np.float32)))
    Vb = np_(rig2.state.V()).copy()
    _say("replay with accepted past the rows")
    spin.spin_mtp_replay(rig2.h, 0, rig2.batch, torch.tensor([1, 2], dtype=torch.int32, device=DEV),
                         rig2.scores, rig2.kept, rig2.kept_count)
    torch.cuda.synchronize()
    assert rig2.state.error() & spin.ERR_ACCEPT
    Va = np_(rig2.state.V())
    assert np.array_equal(Va[0, 1], Vb[0, 1]) and int(rig2.state.step()[0, 1]) == 0
    assert np.all(np.isfinite(Va[0, 0, : 64 * 4 + 2])) and int(rig2.state.step()[0, 0]) == 1
