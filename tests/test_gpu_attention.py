"""GPU parity of the sparse core attention over the top-k against the oracle.

Tolerance, from the arithmetic: the kernel rounds each softmax weight to bf16
before the value product (relative error <= 2^-9 per weight, so <= 2^-9 *
max_i |v_ic| on output channel c), rounds each share's normalised partial to
bf16 (<= 2^-9 |o_s| <= 2^-9 max_i |v_ic|, and the merge is a convex
combination of the partials) and rounds the output to bf16 (<= 2^-9 |o|);
fp32 sums and exp2 add far less.  Bound used:
|o - o_ref| <= 2^-8 * max_i |v_ic| + 2^-8 * |o_ref|.  The log-sum-exp moves by
at most the largest score error, which for fp32 sums of 576 bf16 products is
below scale * 576 * 2^-23 * max_i sum_d |q_d k_id|; 1e-5 (1 + |lse|) covers
the exp2 / log2 steps.
"""
import numpy as np
import pytest
import torch

import predictive_kv_block_amd as spin
from oracle import spin_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"
H, D, DV = 128, 576, 512


def _say(*a):
    print("[case]", *a, flush=True)


def _bf16(rng, shape, scale=1.0):
    x = torch.from_numpy((rng.standard_normal(size=shape) * scale).astype(np.float32))
    return x.to(torch.bfloat16)


def _topk_lists(rng, B, R, K, qpos, fill):
    """Ascending valid positions (<= q + r) then -1 padding; `fill` = share of K used."""
    out = np.full((B, R, K), -1, dtype=np.int32)
    for b in range(B):
        for r in range(R):
            q = int(qpos[b]) + r
            n = min(q + 1, int(round(K * fill)))
            if n > 0:
                out[b, r, :n] = np.sort(rng.choice(q + 1, size=n, replace=False))
    return out


def _run(B, R, K, mb, pool_pages, qpos, topk, scale, table, seed):
    rng = np.random.default_rng(seed)
    q = _bf16(rng, (B, R, H, D))
    kv = _bf16(rng, (pool_pages, 64, D))
    qd, kvd = q.to(DEV), kv.to(DEV)
    bt = spin.make_batch(torch.arange(B, dtype=torch.int32, device=DEV),
                         torch.as_tensor(np.asarray(qpos, dtype=np.int32), device=DEV), R, mb)
    ws_n = spin.spin_attention_workspace_bytes(bt, K)
    ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device=DEV) if ws_n else None
    out = torch.full((B, R, H, DV), 7.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, R, H), 7.0, dtype=torch.float32, device=DEV)
    spin.spin_sparse_attention(bt, K, torch.as_tensor(topk, device=DEV), qd, kvd,
                               torch.as_tensor(table, device=DEV), scale, out, lse, ws)
    torch.cuda.synchronize()
    return q.float().numpy(), kv.float().numpy(), out.float().cpu().numpy(), lse.cpu().numpy(), ws_n


def _check_row(qb, kv, table_b, top, qr, scale, o_gpu, lse_gpu, what):
    # the kernel's masking rule: entries < 0, past the row's position, or in a
    # block whose page is outside the pool are skipped
    t = np.asarray(top, dtype=np.int64)
    t = t[(t >= 0) & (t <= qr)]
    pg = np.asarray(table_b, dtype=np.int64)[t // 64]
    t = t[(pg >= 0) & (pg < kv.shape[0])]
    if len(t) == 0:
        assert np.all(o_gpu == 0.0) and np.all(lse_gpu == -np.inf), what
        return
    o_ref, lse_ref = O.sparse_attention(qb, kv, table_b, t, qr, scale, DV)
    rows = kv[np.asarray(table_b, dtype=np.int64)[t // 64], t % 64].astype(np.float64)
    vmax = np.abs(rows[:, :DV]).max(axis=0)
    tol = 2.0 ** -8 * vmax[None, :] + 2.0 ** -8 * np.abs(o_ref)
    err = np.abs(o_gpu - o_ref)
    assert np.all(err <= tol), (what, float((err - tol).max()))
    smag = np.abs(qb.astype(np.float64)) @ np.abs(rows).T            # [H][n]
    ltol = scale * 576 * 2.0 ** -23 * smag.max(axis=1) + 1e-5 * (1 + np.abs(lse_ref))
    assert np.all(np.abs(lse_gpu - lse_ref) <= ltol), (what, float(np.abs(lse_gpu - lse_ref).max()))


@pytest.mark.parametrize("B,R,K,blocks,fill,scale", [
    (2, 1, 2048, 80, 1.0, 0.0722),        # 2 rows: 16 shares each
    (3, 4, 256, 20, 1.0, 0.0722),         # MTP rows
    (1, 2, 100, 10, 1.0, 0.3),            # ragged K, sharp softmax
    (4, 1, 4096, 100, 0.6, 0.0722),       # K = 4096, lists 60% full
    (128, 4, 64, 3, 1.0, 0.05),           # 512 rows: one share per row (no merge)
])
def test_attention_matches_oracle(gpu_lib, B, R, K, blocks, fill, scale):
    rng = np.random.default_rng(B * 100 + K)
    mb = blocks
    qpos = np.array([64 * blocks - R - int(rng.integers(0, 60)) for _ in range(B)])
    pool = B * blocks
    table = rng.permutation(pool)[: B * mb].reshape(B, mb).astype(np.int32)
    topk = _topk_lists(rng, B, R, K, qpos, fill)
    _say("attention", B, R, K, blocks, fill, scale)
    q, kv, o, lse, ws_n = _run(B, R, K, mb, pool, qpos, topk, scale, table, seed=K + B)
    rows = [(b, r) for b in range(B) for r in range(R)]
    if len(rows) > 24:
        rows = [rows[i] for i in rng.choice(len(rows), size=24, replace=False)]
    for b, r in rows:
        _check_row(q[b, r], kv, table[b], topk[b, r], int(qpos[b]) + r, scale, o[b, r], lse[b, r],
                   (b, r))


def test_attention_masks_and_bad_rows(gpu_lib):
    """Entries past the row's position, block-table entries outside the pool,
    an empty list (o = 0, lse = -inf) and a request whose position is out of
    range (o = 0, lse = NaN)."""
    rng = np.random.default_rng(5)
    B, R, K, mb = 4, 2, 128, 12
    pool = 30
    table = rng.integers(0, pool, size=(B, mb)).astype(np.int32)
    table[0, 3] = pool + 5                 # outside the pool
    table[1, 2] = -1
    qpos = np.array([64 * mb - 2, 64 * 7 + 3, 64 * 5, 64 * mb])   # request 3: row 1 past max_blocks
    topk = _topk_lists(rng, B, R, K, qpos, 1.0)
    topk[0, 0, 5] = 3 * 64 + 7             # in the block that maps outside the pool
    topk[1, 1, 0] = int(qpos[1]) + 5       # past the row's position
    topk[2, :, :] = -1                     # nothing to attend to
    _say("attention masks")
    q, kv, o, lse, _ = _run(B, R, K, mb, pool, qpos, topk, 0.0722, table, seed=11)
    for b in range(3):
        for r in range(R):
            _check_row(q[b, r], kv, table[b], topk[b, r], int(qpos[b]) + r, 0.0722, o[b, r],
                       lse[b, r], (b, r))
    assert np.all(o[3] == 0.0) and np.all(np.isnan(lse[3]))


def test_attention_bench_shape_sampled(gpu_lib):
    """The launch the benchmark times: batch 96, one row, top-2048, 8192
    blocks per request (512K context); pages drawn from a smaller pool.
    Eight rows are checked in full against the oracle."""
    rng = np.random.default_rng(96)
    B, R, K, mb = 96, 1, 2048, 8192
    pool = 2048
    table = rng.integers(0, pool, size=(B, mb)).astype(np.int32)
    qpos = np.full(B, 64 * mb - 1)
    topk = np.stack([np.sort(rng.choice(64 * mb, size=K, replace=False)) for _ in range(B)])
    topk = topk.astype(np.int32)[:, None, :]
    _say("attention bench shape")
    q, kv, o, lse, ws_n = _run(B, R, K, mb, pool, qpos, topk, 0.0722, table, seed=3)
    assert ws_n > 0                        # several shares per row: merged
    for b in rng.choice(B, size=8, replace=False):
        _check_row(q[b, 0], kv, table[b], topk[b, 0], int(qpos[b]), 0.0722, o[b, 0], lse[b, 0],
                   int(b))
