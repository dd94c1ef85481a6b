"""spin_topk_scores_noalloc (the top-k for callers that cannot allocate: its
chunked levels keep their survivors in the library's static device scratch)
against spin_topk_scores with a caller workspace: identical results on two
calls in a row, the second with a smaller batch, and a clear rejection of a
batch whose chunked path needs more than the scratch holds."""
import numpy as np
import pytest
import torch

import predictive_kv_block_amd as spin
from tests.spin_harness import nblocks, np_

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(B, R, mb, K, seed, ties):
    rng = np.random.default_rng(seed)
    qpos = np.array([64 * (mb - 1 - (b % 3)) + int(rng.integers(0, 64)) - R for b in range(B)],
                    dtype=np.int64)
    kept = []
    for q in qpos:
        n = nblocks(q + R - 1)
        k = np.sort(rng.choice(n, max(1, n * 3 // 4), replace=False))
        kept.append(np.union1d(k, [n - 1]))
    sc = rng.random((B, R, mb * 64)).astype(np.float32)
    if ties:
        sc = (np.round(sc * 32) / 32).astype(np.float32)
    kt = np.full((B, mb), -1, dtype=np.int32)
    for b in range(B):
        kt[b, : len(kept[b])] = kept[b]
    qp = torch.as_tensor(qpos.astype(np.int32), device=DEV)
    bt = spin.make_batch(torch.zeros(B, dtype=torch.int32, device=DEV), qp, R, mb)
    d = dict(bt=bt, qp=qp, scores=torch.as_tensor(sc, device=DEV),
             kept=torch.as_tensor(kt, device=DEV),
             cnt=torch.as_tensor([len(k) for k in kept], dtype=torch.int32, device=DEV))
    # page quarter maxima over each row's valid slots, in kept order
    pm = np.full((B, R, mb, 4), -np.inf, dtype=np.float32)
    for b in range(B):
        for r in range(R):
            nk = len(kept[b])
            slot = (kept[b][:, None] * 64 + np.arange(64)).reshape(nk, 64)
            v = np.where(slot <= qpos[b] + r, sc[b, r, : nk * 64].reshape(nk, 64), -np.inf)
            pm[b, r, :nk] = v.reshape(nk, 4, 16).max(axis=2)
    d["pm"] = torch.as_tensor(pm, device=DEV)
    return d


def _pair(d, K, with_pm):
    B, R = d["scores"].shape[0], d["scores"].shape[1]
    pm = d["pm"] if with_pm else None
    ref = torch.full((B, R, K), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(256, spin.spin_topk_workspace_bytes(d["bt"], K)), dtype=torch.uint8,
                     device=DEV)
    spin.spin_topk_scores(d["bt"], K, d["scores"], d["kept"], d["cnt"], ref, ws, pm)
    got = torch.full((B, R, K), -9, dtype=torch.int32, device=DEV)
    spin.spin_topk_scores_noalloc(d["bt"], K, d["scores"], d["kept"], d["cnt"], got, pm)
    torch.cuda.synchronize()
    return np_(ref), np_(got)


def test_noalloc_topk_equals_workspace_topk_twice(gpu_lib):
    # first call: 8 rows of 2048 blocks (8 chunks of 16384 slots: two levels),
    # then a smaller one: 2 rows of 700 blocks, K 512, heavy ties
    for i, (B, R, mb, K, ties) in enumerate(((4, 2, 2048, 2048, False), (2, 1, 700, 512, True))):
        d = _case(B, R, mb, K, seed=40 + i, ties=ties)
        need = spin.spin_topk_workspace_bytes(d["bt"], K)
        print("[case] noalloc call", i, "rows", B * R, "blocks", mb, "K", K, "scratch", need,
              flush=True)
        assert 0 < need <= 32 << 20
        ref, got = _pair(d, K, with_pm=False)
        assert np.array_equal(ref, got), i
        assert np.all(got[:, :, 0] >= 0)
        # with page quarter maxima (no scratch used): the same answer
        ref2, got2 = _pair(d, K, with_pm=True)
        assert np.array_equal(ref2, got2) and np.array_equal(ref2, ref), i


def test_noalloc_topk_rejects_batches_beyond_the_scratch(gpu_lib):
    B, R, mb, K = 64, 1, 8192, 2048            # chunked path: about 67 MB of survivors
    qp = torch.full((B,), 64 * mb - 1, dtype=torch.int32, device=DEV)
    bt = spin.make_batch(torch.zeros(B, dtype=torch.int32, device=DEV), qp, R, mb)
    assert spin.spin_topk_workspace_bytes(bt, K) > 32 << 20
    sc = torch.zeros(16, dtype=torch.float32, device=DEV)       # never read: rejected first
    kept = torch.zeros(16, dtype=torch.int32, device=DEV)
    out = torch.zeros(16, dtype=torch.int32, device=DEV)
    with pytest.raises(spin.SpinError) as ei:
        spin.spin_topk_scores_noalloc(bt, K, sc, kept, kept, out)
    assert ei.value.status == spin.SPIN_ESCRATCH
    assert "static scratch" in str(ei.value)
