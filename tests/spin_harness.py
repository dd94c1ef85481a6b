"""Helpers shared by the GPU parity tests: state injection, oracle operands and
the acceptance rules (score tolerance, tie-aware set comparison)."""
import numpy as np
import torch

import predictive_kv_block_amd as spin
from oracle import spin_oracle as O

NEG = float("-inf")
BLOCK = 64


def np_(t):
    return t.detach().cpu().numpy()


def nblocks(q):
    return (q + BLOCK) // BLOCK


# --------------------------------------------------------------- tolerances
def score_mag(qv, wv, key_values, page_scale, table, kept):
    """mag(i) = scale * sum_h |w_h| * sum_d |q_hd k_id| per kept slot, per row."""
    kept = np.asarray(kept, dtype=np.int64)
    R = qv.shape[0]
    out = np.zeros((R, len(kept) * BLOCK))
    if len(kept) == 0:
        return out
    pages = np.asarray(table, dtype=np.int64)[kept]
    keys = np.abs(key_values[pages].reshape(len(kept) * BLOCK, -1))
    sc = np.repeat(np.asarray(page_scale, dtype=np.float64)[pages], BLOCK)
    for r in range(R):
        out[r] = sc * (np.abs(wv[r])[:, None] * (np.abs(qv[r]) @ keys.T)).sum(0)
    return out


def score_tol(ref, mag):
    return np.maximum(1e-3 * np.abs(ref), 1e-5 * mag)


def assert_scores_close(gpu, ref, mag, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(gpu)), f"{what}: masked slots differ"
    err = np.abs(gpu[fin] - ref[fin])
    tol = score_tol(ref[fin], mag[fin])
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {fin.sum()} scores outside tolerance; "
                           f"worst err {err.max():.3e} at tol {tol[np.argmax(err)]:.3e}")


def assert_topk_tie_aware(gpu_row, ref_row, score_of, tol_of, what=""):
    """Equal size; every element of the symmetric difference within 2 tol of theta."""
    g = np.asarray(gpu_row)
    r = np.asarray(ref_row)
    gv = g[g >= 0]
    rv = r[r >= 0]
    assert np.all(g[len(gv):] == -1) and np.all(np.diff(gv) > 0), f"{what}: not ascending/padded"
    assert len(gv) == len(rv), f"{what}: sizes {len(gv)} vs {len(rv)}"
    diff = set(gv.tolist()) ^ set(rv.tolist())
    if diff:
        theta = min(score_of(x) for x in rv.tolist())
        for x in diff:
            assert abs(score_of(x) - theta) <= 2 * tol_of(x), \
                f"{what}: slot {x} score {score_of(x)} vs theta {theta}"
    return len(diff)


# ------------------------------------------------------------ state handling
class Rig:
    """A bound GPU state plus the per-call device buffers of one batch shape."""

    def __init__(self, cfg, B, R, max_blocks):
        self.cfg = cfg
        self.B, self.R, self.mb = B, R, max_blocks
        self.state = spin.SpinState(cfg)
        dev = "cuda"
        self.slot = torch.arange(B, dtype=torch.int32, device=dev)
        self.qpos = torch.zeros(B, dtype=torch.int32, device=dev)
        self.kept = torch.full((B, max_blocks), -7, dtype=torch.int32, device=dev)
        self.kept_count = torch.zeros(B, dtype=torch.int32, device=dev)
        self.flags = torch.full((B, max_blocks), 9, dtype=torch.uint8, device=dev)
        self.scores = torch.zeros(B, R, max_blocks * BLOCK, dtype=torch.float32, device=dev)
        self.topk = torch.zeros(B, R, cfg.topk, dtype=torch.int32, device=dev)
        self.batch = spin.make_batch(self.slot, self.qpos, R, max_blocks)
        self.topk_ws = torch.empty(max(256, spin.spin_topk_workspace_bytes(self.batch, cfg.topk)),
                                   dtype=torch.uint8, device=dev)

    @property
    def h(self):
        return self.state.handle

    def set_qpos(self, q):
        self.qpos.copy_(torch.as_tensor(np.asarray(q), dtype=torch.int32))

    def reset(self, request_ids):
        rid = torch.as_tensor(np.asarray(request_ids, dtype=np.uint64).view(np.int64),
                              device="cuda")
        spin.spin_reset_slots(self.h, self.slot[: len(request_ids)].clone(), rid)

    def inject(self, layer, b, V, D, step):
        """Write V, D (fp32) and step of (layer, slot b); VB := block max of V."""
        Vs, Ds, VBs, St = self.state.V(), self.state.D(), self.state.VB(), self.state.step()
        n = len(V)
        Vs[layer, b, :n] = torch.as_tensor(V, dtype=torch.float32)
        Ds[layer, b, :n] = torch.as_tensor(D, dtype=torch.float32)
        full = Vs[layer, b]
        nb = self.state.layout["max_blocks"]
        pad = torch.full((nb * BLOCK - full.numel(),), NEG, device=full.device)
        VBs[layer, b] = torch.cat([full, pad]).view(nb, BLOCK).amax(dim=1)
        St[layer, b] = int(step)

    def read_state(self, layer, b):
        return (np_(self.state.V()[layer, b]).astype(np.float64),
                np_(self.state.D()[layer, b]).astype(np.float64),
                np_(self.state.VB()[layer, b]).astype(np.float64),
                int(self.state.step()[layer, b]))

    def kept_list(self, b):
        c = int(self.kept_count[b])
        return np_(self.kept[b, :c]).astype(np.int64)


def oracle_fp8_operands(q_bf16, w):
    """Oracle-side (qv, wv, codes, e) from the same bf16 queries."""
    q = np_(q_bf16.float()).astype(np.float64)
    return O.fp8_query_operands(q, np_(w).astype(np.float64))


def pool_values(pool, pages=None):
    """Decoded key values (fp64) and scales of (a subset of) the pool pages."""
    codes = pool.key_codes if pages is None else pool.key_codes[pages]
    sc = pool.key_scale if pages is None else pool.key_scale[pages]
    return O.e4m3fn_decode(np_(codes)), np_(sc).astype(np.float64)


def sync_from_oracle(rig, layer, b, ost, lockstep=False):
    """Set GPU slot b of `layer` to the oracle's state rounded to fp32 (V, D,
    VB = block max of V, step).  Data flows oracle -> GPU only.  With
    `lockstep` the oracle's own state is rounded to the same fp32 values, so
    both sides start the next round from identical numbers."""
    V32 = ost.V.astype(np.float32)
    D32 = ost.D.astype(np.float32)
    if lockstep:
        ost.V[:] = V32.astype(np.float64)
        ost.D[:] = D32.astype(np.float64)
    rig.inject(layer, b, V32, D32, ost.step)


def predicted_sets_tie_only(ost_before, q, R, keep_bp, explore_bp, gpu_pred, ref_pred, rel=2e-3):
    """True if the predicted block sets differ and every block in their
    symmetric difference lies, for at least one row r, within `rel` of that
    row's predicted-set threshold (the P-th largest block score from the
    oracle's state before the round): an fp32-vs-fp64 tie, not an error."""
    from oracle import spin_oracle as O
    gp, rp = set(gpu_pred), set(ref_pred)
    if gp == rp:
        return False
    near = set()
    for r in range(R):
        S = O.block_scores(ost_before.V, ost_before.D, q + r)
        kb, ne, p = O.budget(keep_bp, len(S), explore_bp)
        if kb >= len(S) or p == 0:
            continue
        theta = np.sort(S)[::-1][p - 1]
        near |= {j for j in gp ^ rp if j < len(S) and abs(S[j] - theta) <= rel * abs(theta)}
    return near == gp ^ rp


class StateView:
    """The injectable parts (V, D, VB, step) of a bound SpinState, for
    sync_from_oracle outside a Rig."""

    def __init__(self, st):
        self.state = st

    def inject(self, layer, b, V, D, step):
        Vs, Ds, VBs, St = self.state.V(), self.state.D(), self.state.VB(), self.state.step()
        Vs[layer, b] = torch.as_tensor(V, dtype=torch.float32)
        Ds[layer, b] = torch.as_tensor(D, dtype=torch.float32)
        nb = self.state.layout["max_blocks"]
        pad = torch.full((nb * BLOCK - Vs.shape[2],), NEG, device=Vs.device)
        VBs[layer, b] = torch.cat([Vs[layer, b], pad]).view(nb, BLOCK).amax(dim=1)
        St[layer, b] = int(step)
