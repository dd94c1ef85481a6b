"""Seeded synthetic inputs for SPIN decode rounds.

This module only draws inputs: paged fp8 indexer keys with per-page scales,
block tables, bf16 queries, head weights, query positions and MTP
acceptances.  It holds none of the method's arithmetic (no scores, EMAs,
selection or exploration) and is the only code the oracle and the HIP path
have in common.

Structure follows the pages' Figure 1 caption (vertical lines and diagonal
bands in the indexer top-k patterns): a share of "heavy" slots whose keys align
with a slowly drifting query direction (vertical lines), and a query term
pointing at the key a fixed distance back (a diagonal band).  All generation
runs in torch on the requested device, in chunks, so the 512K-token pool can
be drawn on the GPU in seconds; the same seed on the same device always gives
the same arrays.
"""

import math
from dataclasses import dataclass, field

import torch

BLOCK = 64
FP8_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    ctx: int                    # context length (tokens) at the last round
    heads: int
    head_dim: int
    topk: int
    steps: int                  # decode rounds
    sparsity_bp: tuple          # target block sparsities (basis points)
    explore_bp: int             # exploration share of the kept budget
    alpha: float                # EMA history weight
    rows: int = 1               # query rows per request (1 + draft length)
    fp8: bool = True            # False: fp32 keys and queries, no quantisation
    heavy: tuple = (0.01,)      # heavy-slot share per layer (or absolute count if >= 1)
    g_v: float = 4.0            # gain of the drifting direction in the queries
    g_d: float = 0.0            # gain of the diagonal term
    o_d: int = 256              # diagonal offset
    redraw: int = 0             # rounds per heavy-set epoch (0: one epoch)
    shuffle: bool = False       # shuffled block table over the pool
    pool_factor: float = 1.0    # pool pages / (batch * blocks per request)
    seed: int = 0x5350494E
    omega: float = 0.01         # drift of the query direction, rad / round

    @property
    def blocks(self):
        return (self.ctx + BLOCK - 1) // BLOCK

    @property
    def pool_pages(self):
        return int(round(self.batch * self.blocks * self.pool_factor))


WORKLOADS = {
    # One layer, batch 1, 4096 tokens, fp32 keys and queries, 16 planted
    # vertical slots, one diagonal band at offset 128.
    "tiny-4k": Workload("tiny-4k", 1, 1, 4096, 4, 32, 256, 32, (4000,), 500, 0.9,
                        fp8=False, heavy=(16,), g_v=4.0, g_d=4.0, o_d=128),
    # DeepSeek-indexer shapes (64 heads x 128), 9728-token context, batch 1.
    "ctx9k-b1": Workload("ctx9k-b1", 1, 1, 9728, 64, 128, 2048, 256,
                         (2000, 3000, 4000, 5000), 500, 0.9,
                         heavy=(0.01,), g_v=4.0, g_d=2.0, o_d=256),
    # 96256-token context, batch 8; heavy set re-drawn every 64 rounds.
    "ctx94k-b8": Workload("ctx94k-b8", 1, 8, 96256, 64, 128, 2048, 128, (3000, 5000),
                          500, 0.9, heavy=(0.02,), g_v=4.0, g_d=0.0, redraw=64),
    # Serving-shaped round: batch 96, 507K cached + 5K new = 524288 tokens,
    # 8192 pages of 64 per request, shuffled paged pool.
    "ctx512k-b96": Workload("ctx512k-b96", 1, 96, 524288, 64, 128, 2048, 64,
                            (0, 4000, 5000), 500, 0.9, heavy=(0.02,), g_v=4.0,
                            g_d=0.0, redraw=64, shuffle=True),
    # MTP: 4 query rows, batch 32, 256K context, 4 layers with their own keys.
    "mtp-ctx256k-b32": Workload("mtp-ctx256k-b32", 4, 32, 262144, 64, 128, 2048, 64,
                                (5000,), 1000, 0.9, rows=4,
                                heavy=(0.005, 0.01, 0.02, 0.04), g_v=4.0, g_d=1.0,
                                o_d=64, shuffle=True),
}


def _gen(device, *tags):
    """A torch.Generator on `device` seeded from the integer tags."""
    g = torch.Generator(device=device)
    h = 0
    for t in tags:
        h = (h * 1000003 + (int(t) & 0xFFFFFFFF)) % (1 << 62)
    g.manual_seed(h)
    return g


def _unit(x):
    return x / x.norm(dim=-1, keepdim=True)


@dataclass
class Pool:
    """One layer's paged indexer keys and the requests' block tables."""
    key_codes: torch.Tensor          # uint8 [P, 64, d] e4m3fn codes (fp8 mode)
    key_scale: torch.Tensor          # fp32 [P]
    key_f32: torch.Tensor            # fp32 [P, 64, d] (fp32 mode only, else None)
    block_table: torch.Tensor        # int32 [B, blocks]
    dir_a: torch.Tensor              # fp32 [B, E, d] epoch directions
    dir_b: torch.Tensor              # fp32 [B, E, d]
    heavy: list = field(default_factory=list)   # per epoch: int64 [B, n_heavy] positions


def positions(wl, accepted=None):
    """Row-0 query position of every round, int64 [steps, B].

    Single-row workloads: q_t = ctx - steps + t, so the last round sees exactly
    ctx tokens.  MTP workloads advance each request by accepted + 1 per round
    from ctx - rows * steps, so q + rows - 1 < ctx always.
    """
    if wl.rows == 1:
        q = torch.arange(wl.steps, dtype=torch.int64) + (wl.ctx - wl.steps)
        return q[:, None].repeat(1, wl.batch)
    acc = accepted if accepted is not None else acceptances(wl)
    q = torch.empty(wl.steps, wl.batch, dtype=torch.int64)
    cur = torch.full((wl.batch,), wl.ctx - wl.rows * wl.steps, dtype=torch.int64)
    for t in range(wl.steps):
        q[t] = cur
        cur = cur + acc[t] + 1
    return q


def acceptances(wl):
    """Accepted draft count per (round, request), uniform on 0..rows-1."""
    g = _gen("cpu", wl.seed, 7, 0)
    return torch.randint(0, wl.rows, (wl.steps, wl.batch), generator=g, dtype=torch.int64)


def _heavy_count(wl, layer):
    h = wl.heavy[layer % len(wl.heavy)]
    return int(h) if h >= 1 else max(1, int(round(h * wl.ctx)))


def make_pool(wl, layer, device="cpu", chunk_pages=8192):
    """Draw one layer's key pool and block tables."""
    B, nb, d = wl.batch, wl.blocks, wl.head_dim
    P = wl.pool_pages
    g = _gen(device, wl.seed, layer, 1)
    gc = _gen("cpu", wl.seed, layer, 2)
    if wl.shuffle:
        perm = torch.randperm(P, generator=gc)[: B * nb]
    else:
        perm = torch.arange(B * nb)
    table = perm.view(B, nb).to(torch.int32)

    epochs = 1 if wl.redraw == 0 else (wl.steps + wl.redraw - 1) // wl.redraw
    dir_a = _unit(torch.randn(B, epochs, d, generator=g, device=device))
    rb = torch.randn(B, epochs, d, generator=g, device=device)
    rb = rb - (rb * dir_a).sum(-1, keepdim=True) * dir_a
    dir_b = _unit(rb)

    # Heavy (vertical) slots: disjoint sets per epoch inside the prompt region.
    n_heavy = _heavy_count(wl, layer)
    prompt = max(1, wl.ctx - wl.rows * wl.steps)
    heavy = []
    order = torch.argsort(torch.rand(B, prompt, generator=gc), dim=1)
    for e in range(epochs):
        heavy.append(order[:, e * n_heavy:(e + 1) * n_heavy].contiguous())

    # physical page -> (request, block) of the pages in use
    owner = torch.full((P,), -1, dtype=torch.int64)
    owner[perm] = torch.arange(B * nb)
    heavy_dir = torch.zeros(B, wl.ctx, dtype=torch.int8)         # epoch + 1, 0 = none
    for e, hs in enumerate(heavy):
        heavy_dir.scatter_(1, hs, e + 1)

    codes = torch.empty(P, BLOCK, d, dtype=torch.uint8, device=device) if wl.fp8 else None
    kf32 = None if wl.fp8 else torch.empty(P, BLOCK, d, dtype=torch.float32, device=device)
    scale = torch.ones(P, dtype=torch.float32, device=device)
    for p0 in range(0, P, chunk_pages):
        p1 = min(P, p0 + chunk_pages)
        k = torch.randn(p1 - p0, BLOCK, d, generator=g, device=device)
        own = owner[p0:p1]
        used = own >= 0
        if bool(used.any()):
            req = torch.where(used, own // nb, 0)
            blk = torch.where(used, own % nb, 0)
            pos = blk[:, None] * BLOCK + torch.arange(BLOCK)[None, :]
            inctx = used[:, None] & (pos < wl.ctx)
            posc = pos.clamp(max=wl.ctx - 1)
            ep = torch.where(inctx, heavy_dir[req[:, None].expand_as(posc), posc].long(), 0)
            hv = ep > 0
            if bool(hv.any()):
                hv_d = hv.to(device)
                r_idx = req[:, None].expand_as(posc)[hv].to(device)
                e_idx = (ep[hv] - 1).to(device)
                a = dir_a[r_idx, e_idx]
                n = torch.randn(a.shape, generator=g, device=device)
                n = _unit(n - (n * a).sum(-1, keepdim=True) * a)
                k[hv_d] = math.sqrt(d) * (0.8 * a + 0.6 * n)
        if wl.fp8:
            amax = k.abs().amax(dim=(1, 2))
            sc = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
            kq = (k / sc[:, None, None]).clamp(-FP8_MAX, FP8_MAX)
            codes[p0:p1] = kq.to(torch.float8_e4m3fn).view(torch.uint8)
            scale[p0:p1] = sc
        else:
            kf32[p0:p1] = k
    return Pool(codes, scale, kf32, table.to(device), dir_a, dir_b, heavy)


def key_values_of(pool, pages):
    """fp32 keys (fp32 mode) of the given pages, as [n, 64, d] (for diagonals)."""
    return pool.key_f32[pages]


def make_queries(wl, pool, layer, step, qpos, device="cpu"):
    """Queries and head weights of one round.

    q[b, r, h] = g_v * u_t + g_d * khat(qpos + r - o_d) + xi,  xi ~ N(0, I),
    u_t = cos(omega t) a_e + sin(omega t) b_e  (e = epoch of round t),
    khat = the unit key at that position (term dropped if it is < 0).
    Returns q (bf16 in fp8 mode, else fp32) [B, R, H, d] and w fp32 [B, R, H]
    with w ~ U(0.5, 1.5).
    """
    B, R, H, d = wl.batch, wl.rows, wl.heads, wl.head_dim
    g = _gen(device, wl.seed, layer, 100 + step)
    e = 0 if wl.redraw == 0 else min(step // wl.redraw, pool.dir_a.shape[1] - 1)
    u = math.cos(wl.omega * step) * pool.dir_a[:, e] + math.sin(wl.omega * step) * pool.dir_b[:, e]
    q = wl.g_v * u[:, None, None, :].expand(B, R, H, d).clone()
    if wl.g_d != 0.0:
        qpos = torch.as_tensor(qpos, dtype=torch.int64).cpu()
        for r in range(R):
            tgt = qpos + r - wl.o_d
            ok = tgt >= 0
            tgt = tgt.clamp(min=0)
            pages = pool.block_table.cpu()[torch.arange(B), (tgt // BLOCK)].to(torch.int64)
            tok = tgt % BLOCK
            if wl.fp8:
                kv = pool.key_codes[pages.to(device), tok.to(device)].view(torch.float8_e4m3fn).float()
            else:
                kv = pool.key_f32[pages.to(device), tok.to(device)]
            kv = _unit(kv) * ok.to(device)[:, None]
            q[:, r] += wl.g_d * kv[:, None, :]
    q = q + torch.randn(B, R, H, d, generator=g, device=device)
    w = torch.rand(B, R, H, generator=g, device=device) + 0.5
    if wl.fp8:
        q = q.to(torch.bfloat16)
    return q, w.float()


def random_state(n, neg_inf_share, seed, device="cpu"):
    """A synthetic EMA-like array of n fp32 values for single-round tests.

    Values are |N(0, 1)| * 10 with a `neg_inf_share` of entries set to -inf
    (never observed), plus a few exact duplicates so that ties occur.
    """
    g = _gen(device, seed, 55)
    x = torch.randn(n, generator=g, device=device).abs() * 10.0
    dup = torch.randint(0, n, (max(1, n // 50),), generator=g, device=device)
    x[dup] = x[dup[0]].clone()
    ninf = torch.rand(n, generator=g, device=device) < neg_inf_share
    x[ninf] = float("-inf")
    return x
