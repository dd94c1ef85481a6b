"""SPIN oracle: a plain, slow, fp64 CPU statement of one SPIN decode step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check in the package entry
file and the CPU-baseline leg of the benchmark may import or call this module.
It shares no code, table or constant generator with the HIP library, and the
HIP library never calls it.

Sources (the pages describing SPIN, arXiv 2610.09025):
  [radio]  AI Radio episode "SPIN: Shadow Predictive Indexer for Sparse
           Attention", segment "Title and authors": the predicted slot score
           z_{t,i} = max(V_i, D_{q_t - i}), logical blocks of b slots, the block
           score S_{t,j} = max over slots of block j; segment "The paper's
           summary": skipped blocks get no EMA update, a share gamma of the block
           budget goes to random exploration.
  [digest] ai4snews digest "SPIN用历史索引分数预测KV块重要性…", section
           "arXiv深度剖析": per-slot (vertical) and per-relative-offset (diagonal)
           EMA state of past indexer scores; sparsity applied per KV block; a
           reserved exploration share inside the same block budget; for MTP the
           block masks of all verification queries are unioned and the EMA
           update is deferred and replayed over the prefix-valid rows.
  [v1]     "SPIN: Shadow Predictive Indexer for Sparse Attention" (v1 listing):
           Abstract (the indexer scores the whole KV cache every step; a fixed
           top-k goes to core attention); Table 1 (prev-iter and random
           predictors); Table 5 caption (mean/p99 miss over eligible sparse
           decode rows); Table 7 (row-local union + prefix-valid update).
  [v3]     paperdot record of arXiv 2610.09025 v3, abstract: the block budget
           is allocated across layers by their measured miss rates.

The pages leave the indexer formula, dtypes, alpha, initialisation, tie rules
and RNG unstated.  The readings taken here (each marked READING below) are:
  * indexer score  s(i) = sum_h w_h * ReLU(q_h . k_i)   (the DSA indexer), keys
    stored as fp8 e4m3fn with one fp32 scale per 64-token page, queries
    quantised to e4m3fn with a power-of-two scale per (row, head);
  * EMA  x <- alpha*x + (1-alpha)*s, alpha the history weight, alpha and
    beta = fp32(1 - alpha) both fp32 values; -inf = never observed, the first
    observation sets x <- s; unobserved entries do not change;
  * block budget K_b = ceil(keep_bp * N / 10^4) in integers, exploration count
    n_exp = floor(explore_bp * K_b / 10^4), predicted count P = K_b - n_exp;
  * ties go to the lower block index / lower position;
  * exploration draws: Philox4x64-10 (Salmon et al., SC'11) with
    key = (seed, layer), counter = (j div 4, step, request_id, 0), word j mod 4;
    the n_exp non-predicted blocks with the smallest words are explored;
  * the first decode step of a (layer, request) is all-keep (warm-up);
  * block pooling variants (v1, Figure 3 caption, "Mean and Top-4 compared
    with Max pooling"): mean = the average of z over the block's existing
    slots whose z is finite (never-observed slots carry no score), top-4 = the
    average of the 4 largest such z (fewer if the block has fewer); a block
    with no finite z scores -inf under every pooling;
  * predictor quality (v1 Table 1): Pearson correlation over the slots where
    prediction and indexer score are both finite; top-k recall = shared
    slots of the two top-k sets over the indexer's top-k size;
  * online miss estimate: the explored blocks are a uniform sample of the
    non-predicted ones; weighting each explored slot by the inverse sampling
    rate places the all-keep top-k threshold inside the sparse round's own
    top-k, and the explored slots above it, scaled by skipped / explored,
    estimate the miss (estimate_miss);
  * core attention over the top-k: every head attends to one shared cache
    row per token (absorbed multi-head latent attention), softmax over the
    row's valid top-k entries, the value being the row's first d_v entries;
  * row-0 mask policy (v1 Table 7 and Figure 2, "row-0" vs "row-local union"):
    the mask built for row 0 serves every row; the blocks past row 0's last
    block, which only the later rows reach (they hold the draft positions),
    are kept as predicted.  The row-0 update policy is the replay with
    accepted = 0 (only row 0's scores update the EMAs).

Every floating-point step runs in fp64 on the exact values of the inputs
(fp8 codes decoded exactly, bf16/fp32 widened exactly).
"""

import math

import numpy as np

BLOCK = 64
FP8_MAX = 448.0
NEG_INF = float("-inf")
MASK64 = (1 << 64) - 1


# ---------------------------------------------------------------------------
# fp8 e4m3fn (OCP 8-bit floating point specification): 1 sign bit, 4 exponent
# bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN.
# ---------------------------------------------------------------------------
def e4m3fn_value(code):
    """Exact real value of one e4m3fn code (NaN for the two NaN codes)."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6          # subnormal
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3FN = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)
# Non-negative finite codes 0x00..0x7E have strictly increasing values.
_POS_CODES = np.arange(0x7F)
_POS_VALUES = E4M3FN[:0x7F]


def e4m3fn_decode(codes):
    """Decode an array of uint8 e4m3fn codes to fp64 values."""
    return E4M3FN[np.asarray(codes, dtype=np.uint8)]


def e4m3fn_encode(x):
    """Round fp64 values with |x| <= 448 to the nearest e4m3fn code.

    Ties go to the code with an even mantissa (round-to-nearest-even).  The
    sign bit follows the sign of x, so negative values that round to zero give
    the code 0x80.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > FP8_MAX) or np.any(np.isnan(x)):
        raise ValueError("e4m3fn_encode: input outside [-448, 448]")
    hi = np.searchsorted(_POS_VALUES, a, side="left")        # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(a == _POS_VALUES[hi], hi, np.where(pick_hi, hi, lo))
    code = code.astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


# ---------------------------------------------------------------------------
# Query quantisation (READING: exact power-of-two scale per (row, head)).
# ---------------------------------------------------------------------------
def q_exponent(amax):
    """Smallest integer e with amax * 2**-e <= 448; 0 when amax == 0."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    e = math.frexp(amax)[1] - 12          # amax * 2**-e >= 2**11 > 448 here
    while amax * 2.0 ** -e > FP8_MAX:
        e += 1
    return e


def quantize_q(q):
    """q: [..., H, d] real values (bf16 widened).  Returns (codes, e, q8 values).

    Each (row, head) vector is multiplied by 2**-e, e = q_exponent(max |q|),
    which is exact, and rounded to e4m3fn.
    """
    q = np.asarray(q, dtype=np.float64)
    amax = np.abs(q).max(axis=-1)
    e = np.vectorize(q_exponent, otypes=[np.int64])(amax)
    scaled = q * np.exp2(-e.astype(np.float64))[..., None]
    codes = e4m3fn_encode(scaled)
    return codes, e, e4m3fn_decode(codes)


# ---------------------------------------------------------------------------
# Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
# easy as 1, 2, 3", SC'11): ten rounds of two 64x64->128 multiplies, with the
# key bumped by the Weyl increments between rounds.
# ---------------------------------------------------------------------------
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15        # golden ratio
PHILOX_W1 = 0xBB67AE8584CAA73B        # sqrt(3) - 1


def philox4x64_10(counter, key):
    c0, c1, c2, c3 = (int(v) & MASK64 for v in counter)
    k0, k1 = (int(v) & MASK64 for v in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        c0, c1, c2, c3 = ((p1 >> 64) ^ c1 ^ k0, p1 & MASK64,
                          (p0 >> 64) ^ c3 ^ k1, p0 & MASK64)
    return c0, c1, c2, c3


def explore_keys(n_blocks, seed, layer, step, request_id):
    """Random sort key u_j of every block j < n_blocks (Python ints)."""
    out = []
    for g in range((n_blocks + 3) // 4):
        words = philox4x64_10((g, step, request_id, 0), (seed, layer))
        out.extend(words)
    return out[:n_blocks]


# ---------------------------------------------------------------------------
# Predictor: z, block max-pool, budget, selection, exploration, MTP union.
# ---------------------------------------------------------------------------
def num_blocks(qpos):
    """Blocks of the context 0..qpos: ceil((qpos+1)/64)."""
    return (qpos + 1 + BLOCK - 1) // BLOCK


def budget(keep_bp, n_blocks, explore_bp):
    """(K_b, n_exp, P): kept blocks, of which n_exp explored, P predicted."""
    k_b = (keep_bp * n_blocks + 9999) // 10000
    n_exp = (explore_bp * k_b) // 10000
    return k_b, n_exp, k_b - n_exp


def slot_scores(V, D, qpos):
    """z_i = max(V_i, D_{qpos - i}) for i = 0..qpos  [radio, Title and authors]."""
    i = np.arange(qpos + 1)
    return np.maximum(V[i], D[qpos - i])


POOL_MAX, POOL_MEAN, POOL_TOP4 = "max", "mean", "top4"


def block_scores(V, D, qpos, pooling=POOL_MAX):
    """S_j = max of z over the existing slots of block j  [radio]; or, as the
    v1 Figure 3 variants (READING above), the mean of the finite z, or the mean
    of the 4 largest finite z."""
    z = slot_scores(V, D, qpos)
    n = num_blocks(qpos)
    padded = np.full(n * BLOCK, NEG_INF)
    padded[: qpos + 1] = z
    blocks = padded.reshape(n, BLOCK)
    if pooling == POOL_MAX:
        return blocks.max(axis=1) + 0.0     # -0 -> +0
    out = np.full(n, NEG_INF)
    for j in range(n):
        fin = blocks[j][np.isfinite(blocks[j])]
        if len(fin) == 0:
            continue
        if pooling == POOL_TOP4:
            fin = np.sort(fin)[::-1][:4]
        elif pooling != POOL_MEAN:
            raise ValueError(pooling)
        out[j] = fin.mean() + 0.0
    return out


def top_blocks(S, count):
    """Indices of the `count` largest S, ties to the lower index."""
    order = np.argsort(-S, kind="stable")
    return np.sort(order[:count])


def explored_blocks(pred_mask, n_exp, keys):
    """The n_exp non-predicted blocks with the smallest keys, ties -> lower j."""
    cand = [j for j in range(len(pred_mask)) if not pred_mask[j]]
    cand.sort(key=lambda j: (keys[j], j))
    return np.sort(np.array(cand[:n_exp], dtype=np.int64))


def predict_row(V, D, qpos, keep_bp, explore_bp, keys, all_keep, pooling=POOL_MAX):
    """Masks of one query row: (predicted bool[N], explored bool[N])."""
    n = num_blocks(qpos)
    pred = np.zeros(n, dtype=bool)
    expl = np.zeros(n, dtype=bool)
    k_b, n_exp, p = budget(keep_bp, n, explore_bp)
    if all_keep or keep_bp >= 10000 or k_b >= n:
        pred[:] = True
        return pred, expl
    S = block_scores(V, D, qpos, pooling)
    pred[top_blocks(S, p)] = True
    expl[explored_blocks(pred, n_exp, keys)] = True
    return pred, expl


MASK_UNION, MASK_ROW0 = "union", "row0"


def predict_blocks(V, D, qpos, rows, keep_bp, explore_bp, seed, layer, step,
                   request_id, warmup_steps=1, pooling=POOL_MAX, mask=MASK_UNION):
    """One request's kept block list for a round of `rows` query rows.

    Row r has query position qpos + r and builds its own mask; the kept set is
    the union over rows [digest; v1 Table 7, row-local union].  Exploration
    keys do not depend on the row.  With mask = MASK_ROW0 only row 0 builds a
    mask, and the blocks past row 0's last block are added as predicted
    (READING above).  Returns (kept ascending int64[], flags uint8[N_last])
    with flag 1 = predicted by some row, 2 = explored only.
    """
    n_last = num_blocks(qpos + rows - 1)
    all_keep = step < warmup_steps
    keys = explore_keys(n_last, seed, layer, step, request_id)
    pred_u = np.zeros(n_last, dtype=bool)
    expl_u = np.zeros(n_last, dtype=bool)
    mask_rows = 1 if mask == MASK_ROW0 else rows
    if mask not in (MASK_UNION, MASK_ROW0):
        raise ValueError(mask)
    for r in range(mask_rows):
        pred, expl = predict_row(V, D, qpos + r, keep_bp, explore_bp, keys, all_keep, pooling)
        pred_u[: len(pred)] |= pred
        expl_u[: len(expl)] |= expl
    if mask == MASK_ROW0:
        pred_u[num_blocks(qpos):] = True
    flags = np.where(pred_u, 1, np.where(expl_u, 2, 0)).astype(np.uint8)
    return np.nonzero(flags)[0].astype(np.int64), flags


# ---------------------------------------------------------------------------
# Indexer on the kept blocks (READING: DSA indexer score).
# ---------------------------------------------------------------------------
def indexer_scores(qv, wv, key_values, page_scale, block_table, kept, qpos):
    """Scores of every slot of every kept block, for each row.

    qv [R, H, d] and wv [R, H]: query values and head weights as the indexer
    multiplies them (decoded q8 and w * 2**e for fp8 queries).
    key_values [pages, 64, d]: key values (decoded e4m3fn codes).
    page_scale [pages]: per-page key scale.  Slot 64*j + t of kept block j
    lives in page block_table[j], token t.  Returns [R, len(kept)*64], in kept
    order, with -inf for slots after the row's query position.
    """
    R = qv.shape[0]
    kept = np.asarray(kept, dtype=np.int64)
    out = np.full((R, len(kept) * BLOCK), NEG_INF)
    if len(kept) == 0:
        return out
    pages = np.asarray(block_table, dtype=np.int64)[kept]
    keys = key_values[pages].reshape(len(kept) * BLOCK, -1)          # [slots, d]
    scale = np.repeat(np.asarray(page_scale, dtype=np.float64)[pages], BLOCK)
    slot = (kept[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
    for r in range(R):
        dots = qv[r] @ keys.T                                        # [H, slots]
        s = scale * (wv[r][:, None] * np.maximum(dots, 0.0)).sum(axis=0) + 0.0
        out[r] = np.where(slot <= qpos + r, s, NEG_INF)
    return out


def topk_positions(scores_row, kept, qpos_r, k):
    """The k kept slots <= qpos_r with the largest scores, ties -> lower slot.

    Returned ascending, padded with -1 to length k.
    """
    kept = np.asarray(kept, dtype=np.int64)
    slot = (kept[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
    valid = slot <= qpos_r
    cand_slot = slot[valid]
    cand_score = np.asarray(scores_row)[valid] + 0.0
    order = np.argsort(-cand_score, kind="stable")        # slot order is ascending
    chosen = np.sort(cand_slot[order[:k]])
    out = np.full(k, -1, dtype=np.int64)
    out[: len(chosen)] = chosen
    return out


# ---------------------------------------------------------------------------
# Sparse core attention over the top-k  [v1 Abstract: a fixed top-k of
# tokens goes to core attention].
# ---------------------------------------------------------------------------
def sparse_attention(q, kv_pages, block_table, topk, qpos_r, scale, d_v):
    """Softmax attention of one query row over the slots of its top-k.

    READING (the pages name DeepSeek-V3.2 / V4 and say only that a fixed top-k
    of tokens goes to core attention): multi-head attention in which every
    head attends to one shared cache row per token (the absorbed form of
    multi-head latent attention): s_h(i) = scale * q_h . c_i over the valid
    entries i of the top-k (>= 0 and <= qpos_r), o_h = sum_i softmax_i(s_h)
    c_i[:d_v], lse_h = log sum_i exp(s_h(i)).  The cache row of slot i sits in
    page block_table[i // 64] at row i % 64 (the indexer's block table).  A
    row with no valid entry gives o = 0 and lse = -inf.
    q: [H][d]; kv_pages: [P][64][d]; returns o [H][d_v], lse [H] (fp64).
    """
    q = np.asarray(q, dtype=np.float64)
    H = q.shape[0]
    t = np.asarray(topk, dtype=np.int64)
    t = t[(t >= 0) & (t <= qpos_r)]
    if len(t) == 0:
        return np.zeros((H, d_v)), np.full(H, NEG_INF)
    pages = np.asarray(block_table, dtype=np.int64)[t // BLOCK]
    rows = np.asarray(kv_pages, dtype=np.float64)[pages, t % BLOCK]    # [n][d]
    s = scale * (q @ rows.T)                                           # [H][n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1)
    o = (e @ rows[:, :d_v]) / l[:, None]
    return o, m[:, 0] + np.log(l)


# ---------------------------------------------------------------------------
# EMA update from observed slots only, with prefix-valid MTP replay.
# ---------------------------------------------------------------------------
def ema_weights(alpha):
    """(alpha, beta) as fp64 widenings of fp32 alpha and fp32(1 - alpha)."""
    a32 = np.float32(alpha)
    return float(a32), float(np.float32(1.0) - a32)


def ema_observe(x, s, alpha, beta):
    """One EMA observation: -inf (never seen) takes s, else alpha*x + beta*s."""
    x = np.asarray(x, dtype=np.float64)
    s = np.broadcast_to(np.asarray(s, dtype=np.float64), x.shape)
    out = s.copy()
    seen = x != NEG_INF
    out[seen] = alpha * x[seen] + beta * s[seen]
    return out


def ema_update(V, D, scores, kept, qpos, accepted, alpha):
    """Apply rows 0..accepted in order to V (per slot) and D (per offset).

    Row r observes every kept slot i <= qpos + r and updates V_i and
    D_{qpos + r - i} with its score; blocks that were not kept and rows above
    `accepted` change nothing.  V, D are modified in place.
    """
    a64, b64 = ema_weights(alpha)
    kept = np.asarray(kept, dtype=np.int64)
    slot = (kept[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
    for r in range(accepted + 1):
        seen = slot <= qpos + r
        i = slot[seen]
        s = np.asarray(scores[r])[seen]
        V[i] = ema_observe(V[i], s, a64, b64)
        o = qpos + r - i
        D[o] = ema_observe(D[o], s, a64, b64)


# ---------------------------------------------------------------------------
# Selection fidelity and per-layer budgets  [v1 Table 5 caption; v3 abstract].
# ---------------------------------------------------------------------------
def miss_rate(full_topk, flags):
    """Share of the all-keep top-k slots that fall in skipped blocks."""
    full = np.asarray(full_topk, dtype=np.int64)
    full = full[full >= 0]
    if len(full) == 0:
        return 0.0
    blk = full // BLOCK
    flags = np.asarray(flags)
    skipped = np.array([blk_j >= len(flags) or flags[blk_j] == 0 for blk_j in blk])
    return float(skipped.sum()) / len(full)


def estimate_miss(sparse_topk, topk_scores, flags, qpos_r, k):
    """Online estimate of one row's miss from its exploration blocks, with no
    all-keep indexer.  Returns (estimate, upper bound).

    READING (the miss of the v1 Table 5 caption; the exploration share of
    the digest and the radio summary, a random sample inside the budget): the
    explored blocks E (flag 2) are a uniform sample without replacement of the
    blocks U not predicted (flag != 1) among the row's N_r blocks, and
    S = U minus E (flag 0) are skipped; k_r = min(k, qpos_r + 1) is the size
    of the all-keep top-k.

    estimate: each slot of E stands for |U| / |E| slots of U, so the all-keep
    top-k threshold is placed where the sparse round's own top-k, walked from
    the highest score down (ties to the lower position) with weight 1 per
    predicted slot and |U| / |E| per explored slot, first reaches k_r.  That
    threshold is never below the sparse top-k's own, so the walk ends inside
    it (or takes all of it when it is not full).  With c_E explored slots
    passed on the way, c_E * |S| / (|E| * k_r) estimates the share of the
    all-keep top-k in S.  Integer weights (|E| and |U|, target k_r * |E|)
    make the walk exact.

    upper bound: h * |S| / (|E| * k_r) with h all explored slots of the
    sparse top-k; every all-keep top-k slot in a kept block is in it, and
    when top slots are missed lower ones take their places, so h >= c_E.

    Both clamped to 1; (0, 0) when nothing is skipped; (-1, -1) when blocks
    are skipped but none explored.  Ratios in fp64, rounded to fp32.
    """
    n = num_blocks(qpos_r)
    f = np.asarray(flags)[:n]
    n_skip = int((f == 0).sum())
    n_expl = int((f == 2).sum())
    n_u = n_skip + n_expl
    if n_skip == 0:
        return 0.0, 0.0
    if n_expl == 0:
        return -1.0, -1.0
    t = np.asarray(sparse_topk, dtype=np.int64)
    sc = np.asarray(topk_scores, dtype=np.float64)
    ok = (t >= 0) & (t <= qpos_r)
    t, sc = t[ok], sc[ok]
    blk = t // BLOCK
    keep = f[blk] != 0                   # the top-k of a sparse round holds kept slots only
    t, sc, blk = t[keep], sc[keep], blk[keep]
    is_e = f[blk] == 2
    k_r = min(k, qpos_r + 1)
    order = np.lexsort((t, -(sc + 0.0)))   # score descending, then lower position
    c_e = 0
    acc = 0
    for idx in order:
        acc += n_u if is_e[idx] else n_expl
        c_e += int(is_e[idx])
        if acc >= k_r * n_expl:
            break
    h = int(is_e.sum())
    ratio = lambda c: float(np.float32(min(1.0, c * n_skip / (n_expl * k_r))))
    return ratio(c_e), ratio(h)


def pearson(pred, actual):
    """Pearson correlation of a predictor's slot scores with the indexer's.

    READING of v1 Table 1 ("Pearson correlation" of predicted and actual
    indexer scores): over the slots where both are finite (a slot never
    observed has no prediction); 0 when fewer than 2 such slots remain or
    either side is constant on them.
    """
    x = np.asarray(pred, dtype=np.float64)
    y = np.asarray(actual, dtype=np.float64)
    m = np.isfinite(x) & np.isfinite(y)
    x, y = x[m], y[m]
    if len(x) < 2 or np.all(x == x[0]) or np.all(y == y[0]):
        return 0.0
    return float(np.corrcoef(x, y)[0, 1])


def topk_recall(pred, actual, k):
    """Top-k recall of a slot predictor (v1 Table 1): the share of the
    indexer's top-k slots that are also in the predictor's top-k.

    Both sets are taken by topk_positions over slots 0..len-1 (ties to the
    lower slot; a -inf prediction ranks last); the share is of the
    min(k, len) actual top-k slots.
    """
    n = len(actual)
    nb = (n + BLOCK - 1) // BLOCK
    allb = np.arange(nb)
    pad = lambda v: np.concatenate([np.asarray(v, dtype=np.float64),
                                    np.full(nb * BLOCK - n, NEG_INF)])
    tp = topk_positions(pad(pred), allb, n - 1, k)
    ta = topk_positions(pad(actual), allb, n - 1, k)
    tp, ta = tp[tp >= 0], ta[ta >= 0]
    return len(np.intersect1d(tp, ta)) / len(ta) if len(ta) else 0.0


def allocate_budgets(miss, mean_keep_bp, eps=1e-3):
    """Per-layer keep budgets (basis points) from measured mean miss rates.

    READING of the v3 abstract: keep_l = clamp(c * (miss_l + eps), mean/2,
    10000), with the water level c found by bisection so that the layers'
    total equals L * mean_keep_bp; then rounded to integer basis points by
    largest remainder (ties to the lower layer), which keeps the total exact.
    """
    m = np.asarray(miss, dtype=np.float64)
    L = len(m)
    total = float(L * mean_keep_bp)
    lo, hi = mean_keep_bp / 2.0, 10000.0
    w = m + eps

    def filled(c):
        return np.minimum(np.maximum(c * w, lo), hi)

    c_lo, c_hi = 0.0, float((hi / w).max())
    for _ in range(200):
        mid = 0.5 * (c_lo + c_hi)
        if filled(mid).sum() < total:
            c_lo = mid
        else:
            c_hi = mid
    keep = filled(c_hi)
    base = np.floor(keep)
    rem = int(round(total - base.sum()))
    frac = keep - base
    order = sorted(range(L), key=lambda l: (-frac[l], l))
    out = base.astype(np.int64)
    for l in order[:max(rem, 0)]:
        out[l] += 1
    return out


def allocate_budgets_curve(miss_curve, grid_bp, mean_keep_bp):
    """Per-layer keep budgets from each layer's miss measured at several keeps.

    READING (an alternative to allocate_budgets) of the v3 abstract, where the
    layers' block budget follows their measured miss rates: miss_curve[l][g] is
    layer l's mean miss measured with every layer at keep grid_bp[g] (grid
    ascending).  Every layer starts at grid_bp[0]; while the total
    L * mean_keep_bp still has room for some layer's next grid step, that step
    goes to the layer whose measured miss falls the most per basis point of the
    step (a rise counts as a negative fall), ties to the lower layer.  This is
    marginal allocation: for curves convex in the keep it gives the least summed
    miss over grid points within the total.
    """
    m = np.asarray(miss_curve, dtype=np.float64)
    g = [int(x) for x in grid_bp]
    L = m.shape[0]
    room = L * int(mean_keep_bp) - L * g[0]
    pos = [0] * L
    while True:
        best, best_gain = -1, None
        for l in range(L):
            i = pos[l]
            if i + 1 >= len(g) or g[i + 1] - g[i] > room:
                continue
            gain = (m[l, i] - m[l, i + 1]) / (g[i + 1] - g[i])
            if best < 0 or gain > best_gain:
                best, best_gain = l, gain
        if best < 0:
            break
        room -= g[pos[best] + 1] - g[pos[best]]
        pos[best] += 1
    return np.array([g[i] for i in pos], dtype=np.int64)


# ---------------------------------------------------------------------------
# One decode round for one request and one layer.
# ---------------------------------------------------------------------------
class RequestState:
    """fp64 SPIN state of one (layer, request): V per slot, D per offset."""

    def __init__(self, max_ctx, request_id=0):
        self.V = np.full(max_ctx, NEG_INF)
        self.D = np.full(max_ctx, NEG_INF)
        self.step = 0
        self.request_id = request_id

    def copy(self):
        c = RequestState(len(self.V), self.request_id)
        c.V[:] = self.V
        c.D[:] = self.D
        c.step = self.step
        return c


def decode_round(state, qpos, rows, keep_bp, explore_bp, seed, layer,
                 qv, wv, key_values, page_scale, block_table, topk, alpha,
                 accepted=0, warmup_steps=1, pooling=POOL_MAX, mask=MASK_UNION):
    """predict -> index -> top-k -> update, the step order of [digest].

    Returns a dict with kept, flags, scores [R, kept*64], topk [R, K]; the
    state is updated over rows 0..accepted and its step counter advanced.
    """
    kept, flags = predict_blocks(state.V, state.D, qpos, rows, keep_bp, explore_bp,
                                 seed, layer, state.step, state.request_id,
                                 warmup_steps, pooling, mask)
    scores = indexer_scores(qv, wv, key_values, page_scale, block_table, kept, qpos)
    tk = np.stack([topk_positions(scores[r], kept, qpos + r, topk) for r in range(rows)])
    ema_update(state.V, state.D, scores, kept, qpos, accepted, alpha)
    state.step += 1
    return {"kept": kept, "flags": flags, "scores": scores, "topk": tk}


def fp8_query_operands(q, w):
    """(qv, wv) the fp8 indexer multiplies: decoded q8 codes and w * 2**e.

    q [R, H, d] (bf16 values), w [R, H] fp32.  Because 2**e > 0 and the page
    scale > 0, ReLU(2**e * scale * x) = 2**e * scale * ReLU(x): both scales
    factor out of the ReLU and the head sum.
    """
    codes, e, q8 = quantize_q(q)
    wv = np.asarray(w, dtype=np.float64) * np.exp2(e.astype(np.float64))
    return q8, wv, codes, e
