/*
 * spin.h -- C ABI of the SPIN (Shadow Predictive Indexer) decode-round library
 * for AMD Instinct MI355X (gfx950).
 *
 * SPIN predicts which KV blocks matter before the sparse-attention indexer
 * runs, so the indexer scores only the kept blocks (arXiv 2610.09025).  One
 * decode round for one layer is
 *
 *     spin_predict_blocks  -> kept block list (predicted + explored)
 *     spin_indexer_topk    -> indexer scores of the kept slots, per-row top-k
 *     spin_update          -> EMA update from the observed slots (R == 1)
 *     spin_mtp_replay      -> prefix-valid EMA replay once acceptance is known
 *
 * The selection's consumer: spin_sparse_attention (core attention over the
 * top-k).
 *
 * Measurement calls beside the round: spin_measure_miss (against an all-keep
 * top-k), spin_estimate_miss (from exploration hits alone), spin_slot_scores
 * and spin_predictor_fidelity (a slot predictor against the indexer), and the
 * host allocators spin_allocate_budgets and spin_allocate_budgets_curve.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked [host].
 *   - Every call that takes a hipStream_t enqueues its kernels on that stream
 *     and returns without synchronising.  No call allocates device memory; the
 *     caller owns every buffer, including the state buffer.
 *   - A state is used from one stream at a time: calls that overlap on one
 *     state race on its workspace.  The exceptions, which touch disjoint
 *     state regions: spin_quantize_q (writes q8, wq, qexp; ordered after the
 *     previous round's indexer, which reads them) may run beside
 *     spin_predict_blocks (V, D, VB, step, bscore, ukey) and beside the
 *     previous round's EMA update (spin_update, spin_mtp_replay or the update
 *     half of spin_topk_update: V, D, VB, step, tail_gate); spin_topk_scores
 *     (no state) may run beside spin_update / spin_mtp_replay.
 *   - Return value: SPIN_OK (0) or a negative SPIN_E* code; no C++ exception
 *     crosses this boundary.  Arguments that live in host memory are checked
 *     before anything is enqueued.  Values that live in device arrays (slot,
 *     qpos, kept lists, block tables, accepted counts) cannot be checked on the
 *     host without a synchronisation: the kernels check them, skip the
 *     offending request or entry without touching memory out of bounds, and
 *     set a bit in the state's device error word (spin_state_layout().error).
 *   - Block size is 64 slots; slot i belongs to block i / 64.  Positions are
 *     0-based; a query row at position q attends to slots 0..q (its own key
 *     is in the cache before the indexer runs).
 */
#ifndef SPIN_H
#define SPIN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SPIN_OK = 0,
  SPIN_EINVAL = -1,       /* null pointer, bad size, layer/rows out of range */
  SPIN_EUNSUPPORTED = -2, /* valid configuration this library does not build */
  SPIN_EHIP = -3,         /* a HIP launch failed; see spin_status_string */
  SPIN_ESTATE = -4,       /* state buffer too small or config mismatch */
  SPIN_ESCRATCH = -5      /* needs more than the library's static device scratch */
};

/* Bits of the device error word. */
enum {
  SPIN_ERR_QPOS = 1,      /* qpos < 0 or qpos + R - 1 >= max_ctx, or too many blocks */
  SPIN_ERR_SLOT = 2,      /* slot outside [0, max_slots) */
  SPIN_ERR_KEPT = 4,      /* kept_count or a kept block index out of range */
  SPIN_ERR_PAGE = 8,      /* block_table entry outside [0, pool_pages) */
  SPIN_ERR_ACCEPT = 16    /* accepted outside [0, R-1] */
};

/* [host] Static configuration of one state buffer. */
/* Predictor variants of the v1 listing (Figure 3 caption: Mean and Top-4
 * against Max block pooling; Table 7 and Figure 2: row-0 mask against the
 * row-local union), in spin_config.policy.  Max pooling and the union are the
 * method; the others serve ablations.
 *   SPIN_POOL_MAX   S_j = max of z over the block's existing slots
 *   SPIN_POOL_MEAN  S_j = mean of the block's finite z (never-observed slots
 *                   carry no score); -inf if none
 *   SPIN_POOL_TOP4  S_j = mean of the block's 4 largest finite z (fewer if it
 *                   has fewer); -inf if none
 *   SPIN_MASK_ROW0  with R > 1, only row 0 builds a block mask, shared by
 *                   every row; the blocks past row 0's last block (reached
 *                   only by later rows) are kept as predicted.  The row-0
 *                   EMA update is spin_update (or spin_mtp_replay with
 *                   accepted = 0). */
#define SPIN_POOL_MAX 0u
#define SPIN_POOL_MEAN 1u
#define SPIN_POOL_TOP4 2u
#define SPIN_POOL_BITS 3u
#define SPIN_MASK_ROW0 4u

typedef struct spin_config {
  int32_t num_layers;   /* layers, each with its own V/D state */
  int32_t max_slots;    /* concurrent requests (state slots) */
  int32_t max_ctx;      /* positions per request: qpos + R - 1 < max_ctx */
  int32_t block_size;   /* must be 64 */
  int32_t heads;        /* indexer heads H_I: 64 */
  int32_t head_dim;     /* indexer head dim d_I: 128 */
  int32_t topk;         /* K of the per-row top-k, 4..4096, a multiple of 4 */
  int32_t max_rows;     /* 1 + MTP draft length, 1..4 */
  int32_t warmup_steps; /* leading all-keep rounds of each (layer, request) */
  int32_t explore_bp;   /* exploration share of the kept budget, basis points */
  float alpha;          /* EMA history weight; beta = fp32(1 - alpha) */
  uint32_t policy;      /* SPIN_POOL_* | SPIN_MASK_ROW0; 0 = max pooling, row-local union */
  uint64_t seed;        /* Philox key word 0 for exploration */
} spin_config;

/* [host] One call's batch.  The [B][max_blocks] arrays of a call (block
 * tables, kept lists, flags) all use the row stride max_blocks, which must be
 * at least ceil((qpos + R) / 64) for every request and at most
 * ceil(max_ctx / 64). */
typedef struct spin_batch {
  int32_t B;              /* requests in this call, 1..max_slots */
  int32_t R;              /* query rows per request, 1..max_rows */
  int32_t max_blocks;     /* row stride of the [B][max_blocks] arrays */
  int32_t reserved;       /* must be 0 */
  const int32_t* slot;    /* device [B]: state slot of each request */
  const int32_t* qpos;    /* device [B]: position of row 0; row r is at qpos + r */
} spin_batch;

/* Byte offsets of the regions of a state buffer (for checkpoints, tests and
 * debugging).  Arrays are dense, row-major, fp32 unless noted:
 *   V   [num_layers][max_slots][max_ctx]     vertical EMA per slot (-inf = never observed)
 *   D   [num_layers][max_slots][max_ctx]     diagonal EMA per relative offset q - i
 *   VB  [num_layers][max_slots][max_blocks]  per-block max of V (a derived cache)
 *   step [num_layers][max_slots] int32       completed rounds of each (layer, slot)
 *   request_id [max_slots] uint64            Philox counter word 2
 *   error int32                              SPIN_ERR_* bits, sticky until spin_state_init
 *   tail_gate uint64                         top-k workgroups started by two-stream
 *                                            spin_topk_update calls (never reset)
 *   q8  [max_slots][max_rows][heads][head_dim] uint8   workspace: e4m3fn query codes
 *   wq  [max_slots][max_rows][heads]          workspace: w * 2^e
 *   qexp [max_slots][max_rows][heads] int32   workspace: query exponents e
 *   bscore [max_slots][max_rows][max_blocks]  workspace: block scores S (when several
 *                                            rows build their own masks, each row's
 *                                            block flags once its selection is done)
 *   ukey [max_slots][max_blocks] uint64       workspace: exploration keys
 *   page_qmax [max_slots][max_rows][max_blocks][4] workspace: per-page quarter maxima
 *   topk_ws                                   empty (= total): the state's top-k runs on
 *                                             the page quarter maxima and needs no workspace
 * Workspace arrays are indexed by batch position b, not by slot. */
typedef struct spin_state_layout {
  size_t V, D, VB, step, request_id, error, tail_gate, q8, wq, qexp, bscore, ukey, page_qmax,
      topk_ws, total;
  int32_t max_blocks;     /* ceil(max_ctx / 64) */
  int32_t reserved;
} spin_state_layout;

typedef struct spin_state spin_state; /* opaque host handle */

/* Size in bytes of the state buffer for `cfg`.  Returns SPIN_EINVAL or
 * SPIN_EUNSUPPORTED for a configuration the library does not accept. */
int spin_state_bytes(const spin_config* cfg, size_t* bytes);

/* [host] Region offsets of a state buffer for `cfg`. */
int spin_state_layout_of(const spin_config* cfg, spin_state_layout* out);

/* Bind a caller-owned device buffer of at least spin_state_bytes() bytes
 * (256-byte aligned) and enqueue its initialisation: V, D, VB := -inf (never
 * observed), step := 0, request_id := 0, error := 0.  *out receives a host
 * handle; the buffer must outlive it.  READING of the pages (SPIN's AI Radio
 * episode, "Title and authors" segment; ai4snews digest, "arXiv深度剖析"):
 * V is one EMA per slot, D one EMA per relative offset; the pages leave the
 * initial value open, and -inf marks "never observed". */
int spin_state_init(const spin_config* cfg, void* state_mem, size_t bytes,
                    hipStream_t stream, spin_state** out);

/* [host] Free the host handle only; the caller frees state_mem. */
int spin_state_destroy(spin_state* st);

/* Start new requests in `n` slots: for every layer V, D, VB := -inf,
 * step := 0, and request_id[slots[k]] := request_ids[k].
 * slots: device int32 [n]; request_ids: device uint64 [n]. */
int spin_reset_slots(spin_state* st, int n, const int32_t* slots,
                     const uint64_t* request_ids, hipStream_t stream);

/* Predict and select the kept KV blocks of one layer (AI Radio episode,
 * "Title and authors": z_{t,i} = max(V_i, D_{q_t - i}), S_{t,j} = max of z over
 * block j; "The paper's summary": a share gamma of the block budget is random
 * exploration; ai4snews digest, "arXiv深度剖析": block-level sparsity, and for
 * MTP the union of every verification row's mask).
 * For each request and row r (position q_r = qpos + r, N_r = ceil((q_r+1)/64)
 * blocks): K_b = ceil(keep_bp * N_r / 10^4), n_exp = floor(explore_bp * K_b /
 * 10^4); the K_b - n_exp blocks with the largest S (ties: lower block) are
 * predicted; among the other blocks the n_exp with the smallest Philox4x64-10
 * word (key (seed, layer), counter (j/4, step, request_id, 0), word j%4; ties:
 * lower block) are explored.  A row keeps every block when the (layer, slot)
 * is within warmup_steps, keep_bp >= 10000 or K_b >= N_r.  The kept set is the
 * union over rows.
 * keep_bp: 0..10000 (= 10000 - target sparsity in basis points).
 * Outputs: kept_blocks int32 [B][max_blocks] ascending block indices
 * (entries past kept_count are left unspecified), kept_count int32 [B],
 * block_flags uint8 [B][max_blocks] (0 skipped, 1 predicted by some row,
 * 2 explored only; 0 for blocks past the last row's context). */
int spin_predict_blocks(spin_state* st, int layer, const spin_batch* batch, int keep_bp,
                        int32_t* kept_blocks, int32_t* kept_count, uint8_t* block_flags,
                        hipStream_t stream);

/* Quantise the queries into the state's workspace: per (request, row, head),
 * e = the smallest integer with max|q| * 2^-e <= 448 (0 if q == 0), codes =
 * round-to-nearest-even e4m3fn of q * 2^-e, and wq = w * 2^e, so the indexer
 * score keeps its value (ReLU commutes with positive scales).
 * q_bf16: bf16 [B][R][heads][head_dim]; w: fp32 [B][R][heads]. */
int spin_quantize_q(spin_state* st, const spin_batch* batch, const void* q_bf16,
                    const float* w, hipStream_t stream);

/* Indexer on the kept blocks only, from the queries last quantised into the
 * workspace by spin_quantize_q for this batch (v1 abstract: the indexer scores
 * the KV cache each step; SPIN restricts it to the predicted blocks).  For
 * kept block j (page p = block_table[b][j]) and slot i = 64 j + t <= q_r:
 *   score_r(i) = k_scale[p] * sum_h wq[r][h] * max(0, sum_d q8[r][h][d] * k8[p][t][d])
 * computed with fp8 e4m3fn MFMA and fp32 accumulation.
 * k_pool: e4m3fn codes [pool_pages][64][head_dim]; k_scale: fp32 [pool_pages];
 * block_table: int32 [B][max_blocks] (logical block -> page).
 * scores: fp32 [B][R][max_blocks * 64], 16-byte aligned (SPIN_EINVAL
 * otherwise), in kept order: element k*64 + t is slot 64*kept_blocks[b][k] + t;
 * slots after the row's position get -inf; entries past the row's kept count
 * are not written.
 * page_qmax (may be NULL): fp32 [B][R][max_blocks][4], 16-byte aligned: for kept page k of
 * each row, element c = the largest score of its slots 16c .. 16c+15 (-inf if
 * all are masked); it is the optional top-k prefilter input of
 * spin_topk_scores. */
int spin_indexer_scores(spin_state* st, const spin_batch* batch, const uint8_t* k_pool,
                        const float* k_scale, int64_t pool_pages, const int32_t* block_table,
                        const int32_t* kept_blocks, const int32_t* kept_count, float* scores,
                        float* page_qmax, hipStream_t stream);

/* Bytes of caller-owned device workspace spin_topk_scores needs for this
 * batch shape and K when it is called without page quarter maxima (0 when every row
 * fits one 16384-candidate chunk). */
int spin_topk_workspace_bytes(const spin_batch* batch, int topk, size_t* bytes);

/* Per-row top-k over kept-order scores (v1 abstract: a fixed top-k goes to
 * core attention): the `topk` kept slots i <= q_r with the largest scores,
 * ties to the lower slot, written ascending to topk_out int32 [B][R][topk],
 * padded with -1.  -0.0 ranks equal to +0.0.  scores as spin_indexer_scores
 * writes them, 16-byte aligned (only slots <= q_r are read as candidates).  topk: 4..4096, a
 * multiple of 4.  page_qmax (may be NULL, else 16-byte aligned): the per-page
 * quarter maxima written by spin_indexer_scores for these scores; they belong to distinct
 * slots, so the topk-th largest of them is a lower bound of the answer's
 * smallest score, and scores below it are dropped before ranking (the result
 * is the same).
 * With page_qmax the whole top-k is one kernel and needs no workspace.
 * Without it, workspace: 256-byte aligned device memory of at least
 * spin_topk_workspace_bytes() bytes (may be NULL when the rows fit one
 * 16384-candidate chunk); its contents need no initialisation and are
 * clobbered.  batch->slot is not read. */
int spin_topk_scores(const spin_batch* batch, int topk, const float* scores,
                     const float* page_qmax, const int32_t* kept_blocks, const int32_t* kept_count,
                     int32_t* topk_out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * spin_topk_scores without a workspace argument.  The chunked path (no
 * page_qmax) keeps its survivors in a static device array of the library,
 * 32 MiB per device, held by each device the library runs on until the
 * process ends; a batch whose chunked path needs more (see
 * spin_topk_workspace_bytes) is rejected with SPIN_ESCRATCH before anything
 * is enqueued.  With page_qmax the top-k needs no scratch.  Every call on a
 * device shares that device's array: calls that overlap on one device (on
 * different streams, or from different threads) race and must not be made.
 * Results are those of spin_topk_scores. */
int spin_topk_scores_noalloc(const spin_batch* batch, int topk, const float* scores,
                             const float* page_qmax, const int32_t* kept_blocks,
                             const int32_t* kept_count, int32_t* topk_out, hipStream_t stream);

/* spin_quantize_q + spin_indexer_scores + spin_topk_scores with the state's
 * top-k K, the state's page-max and top-k workspaces.  `scores` must stay alive until spin_update / spin_mtp_replay
 * (the deferred update of the ai4snews digest, "arXiv深度剖析"). */
int spin_indexer_topk(spin_state* st, const spin_batch* batch, const void* q_bf16,
                      const float* w, const uint8_t* k_pool, const float* k_scale,
                      int64_t pool_pages, const int32_t* block_table,
                      const int32_t* kept_blocks, const int32_t* kept_count, float* scores,
                      int32_t* topk_out, hipStream_t stream);

/* EMA update from the observed slots of row 0 (AI Radio episode, "The paper's
 * summary": blocks that were skipped get no update).  For every kept slot
 * i <= qpos: V_i and D_{qpos - i} := s if never observed, else
 * alpha * x + beta * s, beta = fp32(1 - alpha); VB of the kept blocks is
 * refreshed and the (layer, slot) round counter is advanced.  Rows r > 0 of
 * the scores are ignored (with R > 1 this is the row-0 update policy). */
int spin_update(spin_state* st, int layer, const spin_batch* batch, const float* scores,
                const int32_t* kept_blocks, const int32_t* kept_count, hipStream_t stream);

/* The round's tail: spin_topk_scores (K = the state's topk, with page_qmax
 * when given, else without it, no workspace) and spin_update (accepted ==
 * NULL) or spin_mtp_replay (accepted: device int32 [B]), scheduled by the
 * library.  With update_stream NULL or equal to stream, both run on stream,
 * the update behind the top-k.  With a second stream, the top-k runs on
 * `stream` and the update on `update_stream`, beside it: update_stream first
 * waits for the work enqueued on `stream` before this call (the indexer that
 * wrote the scores), then for a gate that opens once every top-k workgroup
 * has started (a one-wave kernel polling the state's tail_gate counter, which
 * each top-k workgroup of such a call increments; the wait gives up after
 * 2 ms of device time, so it cannot hang).  The update's many small
 * workgroups therefore never take the compute units the top-k's one
 * workgroup per row needs, whatever the caller's streams do.  The top-k's
 * completion is ordered on `stream`, the update's on update_stream: the
 * next round (whose predictor reads the EMAs) must wait for both.  Results
 * are those of the two calls made one after the other.  scores and
 * page_qmax: 16-byte aligned. */
int spin_topk_update(spin_state* st, int layer, const spin_batch* batch, const float* scores,
                     const float* page_qmax, const int32_t* kept_blocks,
                     const int32_t* kept_count, int32_t* topk_out, const int32_t* accepted,
                     hipStream_t stream, hipStream_t update_stream);

/* Prefix-valid MTP replay (ai4snews digest, "arXiv深度剖析"; v1 Table 7,
 * row-local union + prefix-valid update): with a = accepted[b] in 0..R-1,
 * apply the update of rows 0..a in row order, row r observing the kept slots
 * i <= qpos + r with offsets qpos + r - i; rows above a change nothing.  Then
 * the round counter is advanced once.  accepted: device int32 [B]. */
int spin_mtp_replay(spin_state* st, int layer, const spin_batch* batch, const int32_t* accepted,
                    const float* scores, const int32_t* kept_blocks, const int32_t* kept_count,
                    hipStream_t stream);

/* Selection fidelity (v1, Table 5 caption: mean and p99 miss over eligible
 * sparse decode rows): miss[b][r] = (number of entries of the all-keep top-k
 * full_topk[b][r][:] that lie in blocks with block_flags == 0) / (number of
 * non-negative entries), 0 when there are none.  full_topk: int32
 * [B][R][topk]; block_flags: uint8 [B][max_blocks]; miss: fp32 [B][R]. */
int spin_measure_miss(const spin_batch* batch, int topk, const int32_t* full_topk,
                      const uint8_t* block_flags, float* miss, hipStream_t stream);

/* Predicted slot scores z_i = max(V_i, D_{q+r-i}) of every row (AI Radio
 * episode, "Title and authors"), the values that block pooling reduces, for
 * measuring a predictor against the indexer.  z_out: fp32
 * [B][R][batch->max_blocks * 64]; entries past q + r are -inf, never-observed
 * slots are -inf.  Requests with a bad slot or position are left untouched
 * and flagged in the state's error word. */
int spin_slot_scores(spin_state* st, int layer, const spin_batch* batch, float* z_out,
                     hipStream_t stream);

/* Online miss estimate of every row from its exploration blocks, with no
 * all-keep indexer (the miss of the v1 Table 5 caption; the random
 * exploration share of the ai4snews digest, "arXiv深度剖析").  The explored
 * blocks E (flag 2) are a uniform sample of the blocks U not predicted
 * (flag != 1) among the row's N_r blocks; S (flag 0) are skipped;
 * k_r = min(topk, q + r + 1).
 *   est[b][r][0]: walk this round's top-k topk_out[b][r][:] from the highest
 *     score down (ties to the lower position) with weight |E| per predicted
 *     slot and |U| per explored slot (each explored slot stands for |U|/|E|
 *     slots of U); the walk stops at the first entry whose running weight
 *     reaches k_r * |E|, which places the all-keep top-k threshold; with c_E
 *     explored entries up to there, est = c_E * |S| / (|E| * k_r).
 *   est[b][r][1]: the same ratio with every explored entry of the top-k (an
 *     upper bound: when top slots are skipped, lower ones fill their places).
 * Both in fp64, clamped to 1, rounded to fp32.  (0, 0) when nothing is
 * skipped; (-1, -1) when blocks are skipped but none explored; NaN for a
 * request whose qpos is negative or whose last row needs more than
 * max_blocks blocks.
 * scores: fp32 [B][R][max_blocks * 64] in kept-list layout (as written by
 * spin_indexer_scores for these kept lists); kept_blocks / kept_count: the
 * round's ascending kept lists; topk_out: int32 [B][R][topk], topk <= 4096
 * (entries < 0, past q + r, or in blocks outside the kept list are
 * ignored); block_flags: uint8 [B][max_blocks]; est: fp32 [B][R][2].
 * batch->slot is not read. */
int spin_estimate_miss(const spin_batch* batch, int topk, const float* scores,
                       const int32_t* kept_blocks, const int32_t* kept_count,
                       const int32_t* topk_out, const uint8_t* block_flags, float* est,
                       hipStream_t stream);

/* Quality of a slot predictor against the indexer (v1, Table 1: Pearson
 * correlation and top-k recall).  pred, actual: fp32
 * [B][R][batch->max_blocks * 64] slot scores; pred_topk, actual_topk: int32
 * [B][R][topk], ascending with -1 padding (as spin_topk_scores writes them).
 * out: fp64 [B][R][2] = (Pearson over the slots 0..q+r where both scores are
 * finite, computed in fp64 from the means; 0 when fewer than 2 such slots
 * remain or either side is constant on them;  recall = entries of pred_topk
 * found in actual_topk / valid entries of actual_topk, 0 if none).  NaN for a
 * request whose qpos is out of range.  batch->slot is not read. */
int spin_predictor_fidelity(const spin_batch* batch, int topk, const float* pred,
                            const float* actual, const int32_t* pred_topk,
                            const int32_t* actual_topk, double* out, hipStream_t stream);

/* [host] Workspace for spin_sparse_attention: 0 when each row runs as one
 * share of its top-k list, else the per-share partial outputs.  The share
 * count depends on the current device's compute-unit count: query it with
 * the device current that will run the call. */
int spin_attention_workspace_bytes(const spin_batch* batch, int topk, size_t* bytes);

/* Sparse core attention over each row's top-k, the consumer of the selection
 * (v1 listing, Abstract: a fixed top-k of tokens goes to core attention).
 * READING (the pages name DeepSeek-V3.2 / V4 and give no attention shape):
 * the absorbed form of multi-head latent attention, 128 query heads sharing
 * one cache row of 576 values per token (512 latent + 64 rotary), the value
 * being the row's first 512:
 *     s_h(i) = scale * q_h . c_i,   o_h = sum_i softmax_i(s_h) c_i[0:512],
 *     lse_h = log sum_i exp(s_h(i))
 * over the valid entries i of topk_idx[b][r][:] (>= 0, <= qpos + r, with a
 * block-table entry in [0, pool_pages)); the cache row of slot i is row
 * i % 64 of page block_table[b][i / 64] (the indexer's block table).
 * q_bf16: [B][R][128][576] bf16, 16-byte aligned; kv_bf16:
 * [pool_pages][64][576] bf16, 16-byte aligned; out_bf16: [B][R][128][512]
 * bf16 (RNE from fp32), 8-byte aligned; lse: fp32 [B][R][128].  Scores and
 * the softmax run in fp32 on the MFMA's fp32 sums of bf16 products; the
 * weights enter the value product as bf16.  A row with no valid entry gets
 * o = 0 and lse = -inf; a request whose qpos is negative or whose last row
 * needs more than max_blocks blocks gets o = 0 and lse = NaN.  A row may run
 * as several shares of its list whose normalised outputs (bf16) and
 * log-sum-exps are merged in fp32.  workspace:
 * 256-byte aligned, spin_attention_workspace_bytes() bytes (NULL allowed
 * when that is 0), clobbered.  topk <= 4096; batch->slot is not read. */
int spin_sparse_attention(const spin_batch* batch, int topk, const int32_t* topk_idx,
                          const void* q_bf16, const void* kv_bf16, int64_t pool_pages,
                          const int32_t* block_table, float scale, void* out_bf16, float* lse,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* [host] Per-layer keep budgets from measured miss rates (v3 abstract: the
 * block budget is allocated across layers by their measured miss rates).
 * READING: keep_l = clamp(c * (miss_l + 1e-3), mean/2, 10000) with the level
 * c found by bisection so that sum keep_l = L * mean_keep_bp, rounded to
 * integer basis points by largest remainder (ties to the lower layer).
 * miss: [host] double [L]; keep_bp_out: [host] int32 [L]. */
int spin_allocate_budgets(int L, const double* miss, int mean_keep_bp, int32_t* keep_bp_out);

/* [host] Per-layer keep budgets from each layer's miss measured at several
 * keeps (the same v3 abstract passage, read the other way: the measured miss
 * at more than one budget gives each layer's slope).
 * READING: every layer starts at grid_bp[0]; while L * mean_keep_bp has room
 * for some layer's next grid step, that step goes to the layer whose measured
 * miss falls most per basis point of the step (ties to the lower layer); the
 * result is the grid keep each layer reached.  For curves convex in the keep
 * this is the least summed miss over grid points within the total.
 * miss_curve: [host] double [L][G], miss_curve[l][g] = layer l's mean miss with
 * every layer at keep grid_bp[g], each in [0, 1]; grid_bp: [host] int32 [G],
 * strictly ascending in [0, 10000], grid_bp[0] <= mean_keep_bp; keep_bp_out:
 * [host] int32 [L].  1 <= L <= 4096, 1 <= G <= 64; SPIN_EINVAL otherwise. */
int spin_allocate_budgets_curve(int L, int G, const double* miss_curve, const int32_t* grid_bp,
                                int mean_keep_bp, int32_t* keep_bp_out);

/* [host] Static text for a status code (and the last HIP error, if any). */
const char* spin_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPIN_H */
