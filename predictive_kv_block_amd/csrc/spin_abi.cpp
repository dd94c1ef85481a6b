// C ABI of the SPIN library: argument checks, state layout, kernel launches.
#include <math.h>

#include <cmath>
#include <stdio.h>
#include <string.h>

#include <new>

#include "spin_attention.h"
#include "spin_fidelity.h"
#include "spin_internal.h"

namespace {

thread_local char g_status[256];

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

int check_config(const spin_config* c) {
  if (!c) return SPIN_EINVAL;
  if (c->num_layers < 1 || c->max_slots < 1 || c->max_ctx < 1 || c->max_rows < 1 ||
      c->heads < 1 || c->head_dim < 1 || c->topk < 1 || c->warmup_steps < 0 ||
      c->explore_bp < 0 || c->explore_bp > 10000 || (c->policy & ~(SPIN_POOL_BITS | SPIN_MASK_ROW0)) != 0 ||
      (c->policy & SPIN_POOL_BITS) == SPIN_POOL_BITS ||
      !(c->alpha >= 0.0f && c->alpha <= 1.0f))
    return SPIN_EINVAL;
  if (c->block_size != 64 || c->max_rows > 4 || c->topk > 4096 || c->topk % 4 != 0 ||
      c->max_ctx > (1 << 22) ||
      c->num_layers > 1024 || c->max_slots > 65535 || c->heads > 1024 || c->head_dim > 1024)
    return SPIN_EUNSUPPORTED;
  return SPIN_OK;
}

// The fp8 indexer is built for the DeepSeek indexer shape only.
bool indexer_shape_ok(const spin_state* st) {
  return st->cfg.heads == 64 && st->cfg.head_dim == 128;
}

spin_state_layout make_layout(const spin_config* c) {
  spin_state_layout l;
  memset(&l, 0, sizeof(l));
  const size_t L = size_t(c->num_layers), S = size_t(c->max_slots), C = size_t(c->max_ctx);
  const size_t MB = (C + 63) / 64, R = size_t(c->max_rows), H = size_t(c->heads),
               d = size_t(c->head_dim);
  size_t off = 0;
  l.V = off;          off = align_up(off + L * S * C * 4);
  l.D = off;          off = align_up(off + L * S * C * 4);
  l.VB = off;         off = align_up(off + L * S * MB * 4);
  l.step = off;       off = align_up(off + L * S * 4);
  l.request_id = off; off = align_up(off + S * 8);
  l.error = off;      off = align_up(off + 4);
  l.tail_gate = off;  off = align_up(off + 8);
  l.q8 = off;         off = align_up(off + S * R * H * d);
  l.wq = off;         off = align_up(off + S * R * H * 4);
  l.qexp = off;       off = align_up(off + S * R * H * 4);
  l.bscore = off;     off = align_up(off + S * R * MB * 4);
  l.ukey = off;       off = align_up(off + S * MB * 8);
  l.page_qmax = off;   off = align_up(off + S * R * MB * 16);
  l.topk_ws = off;     // empty: with page maxima the top-k needs no workspace
  l.total = off;
  l.max_blocks = int32_t(MB);
  return l;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return SPIN_OK;
  snprintf(g_status, sizeof(g_status), "HIP error: %s", hipGetErrorString(e));
  return SPIN_EHIP;
}

int check_batch(const spin_state* st, const spin_batch* bt) {
  if (!st || !bt || !bt->slot || !bt->qpos) return SPIN_EINVAL;
  if (bt->B < 1 || bt->B > st->cfg.max_slots || bt->R < 1 || bt->R > st->cfg.max_rows ||
      bt->max_blocks < 1 || bt->max_blocks > st->lay.max_blocks || bt->reserved != 0)
    return SPIN_EINVAL;
  return SPIN_OK;
}

int check_plain_batch(const spin_batch* bt) {
  if (!bt || !bt->qpos) return SPIN_EINVAL;
  if (bt->B < 1 || bt->B > 65535 || bt->R < 1 || bt->R > 4 || bt->max_blocks < 1 ||
      bt->max_blocks > (1 << 16) || bt->B * bt->R > 65535 || bt->reserved != 0)
    return SPIN_EINVAL;
  return SPIN_OK;
}

}  // namespace

extern "C" {

int spin_state_bytes(const spin_config* cfg, size_t* bytes) {
  if (!bytes) return SPIN_EINVAL;
  const int rc = check_config(cfg);
  if (rc) return rc;
  *bytes = make_layout(cfg).total;
  return SPIN_OK;
}

int spin_state_layout_of(const spin_config* cfg, spin_state_layout* out) {
  if (!out) return SPIN_EINVAL;
  const int rc = check_config(cfg);
  if (rc) return rc;
  *out = make_layout(cfg);
  return SPIN_OK;
}

int spin_state_init(const spin_config* cfg, void* state_mem, size_t bytes, hipStream_t stream,
                    spin_state** out) {
  if (!out || !state_mem) return SPIN_EINVAL;
  const int rc = check_config(cfg);
  if (rc) return rc;
  if (reinterpret_cast<uintptr_t>(state_mem) % 256 != 0) return SPIN_EINVAL;
  const spin_state_layout lay = make_layout(cfg);
  if (bytes < lay.total) return SPIN_ESTATE;
  spin_state* st = new (std::nothrow) spin_state;
  if (!st) return SPIN_EINVAL;
  st->cfg = *cfg;
  st->lay = lay;
  st->base = static_cast<char*>(state_mem);
  SpinView& v = st->view;
  v.V = reinterpret_cast<float*>(st->base + lay.V);
  v.D = reinterpret_cast<float*>(st->base + lay.D);
  v.VB = reinterpret_cast<float*>(st->base + lay.VB);
  v.step = reinterpret_cast<int32_t*>(st->base + lay.step);
  v.rid = reinterpret_cast<uint64_t*>(st->base + lay.request_id);
  v.err = reinterpret_cast<int32_t*>(st->base + lay.error);
  v.gate = reinterpret_cast<unsigned long long*>(st->base + lay.tail_gate);
  st->gate_target = 0;
  st->tail_event = nullptr;
  v.q8 = reinterpret_cast<uint8_t*>(st->base + lay.q8);
  v.wq = reinterpret_cast<float*>(st->base + lay.wq);
  v.qexp = reinterpret_cast<int32_t*>(st->base + lay.qexp);
  v.bscore = reinterpret_cast<float*>(st->base + lay.bscore);
  v.ukey = reinterpret_cast<uint64_t*>(st->base + lay.ukey);
  v.pqmax = reinterpret_cast<float*>(st->base + lay.page_qmax);
  v.topk_ws = nullptr;
  v.topk_ws_bytes = 0;
  v.L = cfg->num_layers;
  v.S = cfg->max_slots;
  v.max_ctx = cfg->max_ctx;
  v.max_blocks = lay.max_blocks;
  v.H = cfg->heads;
  v.d = cfg->head_dim;
  v.max_rows = cfg->max_rows;
  v.topk = cfg->topk;
  v.warmup = cfg->warmup_steps;
  v.explore_bp = cfg->explore_bp;
  v.pooling = int(cfg->policy & SPIN_POOL_BITS);
  v.mask_row0 = (cfg->policy & SPIN_MASK_ROW0) ? 1 : 0;
  v.alpha = cfg->alpha;
  v.seed = cfg->seed;
  const int hr = hip_status(spin::launch_fill_state(v, stream));
  if (hr) {
    delete st;
    return hr;
  }
  *out = st;
  return SPIN_OK;
}

int spin_state_destroy(spin_state* st) {
  if (!st) return SPIN_EINVAL;
  if (st->tail_event) (void)hipEventDestroy(st->tail_event);
  delete st;
  return SPIN_OK;
}

int spin_reset_slots(spin_state* st, int n, const int32_t* slots, const uint64_t* request_ids,
                     hipStream_t stream) {
  if (!st || n < 0 || n > 65535 || (n > 0 && (!slots || !request_ids))) return SPIN_EINVAL;
  return hip_status(spin::launch_reset_slots(st->view, n, slots, request_ids, stream));
}

int spin_predict_blocks(spin_state* st, int layer, const spin_batch* batch, int keep_bp,
                        int32_t* kept_blocks, int32_t* kept_count, uint8_t* block_flags,
                        hipStream_t stream) {
  int rc = check_batch(st, batch);
  if (rc) return rc;
  if (layer < 0 || layer >= st->cfg.num_layers || keep_bp < 0 || keep_bp > 10000 ||
      !kept_blocks || !kept_count || !block_flags)
    return SPIN_EINVAL;
  return hip_status(spin::launch_predict(st->view, layer, *batch, keep_bp, kept_blocks,
                                         kept_count, block_flags, stream));
}

int spin_quantize_q(spin_state* st, const spin_batch* batch, const void* q_bf16, const float* w,
                    hipStream_t stream) {
  int rc = check_batch(st, batch);
  if (rc) return rc;
  if (!q_bf16 || !w) return SPIN_EINVAL;
  if (!indexer_shape_ok(st)) return SPIN_EUNSUPPORTED;
  return hip_status(spin::launch_quantize(st->view, *batch, q_bf16, w, stream));
}

int spin_indexer_scores(spin_state* st, const spin_batch* batch, const uint8_t* k_pool,
                        const float* k_scale, int64_t pool_pages, const int32_t* block_table,
                        const int32_t* kept_blocks, const int32_t* kept_count, float* scores,
                        float* page_qmax, hipStream_t stream) {
  int rc = check_batch(st, batch);
  if (rc) return rc;
  if (!k_pool || !k_scale || pool_pages < 1 || pool_pages > (int64_t(1) << 31) || !block_table ||
      !kept_blocks || !kept_count || !scores)
    return SPIN_EINVAL;
  if (reinterpret_cast<uintptr_t>(scores) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(page_qmax) % 16 != 0)
    return SPIN_EINVAL;
  if (!indexer_shape_ok(st)) return SPIN_EUNSUPPORTED;
  return hip_status(spin::launch_indexer(st->view, *batch, k_pool, k_scale, pool_pages,
                                         block_table, kept_blocks, kept_count, scores, page_qmax,
                                         stream));
}

int spin_topk_workspace_bytes(const spin_batch* batch, int topk, size_t* bytes) {
  int rc = check_plain_batch(batch);
  if (rc) return rc;
  if (!bytes || topk < 1 || topk > 4096 || topk % 4 != 0) return SPIN_EINVAL;
  *bytes = spin::topk_plan(batch->B * batch->R, batch->max_blocks, topk).bytes;
  return SPIN_OK;
}

int spin_topk_scores(const spin_batch* batch, int topk, const float* scores,
                     const float* page_qmax, const int32_t* kept_blocks, const int32_t* kept_count,
                     int32_t* topk_out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  int rc = check_plain_batch(batch);
  if (rc) return rc;
  if (topk < 1 || topk > 4096 || topk % 4 != 0 || !scores || !kept_blocks || !kept_count ||
      !topk_out)
    return SPIN_EINVAL;
  if (reinterpret_cast<uintptr_t>(scores) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(page_qmax) % 16 != 0)
    return SPIN_EINVAL;
  const spin::TopkPlan p = spin::topk_plan(batch->B * batch->R, batch->max_blocks, topk);
  if (!page_qmax && p.levels > 1 && (!workspace || workspace_bytes < p.bytes))
    return SPIN_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return SPIN_EINVAL;
  return hip_status(spin::launch_topk(*batch, topk, scores, page_qmax, kept_blocks, kept_count,
                                      topk_out, workspace, stream));
}

int spin_topk_scores_noalloc(const spin_batch* batch, int topk, const float* scores,
                             const float* page_qmax, const int32_t* kept_blocks,
                             const int32_t* kept_count, int32_t* topk_out, hipStream_t stream) {
  int rc = check_plain_batch(batch);
  if (rc) return rc;
  if (topk < 1 || topk > 4096 || topk % 4 != 0 || !scores || !kept_blocks || !kept_count ||
      !topk_out)
    return SPIN_EINVAL;
  if (reinterpret_cast<uintptr_t>(scores) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(page_qmax) % 16 != 0)
    return SPIN_EINVAL;
  void* ws = nullptr;
  size_t cap = 0;
  rc = hip_status(spin::noalloc_scratch(&ws, &cap));
  if (rc) return rc;
  const spin::TopkPlan p = spin::topk_plan(batch->B * batch->R, batch->max_blocks, topk);
  if (!page_qmax && p.levels > 1 && p.bytes > cap) {
    snprintf(g_status, sizeof(g_status),
             "spin_topk_scores_noalloc: this batch needs %zu bytes of scratch, more than the "
             "%zu bytes of the library's static scratch",
             p.bytes, cap);
    return SPIN_ESCRATCH;
  }
  return hip_status(spin::launch_topk(*batch, topk, scores, page_qmax, kept_blocks, kept_count,
                                      topk_out, ws, stream));
}

int spin_indexer_topk(spin_state* st, const spin_batch* batch, const void* q_bf16, const float* w,
                      const uint8_t* k_pool, const float* k_scale, int64_t pool_pages,
                      const int32_t* block_table, const int32_t* kept_blocks,
                      const int32_t* kept_count, float* scores, int32_t* topk_out,
                      hipStream_t stream) {
  int rc = check_batch(st, batch);
  if (rc) return rc;
  if (!topk_out) return SPIN_EINVAL;
  if (!indexer_shape_ok(st)) return SPIN_EUNSUPPORTED;
  rc = spin_quantize_q(st, batch, q_bf16, w, stream);
  if (rc) return rc;
  rc = spin_indexer_scores(st, batch, k_pool, k_scale, pool_pages, block_table, kept_blocks,
                           kept_count, scores, st->view.pqmax, stream);
  if (rc) return rc;
  return spin_topk_scores(batch, st->cfg.topk, scores, st->view.pqmax, kept_blocks, kept_count,
                          topk_out, nullptr, 0, stream);
}

int spin_update(spin_state* st, int layer, const spin_batch* batch, const float* scores,
                const int32_t* kept_blocks, const int32_t* kept_count, hipStream_t stream) {
  int rc = check_batch(st, batch);
  if (rc) return rc;
  if (layer < 0 || layer >= st->cfg.num_layers || !scores || !kept_blocks || !kept_count)
    return SPIN_EINVAL;
  return hip_status(spin::launch_update(st->view, layer, *batch, nullptr, scores, kept_blocks,
                                        kept_count, stream));
}

int spin_topk_update(spin_state* st, int layer, const spin_batch* batch, const float* scores,
                     const float* page_qmax, const int32_t* kept_blocks,
                     const int32_t* kept_count, int32_t* topk_out, const int32_t* accepted,
                     hipStream_t stream, hipStream_t update_stream) {
  int rc = check_batch(st, batch);
  if (rc) return rc;
  if (layer < 0 || layer >= st->cfg.num_layers || !scores || !kept_blocks || !kept_count ||
      !topk_out)
    return SPIN_EINVAL;
  if (reinterpret_cast<uintptr_t>(scores) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(page_qmax) % 16 != 0)
    return SPIN_EINVAL;
  const spin_batch& bt = *batch;
  const int K = st->cfg.topk;
  if (update_stream == nullptr || update_stream == stream) {
    // one stream: the top-k, then the update behind it
    rc = hip_status(spin::launch_topk_gated(bt, K, scores, page_qmax, kept_blocks, kept_count,
                                            topk_out, nullptr, stream));
    if (rc) return rc;
    return hip_status(spin::launch_update(st->view, layer, bt, accepted, scores, kept_blocks,
                                          kept_count, stream));
  }
  if (!st->tail_event) {
    rc = hip_status(hipEventCreateWithFlags(&st->tail_event, hipEventDisableTiming));
    if (rc) return rc;
  }
  // the update's stream waits for what `stream` did before this call (the
  // indexer), then for the gate that opens once every top-k workgroup runs
  rc = hip_status(hipEventRecord(st->tail_event, stream));
  if (rc) return rc;
  rc = hip_status(spin::launch_topk_gated(bt, K, scores, page_qmax, kept_blocks, kept_count,
                                          topk_out, st->view.gate, stream));
  if (rc) return rc;
  st->gate_target += static_cast<unsigned long long>(bt.B) * bt.R;
  rc = hip_status(hipStreamWaitEvent(update_stream, st->tail_event, 0));
  if (rc) return rc;
  rc = hip_status(spin::launch_gate(st->view.gate, st->gate_target, update_stream));
  if (rc) return rc;
  return hip_status(spin::launch_update(st->view, layer, bt, accepted, scores, kept_blocks,
                                        kept_count, update_stream));
}

int spin_mtp_replay(spin_state* st, int layer, const spin_batch* batch, const int32_t* accepted,
                    const float* scores, const int32_t* kept_blocks, const int32_t* kept_count,
                    hipStream_t stream) {
  int rc = check_batch(st, batch);
  if (rc) return rc;
  if (layer < 0 || layer >= st->cfg.num_layers || !accepted || !scores || !kept_blocks ||
      !kept_count)
    return SPIN_EINVAL;
  return hip_status(spin::launch_update(st->view, layer, *batch, accepted, scores, kept_blocks,
                                        kept_count, stream));
}

int spin_measure_miss(const spin_batch* batch, int topk, const int32_t* full_topk,
                      const uint8_t* block_flags, float* miss, hipStream_t stream) {
  if (!batch || batch->B < 1 || batch->R < 1 || batch->R > 4 || batch->max_blocks < 1 ||
      topk < 1 || topk > 65536 || !full_topk || !block_flags || !miss)
    return SPIN_EINVAL;
  return hip_status(spin::launch_miss(*batch, topk, full_topk, block_flags, miss, stream));
}

int spin_slot_scores(spin_state* st, int layer, const spin_batch* batch, float* z_out,
                     hipStream_t stream) {
  int rc = check_batch(st, batch);
  if (rc) return rc;
  if (layer < 0 || layer >= st->cfg.num_layers || !z_out) return SPIN_EINVAL;
  return hip_status(spin::launch_slot_scores(st->view, layer, *batch, z_out, stream));
}

int spin_estimate_miss(const spin_batch* batch, int topk, const float* scores,
                       const int32_t* kept_blocks, const int32_t* kept_count,
                       const int32_t* topk_out, const uint8_t* block_flags, float* est,
                       hipStream_t stream) {
  int rc = check_plain_batch(batch);
  if (rc) return rc;
  if (topk < 1 || topk > 4096 || !scores || !kept_blocks || !kept_count || !topk_out ||
      !block_flags || !est)
    return SPIN_EINVAL;
  return hip_status(spin::launch_estimate_miss(*batch, topk, scores, kept_blocks, kept_count,
                                               topk_out, block_flags, est, stream));
}

int spin_predictor_fidelity(const spin_batch* batch, int topk, const float* pred,
                            const float* actual, const int32_t* pred_topk,
                            const int32_t* actual_topk, double* out, hipStream_t stream) {
  int rc = check_plain_batch(batch);
  if (rc) return rc;
  if (topk < 1 || topk > 65536 || !pred || !actual || !pred_topk || !actual_topk || !out)
    return SPIN_EINVAL;
  return hip_status(spin::launch_predictor_fidelity(*batch, topk, pred, actual, pred_topk,
                                                    actual_topk, out, stream));
}

int spin_attention_workspace_bytes(const spin_batch* batch, int topk, size_t* bytes) {
  int rc = check_plain_batch(batch);
  if (rc) return rc;
  if (!bytes || topk < 1 || topk > 4096) return SPIN_EINVAL;
  *bytes = spin::attention_plan(*batch, topk).ws_bytes;
  return SPIN_OK;
}

int spin_sparse_attention(const spin_batch* batch, int topk, const int32_t* topk_idx,
                          const void* q_bf16, const void* kv_bf16, int64_t pool_pages,
                          const int32_t* block_table, float scale, void* out_bf16, float* lse,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_plain_batch(batch);
  if (rc) return rc;
  if (topk < 1 || topk > 4096 || !topk_idx || !q_bf16 || !kv_bf16 || !block_table ||
      !out_bf16 || !lse || pool_pages < 1 || pool_pages > (int64_t(1) << 25) ||
      !std::isfinite(scale))
    return SPIN_EINVAL;
  if (reinterpret_cast<uintptr_t>(q_bf16) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(kv_bf16) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(out_bf16) % 8 != 0 || reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return SPIN_EINVAL;
  const spin::AttnPlan p = spin::attention_plan(*batch, topk);
  if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes ||
                         reinterpret_cast<uintptr_t>(workspace) % 256 != 0))
    return SPIN_EINVAL;
  return hip_status(spin::launch_attention(*batch, topk, topk_idx, q_bf16, kv_bf16, pool_pages,
                                           block_table, scale, out_bf16, lse, workspace, stream));
}

int spin_allocate_budgets(int L, const double* miss, int mean_keep_bp, int32_t* keep_bp_out) {
  if (L < 1 || L > 4096 || !miss || !keep_bp_out || mean_keep_bp < 0 || mean_keep_bp > 10000)
    return SPIN_EINVAL;
  for (int l = 0; l < L; ++l)
    if (!(miss[l] >= 0.0 && miss[l] <= 1.0)) return SPIN_EINVAL;
  const double total = double(L) * mean_keep_bp;
  const double lo = mean_keep_bp / 2.0, hi = 10000.0, eps = 1e-3;
  double* w = new (std::nothrow) double[L];
  double* keep = new (std::nothrow) double[L];
  int* order = new (std::nothrow) int[L];
  if (!w || !keep || !order) {
    delete[] w;
    delete[] keep;
    delete[] order;
    return SPIN_EINVAL;
  }
  double cmax = 0.0;
  for (int l = 0; l < L; ++l) {
    w[l] = miss[l] + eps;
    if (hi / w[l] > cmax) cmax = hi / w[l];
  }
  auto filled_sum = [&](double c) {
    double s = 0.0;
    for (int l = 0; l < L; ++l) s += fmin(fmax(c * w[l], lo), hi);
    return s;
  };
  double c_lo = 0.0, c_hi = cmax;
  for (int it = 0; it < 200; ++it) {
    const double mid = 0.5 * (c_lo + c_hi);
    if (filled_sum(mid) < total)
      c_lo = mid;
    else
      c_hi = mid;
  }
  double base_sum = 0.0;
  for (int l = 0; l < L; ++l) {
    keep[l] = fmin(fmax(c_hi * w[l], lo), hi);
    base_sum += floor(keep[l]);
    order[l] = l;
  }
  // order layers by descending fractional part, ties to the lower layer
  for (int a = 1; a < L; ++a) {
    const int x = order[a];
    const double fx = keep[x] - floor(keep[x]);
    int p = a - 1;
    while (p >= 0) {
      const int y = order[p];
      const double fy = keep[y] - floor(keep[y]);
      if (fy > fx || (fy == fx && y < x)) break;
      order[p + 1] = y;
      --p;
    }
    order[p + 1] = x;
  }
  const long rem = lround(total - base_sum);
  for (int l = 0; l < L; ++l) keep_bp_out[l] = int32_t(floor(keep[l]));
  for (long t = 0; t < rem && t < L; ++t) keep_bp_out[order[t]] += 1;
  delete[] w;
  delete[] keep;
  delete[] order;
  return SPIN_OK;
}

int spin_allocate_budgets_curve(int L, int G, const double* miss_curve, const int32_t* grid_bp,
                                int mean_keep_bp, int32_t* keep_bp_out) {
  if (L < 1 || L > 4096 || G < 1 || G > 64 || !miss_curve || !grid_bp || !keep_bp_out ||
      mean_keep_bp < 0 || mean_keep_bp > 10000)
    return SPIN_EINVAL;
  for (int g = 0; g < G; ++g)
    if (grid_bp[g] < 0 || grid_bp[g] > 10000 || (g > 0 && grid_bp[g] <= grid_bp[g - 1]))
      return SPIN_EINVAL;
  if (grid_bp[0] > mean_keep_bp) return SPIN_EINVAL;
  for (long i = 0; i < long(L) * G; ++i)
    if (!(miss_curve[i] >= 0.0 && miss_curve[i] <= 1.0)) return SPIN_EINVAL;
  // every layer starts at the lowest grid keep; each pass hands the next grid
  // step to the layer whose miss falls most per basis point, among the steps
  // that still fit in the total (ties to the lower layer)
  int* pos = new (std::nothrow) int[L];
  if (!pos) return SPIN_EINVAL;
  for (int l = 0; l < L; ++l) pos[l] = 0;
  long room = long(L) * mean_keep_bp - long(L) * grid_bp[0];
  for (;;) {
    int best = -1;
    double best_gain = 0.0;
    for (int l = 0; l < L; ++l) {
      const int i = pos[l];
      if (i + 1 >= G) continue;
      const int step = grid_bp[i + 1] - grid_bp[i];
      if (step > room) continue;
      const double gain =
          (miss_curve[long(l) * G + i] - miss_curve[long(l) * G + i + 1]) / double(step);
      if (best < 0 || gain > best_gain) {
        best = l;
        best_gain = gain;
      }
    }
    if (best < 0) break;
    room -= grid_bp[pos[best] + 1] - grid_bp[pos[best]];
    ++pos[best];
  }
  for (int l = 0; l < L; ++l) keep_bp_out[l] = grid_bp[pos[l]];
  delete[] pos;
  return SPIN_OK;
}

const char* spin_status_string(int status) {
  switch (status) {
    case SPIN_OK: return "ok";
    case SPIN_EINVAL: return "invalid argument";
    case SPIN_EUNSUPPORTED: return "unsupported configuration (block 64, 64 heads x 128, rows <= 4)";
    case SPIN_EHIP: return g_status[0] ? g_status : "HIP error";
    case SPIN_ESTATE: return "state buffer too small or mismatched";
    case SPIN_ESCRATCH:
      return g_status[0] ? g_status : "the call needs more than the library's static scratch";
    default: return "unknown status";
  }
}

}  // extern "C"
