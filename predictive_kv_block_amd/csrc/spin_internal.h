// Host-side internals shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/spin.h"

// Device pointers and sizes of one bound state buffer.
struct SpinView {
  float* V;          // [L][S][max_ctx]
  float* D;          // [L][S][max_ctx]
  float* VB;         // [L][S][max_blocks]
  int32_t* step;     // [L][S]
  uint64_t* rid;     // [S]
  int32_t* err;      // [1]
  unsigned long long* gate;  // [1] top-k workgroups started by gated launches, ever
  uint8_t* q8;       // [S][max_rows][H][d]
  float* wq;         // [S][max_rows][H]
  int32_t* qexp;     // [S][max_rows][H]
  float* bscore;     // [S][max_rows][max_blocks]
  uint64_t* ukey;    // [S][max_blocks]
  float* pqmax;      // [S][max_rows][max_blocks][4] per-page quarter maxima of the last indexer call
  void* topk_ws;     // unused (the state's top-k runs on the quarter maxima)
  size_t topk_ws_bytes;
  int L, S, max_ctx, max_blocks, H, d, max_rows, topk, warmup, explore_bp;
  int pooling;       // SPIN_POOL_MAX / _MEAN / _TOP4
  int mask_row0;     // 1: row 0's block mask serves every row
  float alpha;
  uint64_t seed;
};

struct spin_state {
  spin_config cfg;
  spin_state_layout lay;
  char* base;
  SpinView view;
  unsigned long long gate_target;  // value of view.gate once the last gated top-k has started
  hipEvent_t tail_event;           // orders a gated update after the indexer (made on first use)
};

namespace spin {

// Candidates per top-k chunk (staged in LDS as uint32 keys).
constexpr int kChunk = 16384;

// Levels of the chunked top-k for `rows` rows of up to max_blocks * 64
// candidates, and the workspace they need (two ping-pong survivor buffers).
struct TopkPlan {
  int rows, K, levels;
  int chunks[16];
  size_t buf_elems, count_elems, bytes;
};
TopkPlan topk_plan(int rows, int max_blocks, int K);

// This device's static scratch of spin_topk_scores_noalloc and its size.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

hipError_t launch_fill_state(const SpinView& v, hipStream_t s);
hipError_t launch_reset_slots(const SpinView& v, int n, const int32_t* slots,
                              const uint64_t* rids, hipStream_t s);
hipError_t launch_predict(const SpinView& v, int layer, const spin_batch& bt, int keep_bp,
                          int32_t* kept, int32_t* kept_count, uint8_t* flags, hipStream_t s);
hipError_t launch_quantize(const SpinView& v, const spin_batch& bt, const void* q_bf16,
                           const float* w, hipStream_t s);
hipError_t launch_indexer(const SpinView& v, const spin_batch& bt, const uint8_t* k_pool,
                          const float* k_scale, int64_t pool_pages, const int32_t* table,
                          const int32_t* kept, const int32_t* kept_count, float* scores,
                          float* page_qmax, hipStream_t s);
hipError_t launch_topk(const spin_batch& bt, int topk, const float* scores, const float* page_qmax,
                       const int32_t* kept, const int32_t* kept_count, int32_t* out, void* ws,
                       hipStream_t s);
// The round's tail on two streams: the top-k launch (one workgroup per row,
// each adding 1 to `arrivals` as it starts) and a gate that waits until
// `arrivals` reaches `target`, which the update's launch then follows.
hipError_t launch_topk_gated(const spin_batch& bt, int topk, const float* scores,
                             const float* page_qmax, const int32_t* kept,
                             const int32_t* kept_count, int32_t* out,
                             unsigned long long* arrivals, hipStream_t s);
hipError_t launch_gate(const unsigned long long* arrivals, unsigned long long target,
                       hipStream_t s);
hipError_t launch_update(const SpinView& v, int layer, const spin_batch& bt,
                         const int32_t* accepted, const float* scores, const int32_t* kept,
                         const int32_t* kept_count, hipStream_t s);
hipError_t launch_miss(const spin_batch& bt, int topk, const int32_t* full_topk,
                       const uint8_t* flags, float* miss, hipStream_t s);

}  // namespace spin
