// Launchers of the sparse core attention kernels (spin_attention.hip).
#pragma once

#include <stddef.h>

#include "../../include/spin.h"

namespace spin {

// Query heads, cache row width and value width the attention kernel is built for.
constexpr int kAttnHeads = 128;
constexpr int kAttnDim = 576;
constexpr int kAttnValueDim = 512;

struct AttnPlan {
  int rows, splits, chunk;   // chunk: top-k entries per split (a multiple of 32)
  size_t ws_o_bytes, ws_bytes;
};
AttnPlan attention_plan(const spin_batch& bt, int topk);

hipError_t launch_attention(const spin_batch& bt, int topk, const int32_t* topk_idx,
                            const void* q, const void* kv, int64_t pool_pages,
                            const int32_t* table, float scale, void* out, float* lse,
                            void* ws, hipStream_t s);

}  // namespace spin
