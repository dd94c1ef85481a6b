// EMA update from the observed slots, with prefix-valid MTP replay.
//
// One wave per kept block j (kept index k).  With a accepted drafts, rows
// 0..a are applied in row order; row r observes kept slots i <= q + r and
// updates V_i and D_{q+r-i}.
//   V: lane t owns slot 64j + t and folds the rows in order; the block's new
//      maximum refreshes VB_j.
//   D: offset o is owned by the wave of the block holding i0 = q - o (the slot
//      row 0 sees at that offset); the rows reach i0 + r, which can spill into
//      block j + 1 (read from kept index k + 1 when that block is kept).  When
//      block j - 1 is not kept, the wave of block j also owns the offsets with
//      i0 in 64j - a .. 64j - 1, whose later rows land in block j.  Each offset
//      therefore has exactly one writer and sees its rows in order.
#include "spin_device.h"
#include "spin_internal.h"

namespace spin {
namespace {

constexpr int kUpdWaves = 4;

__global__ void __launch_bounds__(kUpdWaves * kWave)
k_update(SpinView v, int layer, spin_batch bt, const int32_t* accepted, const float* scores,
         const int32_t* kept, const int32_t* kept_count) {
  const int b = blockIdx.y;
  const int lead = blockIdx.x == 0 && threadIdx.x == 0;
  const int s = bt.slot[b];
  const int q = bt.qpos[b];
  if (s < 0 || s >= v.S) {
    if (lead) flag_error(v.err, SPIN_ERR_SLOT);
    return;
  }
  if (q < 0 || q + bt.R - 1 >= v.max_ctx || num_blocks_of(q + bt.R - 1) > bt.max_blocks) {
    if (lead) flag_error(v.err, SPIN_ERR_QPOS);
    return;
  }
  const int a = accepted ? accepted[b] : 0;
  if (a < 0 || a >= bt.R) {
    if (lead) flag_error(v.err, SPIN_ERR_ACCEPT);
    return;
  }
  const int cnt = kept_count[b];
  if (cnt < 0 || cnt > bt.max_blocks) {
    if (lead) flag_error(v.err, SPIN_ERR_KEPT);
    return;
  }
  const size_t row = size_t(layer) * v.S + s;
  if (lead) v.step[row] += 1;

  const int k = blockIdx.x * kUpdWaves + threadIdx.x / kWave;
  if (k >= cnt) return;
  const size_t mb = size_t(bt.max_blocks);
  const int32_t* kb = kept + size_t(b) * mb;
  const int j = kb[k];
  if (j < 0 || j >= bt.max_blocks) {
    if (lane_id() == 0) flag_error(v.err, SPIN_ERR_KEPT);
    return;
  }
  const bool next_kept = (k + 1 < cnt) && kb[k + 1] == j + 1;
  const bool prev_kept = (k > 0) && kb[k - 1] == j - 1;

  const float alpha = v.alpha, beta = 1.0f - v.alpha;
  float* V = v.V + row * v.max_ctx;
  float* D = v.D + row * v.max_ctx;
  const int l = lane_id();
  const float* sc = scores + size_t(b) * bt.R * mb * kBlock;   // row r at + r * mb * 64
  const size_t rstride = mb * kBlock;
  const size_t here = size_t(k) * kBlock;

  // V of slot i = 64j + l.
  const int i = j * kBlock + l;
  float x = (i < v.max_ctx) ? V[i] : -INFINITY;
  bool changed = false;
  for (int r = 0; r <= a; ++r) {
    if (i <= q + r) {
      x = ema_observe(x, sc[r * rstride + here + l], alpha, beta);
      changed = true;
    }
  }
  if (changed) V[i] = x;
  const float bmax = wave_max(x);
  if (l == 0) v.VB[row * v.max_blocks + j] = bmax;

  // D at offset q - i0 for i0 = 64j + l.
  if (i <= q) {
    const int o = q - i;
    float y = D[o];
    for (int r = 0; r <= a; ++r) {
      const int t = l + r;                       // slot i + r, relative to block j
      if (t < kBlock) {
        y = ema_observe(y, sc[r * rstride + here + t], alpha, beta);
      } else if (next_kept) {
        y = ema_observe(y, sc[r * rstride + here + kBlock + (t - kBlock)], alpha, beta);
      }
    }
    D[o] = y;
  }
  // Offsets whose row-0 slot lies just before block j, in a block not kept.
  if (!prev_kept && l < a) {
    const int i0 = j * kBlock - 1 - l;
    if (i0 <= q) {
      const int o = q - i0;
      float y = D[o];
      for (int r = 0; r <= a; ++r) {
        const int t = i0 + r - j * kBlock;       // slot i0 + r, relative to block j
        if (t >= 0) y = ema_observe(y, sc[r * rstride + here + t], alpha, beta);
      }
      D[o] = y;
    }
  }
}

}  // namespace

hipError_t launch_update(const SpinView& v, int layer, const spin_batch& bt,
                         const int32_t* accepted, const float* scores, const int32_t* kept,
                         const int32_t* kept_count, hipStream_t s) {
  const dim3 grid(unsigned((bt.max_blocks + kUpdWaves - 1) / kUpdWaves), unsigned(bt.B));
  hipLaunchKernelGGL(k_update, grid, dim3(kUpdWaves * kWave), 0, s, v, layer, bt, accepted,
                     scores, kept, kept_count);
  return hipGetLastError();
}

}  // namespace spin
