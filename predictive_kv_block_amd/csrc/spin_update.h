// EMA update from the observed slots, with prefix-valid MTP replay: the work
// of one wave, shared by k_update and the top-k + update launch.
//
// A wave takes NB consecutive entries of the kept list.  With a accepted
// drafts, rows 0..a are applied in row order; row r observes kept slots
// i <= q + r and updates V_i and D_{q+r-i}.
//   V: lane t owns slot 64j + t of kept block j and folds the rows in order;
//      the block's new maximum refreshes VB_j.
//   D: offset o is owned by the wave of the block holding i0 = q - o (the slot
//      row 0 sees at that offset); the rows reach i0 + r, which can spill into
//      block j + 1 (its scores are the next kept entry when that block is
//      kept).  When block j - 1 is not kept, block j's owner also takes the
//      offsets with i0 in 64j - a .. 64j - 1, whose later rows land in block j.
//      Each offset therefore has exactly one writer and sees its rows in order.
// All loads of a wave's blocks are issued before any is used.
#pragma once

#include "spin_device.h"
#include "spin_internal.h"

namespace spin {

// Request b's kept entries k0 .. k0 + NB - 1.  `lead` (one thread per request
// and call) reports bad request arguments and advances the round counter.
template <int NB>
__device__ __forceinline__ void update_wave(const SpinView& v, int layer, const spin_batch& bt,
                                            const int32_t* accepted, const float* scores,
                                            const int32_t* kept, const int32_t* kept_count,
                                            int b, int k0, bool lead) {
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

  if (k0 >= cnt) return;
  const int l = lane_id();
  const size_t mb = size_t(bt.max_blocks);
  const int32_t* kb = kept + size_t(b) * mb;

  // kept entries k0-1 .. k0+NB (lane m holds entry k0 - 1 + m)
  int e = -2;
  if (l < NB + 2) {
    const int k = k0 - 1 + l;
    if (k >= 0 && k < cnt) e = kb[k];
  }
  int jj[NB + 2];
#pragma unroll
  for (int m = 0; m < NB + 2; ++m) jj[m] = __shfl(e, m, kWave);

  const float alpha = v.alpha, beta = 1.0f - v.alpha;
  float* V = v.V + row * v.max_ctx;
  float* D = v.D + row * v.max_ctx;
  float* VB = v.VB + row * v.max_blocks;
  const size_t rstride = mb * kBlock;
  const float* sc = scores + size_t(b) * bt.R * rstride;

  // Issue the loads of every block first.
  float x[NB], y[NB], s0[NB];
  bool okb[NB];
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const int j = jj[m + 1];
    const int k = k0 + m;
    okb[m] = k < cnt && j >= 0 && j < bt.max_blocks;
    const int i = j * kBlock + l;
    x[m] = (okb[m] && i < v.max_ctx) ? V[i] : -INFINITY;
    y[m] = (okb[m] && i <= q) ? D[q - i] : 0.0f;
    s0[m] = okb[m] ? sc[size_t(k) * kBlock + l] : 0.0f;
  }
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const int k = k0 + m;
    if (k < cnt && !okb[m] && l == 0) flag_error(v.err, SPIN_ERR_KEPT);
  }

#pragma unroll
  for (int m = 0; m < NB; ++m) {
    if (!okb[m]) continue;
    const int j = jj[m + 1];
    const int k = k0 + m;
    const bool next_kept = jj[m + 2] == j + 1 && k + 1 < cnt;
    const bool prev_kept = jj[m] == j - 1 && k > 0;
    const size_t here = size_t(k) * kBlock;
    const int i = j * kBlock + l;

    // V of slot i, rows 0..a in order (row 0's score is already loaded)
    float xv = x[m];
    bool changed = false;
    if (i <= q) {
      xv = ema_observe(xv, s0[m], alpha, beta);
      changed = true;
    }
    for (int r = 1; r <= a; ++r) {
      if (i <= q + r) {
        xv = ema_observe(xv, sc[r * rstride + here + l], alpha, beta);
        changed = true;
      }
    }
    if (changed && i < v.max_ctx) V[i] = xv;
    const float bmax = wave_max(i < v.max_ctx ? xv : -INFINITY);
    if (l == 0) VB[j] = bmax;

    // D at offset q - i for row-0 slot i (rows reach i + r)
    if (i <= q) {
      float yv = ema_observe(y[m], s0[m], alpha, beta);
      for (int r = 1; r <= a; ++r) {
        const int t = l + r;
        if (t < kBlock)
          yv = ema_observe(yv, sc[r * rstride + here + t], alpha, beta);
        else if (next_kept)
          yv = ema_observe(yv, sc[r * rstride + here + t], alpha, beta);
      }
      D[q - i] = yv;
    }
    // offsets whose row-0 slot lies just before block j, in a block not kept
    if (!prev_kept && l < a) {
      const int i0 = j * kBlock - 1 - l;
      if (i0 <= q) {
        const int o = q - i0;
        float yv = D[o];
        for (int r = 0; r <= a; ++r) {
          const int t = i0 + r - j * kBlock;
          if (t >= 0) yv = ema_observe(yv, sc[r * rstride + here + t], alpha, beta);
        }
        D[o] = yv;
      }
    }
  }
}

}  // namespace spin
