// EMA update from the observed slots, with prefix-valid MTP replay: the work
// of one wave of k_update.
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
// Every load of a wave (V, D and each row's scores of all its blocks) is
// issued before the first EMA step, so a replay over several rows costs one
// memory latency, not one per row.  The single-row update (kReplay false) has
// no row-1..3 loads.
#pragma once

#include "spin_device.h"
#include "spin_internal.h"

namespace spin {

constexpr int kMaxRows = 4;       // query rows a batch may carry (1 + draft length)

// Request b's kept entries k0 .. k0 + NB - 1.  `lead` (one thread per request
// and call) reports bad request arguments and advances the round counter.
template <int NB, bool kReplay>
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
  const int a = kReplay && accepted ? __builtin_amdgcn_readfirstlane(accepted[b]) : 0;
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
  constexpr int RM = kReplay ? kMaxRows : 1;

  // Issue the loads of every block first.
  //   x, y      V_i and D_{q-i} of slot i = 64j + lane
  //   sv[r]     row r's score of slot i (the V chain)
  //   sd[r]     row r's score of slot i + r (the D chain of offset q - i), r >= 1
  //   yb, sb[r] the offset q - i0 of i0 = 64j - 1 - lane in a block not kept
  //             (lanes < a) and row r's score of slot i0 + r when in block j
  // With replay rows every load is unconditional (one whose value is not
  // needed reads element 0; a conditional load would make the join after it
  // wait for every load in flight), and each value is used only under the
  // condition it was loaded under.  The single-row update keeps conditional
  // loads: measured in the decode round, its unconditional form ran faster
  // alone, but the next round's indexer then took about as much longer as the
  // update saved (more of the update's written lines still on their way to
  // HBM when the key stream starts, by the look of it).
  auto ld = [](const float* p, bool ok, size_t idx, float none) {
    if (kReplay) return p[ok ? idx : 0];
    return ok ? p[idx] : none;
  };
  float x[NB], y[NB], sv[NB][RM], sd[NB][RM], yb[NB], sb[NB][RM];
  bool okb[NB], nxt[NB], prv[NB];
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const int j = jj[m + 1];
    const int k = k0 + m;
    okb[m] = k < cnt && j >= 0 && j < bt.max_blocks;
    nxt[m] = jj[m + 2] == j + 1 && k + 1 < cnt;
    prv[m] = jj[m] == j - 1 && k > 0;
    const int i = j * kBlock + l;
    const size_t here = size_t(k) * kBlock;
    x[m] = ld(V, okb[m] && i < v.max_ctx, size_t(i), -INFINITY);
    y[m] = ld(D, okb[m] && i <= q, size_t(q - i), 0.0f);
    sv[m][0] = ld(sc, okb[m], here + l, 0.0f);
    if (kReplay) {
      const int i0 = j * kBlock - 1 - l;
      const bool edge = okb[m] && !prv[m] && l < a && i0 <= q;
      yb[m] = ld(D, edge, size_t(q - i0), 0.0f);
#pragma unroll
      for (int r = 1; r < RM; ++r) {
        if (r <= a) {
          const size_t rb = size_t(r) * rstride + here;
          sv[m][r] = ld(sc, okb[m] && i <= q + r, rb + l, 0.0f);
          const int t = l + r;
          sd[m][r] = ld(sc, okb[m] && i <= q && (t < kBlock || nxt[m]), rb + t, 0.0f);
          const int tb = i0 + r - j * kBlock;
          sb[m][r] = ld(sc, edge && tb >= 0, rb + tb, 0.0f);
        }
      }
    }
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
    const int i = j * kBlock + l;

    // V of slot i, rows 0..a in order
    float xv = x[m];
    bool changed = false;
    if (i <= q) {
      xv = ema_observe(xv, sv[m][0], alpha, beta);
      changed = true;
    }
#pragma unroll
    for (int r = 1; r < RM; ++r) {
      if (r <= a && i <= q + r) {
        xv = ema_observe(xv, sv[m][r], alpha, beta);
        changed = true;
      }
    }
    if (changed && i < v.max_ctx) V[i] = xv;
    const float bmax = wave_max(i < v.max_ctx ? xv : -INFINITY);
    if (l == 0) VB[j] = bmax;

    // D at offset q - i for row-0 slot i (rows reach i + r)
    if (i <= q) {
      float yv = ema_observe(y[m], sv[m][0], alpha, beta);
#pragma unroll
      for (int r = 1; r < RM; ++r)
        if (r <= a && (l + r < kBlock || nxt[m])) yv = ema_observe(yv, sd[m][r], alpha, beta);
      D[q - i] = yv;
    }
    // offsets whose row-0 slot lies just before block j, in a block not kept
    if (kReplay && !prv[m] && l < a) {
      const int i0 = j * kBlock - 1 - l;
      if (i0 <= q) {
        float yv = yb[m];
#pragma unroll
        for (int r = 1; r < RM; ++r)
          if (r <= a && i0 + r - j * kBlock >= 0) yv = ema_observe(yv, sb[m][r], alpha, beta);
        D[q - i0] = yv;
      }
    }
  }
}

}  // namespace spin
