// Workgroup-wide exact selection with lowest-index tie breaking.
//
// Given n candidates j = 0..n-1, a source that says whether j is valid and
// what its unsigned key is, and a count `want`, the selection is the `want`
// valid candidates with the largest keys, ties going to the lower index.  It is
// described by a threshold key T and a count n_eq: j is selected iff it is
// valid and (key > T, or key == T and fewer than n_eq valid candidates below j
// have key T).  T is found by MSB-first radix passes over 8-bit digits with an
// LDS histogram; the ordered pass then walks each wave's contiguous segment
// with ballots, so selected candidates come out in ascending index order (or,
// without a partial tie at T, a plain marking pass takes every key >= T).
#pragma once

#include "spin_device.h"

namespace spin {

// LDS scratch needed by the helpers below (ints): histogram, broadcast words,
// per-wave counts and prefixes.
constexpr int kSelHist = 256;
constexpr int kSelectScratchInts = kSelHist + 8 + 4 * 32;

// Threshold of the `want` largest valid keys (0 < want <= number valid), by
// MSB-first rounds of 8-bit digits; the search stops early when the whole
// threshold bucket is taken.
template <int NT, int U, typename K, typename Src>
__device__ void radix_threshold(const Src& src, int n, int want, K* thr_out, int* neq_out,
                                int* s_scratch) {
  static_assert(NT % kWave == 0, "whole waves");
  int* s_hist = s_scratch;
  int* s_bc = s_scratch + kSelHist;
  const int tid = threadIdx.x;
  K prefix = 0, mask = 0;
  int remaining = want;
  bool done = false;
  for (int shift = int(sizeof(K)) * 8 - 8; shift >= 0 && !done; shift -= 8) {
    for (int i = tid; i < kSelHist; i += NT) s_hist[i] = 0;
    __syncthreads();
    for (int base = 0; base < n; base += NT * U) {
      K key[U];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = base + u * NT + tid;
        ok[u] = (j < n) && src.get(j, key[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        hist_add(s_hist, int(key[u] >> shift) & 255, ok[u] && (key[u] & mask) == prefix);
    }
    __syncthreads();
    if (tid < kWave) {
      const int l = tid;
      if (l == 0) {
        s_bc[0] = 0;
        s_bc[1] = 0;
        s_bc[2] = 0;
      }
      const int c0 = s_hist[4 * l], c1 = s_hist[4 * l + 1], c2 = s_hist[4 * l + 2],
                c3 = s_hist[4 * l + 3];
      const int tot = c0 + c1 + c2 + c3;
      int sfx = tot;  // inclusive suffix sum over lanes l..63
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_down(sfx, o, kWave);
        if (l + o < kWave) sfx += t;
      }
      const int above = sfx - tot;
      if (above < remaining && remaining <= sfx) {
        int cum = above, digit = 4 * l, at = above;
        const int c[4] = {c0, c1, c2, c3};
        for (int b = 3; b >= 0; --b) {
          if (cum + c[b] >= remaining) {
            digit = 4 * l + b;
            at = cum;
            s_bc[2] = c[b];
            break;
          }
          cum += c[b];
        }
        s_bc[0] = digit;
        s_bc[1] = at;
      }
    }
    __syncthreads();
    const int digit = s_bc[0];
    const int at = s_bc[1];
    const int bucket = s_bc[2];
    prefix |= K(digit) << shift;
    mask |= K(255) << shift;
    remaining -= at;
    done = bucket == remaining;        // the whole bucket is taken: stop early
    __syncthreads();
  }
  // With an early stop, thr is the bucket's lowest key and every key of the
  // bucket (>= thr) is taken.
  *thr_out = prefix;
  *neq_out = done ? 0x7fffffff : remaining;
}

// Ordered emission: calls emit(j, rank) for every selected j, rank being its
// position among the selected candidates in ascending j, and returns the
// number selected.  Each wave owns a contiguous segment of 64-aligned
// candidates.
template <int NT, int U, typename K, typename Src, typename Emit>
__device__ int ordered_emit(const Src& src, int n, K thr, int n_eq, const Emit& emit,
                             int* s_scratch) {
  constexpr int NW = NT / kWave;
  static_assert(NW <= 32, "at most 32 waves");
  int* s_gt = s_scratch + kSelHist + 8;
  int* s_eq = s_gt + 32;
  int* s_gtp = s_eq + 32;
  int* s_eqp = s_gtp + 32;
  const int w = threadIdx.x / kWave;
  const int l = lane_id();
  const int chunks = (n + kWave - 1) / kWave;
  const int per_wave = (chunks + NW - 1) / NW;
  const int c_begin = w * per_wave;
  const int c_end = min(chunks, c_begin + per_wave);

  int gt = 0, eq = 0;
  for (int c = c_begin; c < c_end; c += U) {
    K key[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = (c + u) * kWave + l;
      ok[u] = (c + u < c_end) && (j < n) && src.get(j, key[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      gt += (ok[u] && key[u] > thr) ? 1 : 0;
      eq += (ok[u] && key[u] == thr) ? 1 : 0;
    }
  }
  gt = wave_sum(gt);
  eq = wave_sum(eq);
  if (l == 0) {
    s_gt[w] = gt;
    s_eq[w] = eq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0, b = 0;
    for (int i = 0; i < NW; ++i) {
      s_gtp[i] = a;
      s_eqp[i] = b;
      a += s_gt[i];
      b += s_eq[i];
    }
    s_scratch[kSelHist + 2] = a + min(n_eq, b);
  }
  __syncthreads();
  const int total = s_scratch[kSelHist + 2];
  int eq_base = s_eqp[w];
  int out_base = s_gtp[w] + min(n_eq, eq_base);
  for (int c = c_begin; c < c_end; c += U) {
    K key[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = (c + u) * kWave + l;
      ok[u] = (c + u < c_end) && (j < n) && src.get(j, key[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool is_eq = ok[u] && key[u] == thr;
      const uint64_t eqb = __ballot(is_eq);
      const bool sel = (ok[u] && key[u] > thr) || (is_eq && eq_base + ballot_rank(eqb) < n_eq);
      const uint64_t selb = __ballot(sel);
      if (sel) emit((c + u) * kWave + l, out_base + ballot_rank(selb));
      eq_base += __popcll(eqb);
      out_base += __popcll(selb);
    }
  }
  __syncthreads();
  return total;
}

// Calls mark(j) for every selected j when the selection has no partial tie
// at the threshold (n_eq unbounded: every valid key >= thr), in any order.
template <int NT, int U, typename K, typename Src, typename Mark>
__device__ void mark_at_least(const Src& src, int n, K thr, const Mark& mark) {
  for (int base = 0; base < n; base += NT * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * NT + threadIdx.x;
      K key;
      if (j < n && src.get(j, key) && key >= thr) mark(j);
    }
  }
  __syncthreads();
}

// Count of valid candidates (all threads get the total).
template <int NT, int U, typename K, typename Src>
__device__ int count_valid(const Src& src, int n, int* s_scratch) {
  int* s_w = s_scratch + kSelHist + 8;
  const int tid = threadIdx.x;
  int cnt = 0;
  for (int base = 0; base < n; base += NT * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * NT + tid;
      K key;
      cnt += ((j < n) && src.get(j, key)) ? 1 : 0;
    }
  }
  cnt = wave_sum(cnt);
  if (lane_id() == 0) s_w[tid / kWave] = cnt;
  __syncthreads();
  int total = 0;
  for (int i = 0; i < NT / kWave; ++i) total += s_w[i];
  __syncthreads();
  return total;
}

}  // namespace spin
