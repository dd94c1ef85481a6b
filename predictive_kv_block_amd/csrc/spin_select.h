// Workgroup-wide exact selection with lowest-index tie breaking.
//
// Given n candidates j = 0..n-1, a source that says whether j is valid and
// what its unsigned key is, and a count `want`, the selection is the `want`
// valid candidates with the largest keys, ties going to the lower index.  It is
// described by a threshold key T and a count n_eq: j is selected iff it is
// valid and (key > T, or key == T and fewer than n_eq valid candidates below j
// have key T).  T is found by MSB-first radix passes over 8-bit digits (below
// the prefix all valid keys share) with LDS histograms; the ordered pass then
// walks each wave's contiguous segment with ballots, so selected candidates
// come out in ascending index order.
#pragma once

#include "spin_device.h"

namespace spin {

// LDS scratch needed by the helpers below (ints): kSelHistCopies histograms,
// broadcast words, per-wave counts and prefixes.
constexpr int kSelHistCopies = 4;
constexpr int kSelHist = 256 * kSelHistCopies;
constexpr int kSelectScratchInts = kSelHist + 8 + 4 * 32;

// Smallest and largest key over the valid candidates (all threads get them;
// kmin > kmax when none is valid).
template <int NT, int U, typename K, typename Src>
__device__ void key_range(const Src& src, int n, K* kmin, K* kmax, int* s_scratch) {
  constexpr int NW = NT / kWave;
  K* s_lo = reinterpret_cast<K*>(s_scratch);            // uses the histogram area
  K* s_hi = s_lo + NW;
  const int tid = threadIdx.x;
  K lo = ~K(0), hi = K(0);
  for (int base = 0; base < n; base += NT * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * NT + tid;
      K key;
      if (j < n && src.get(j, key)) {
        lo = key < lo ? key : lo;
        hi = key > hi ? key : hi;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const K a = K(__shfl_xor(lo, o, kWave)), b = K(__shfl_xor(hi, o, kWave));
    lo = a < lo ? a : lo;
    hi = b > hi ? b : hi;
  }
  __syncthreads();
  if (lane_id() == 0) {
    s_lo[tid / kWave] = lo;
    s_hi[tid / kWave] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    lo = s_lo[i] < lo ? s_lo[i] : lo;
    hi = s_hi[i] > hi ? s_hi[i] : hi;
  }
  __syncthreads();
  *kmin = lo;
  *kmax = hi;
}

// Threshold of the `want` largest valid keys (0 < want <= number valid).
// Radix windows of 8 bits; for 32-bit keys they start just below the bits
// that every valid key shares (the common prefix of kmin and kmax), so
// clustered keys waste no round.  Each wave adds into one of kSelHistCopies
// histograms.
template <int NT, int U, typename K, typename Src>
__device__ void radix_threshold(const Src& src, int n, int want, K* thr_out, int* neq_out,
                                int* s_scratch) {
  static_assert(NT % kWave == 0, "whole waves");
  constexpr int KB = int(sizeof(K)) * 8;
  int* s_hist = s_scratch;
  int* s_bc = s_scratch + kSelHist;
  const int tid = threadIdx.x;
  // 32-bit keys (scores) cluster and share leading bits: start below them.
  // 64-bit keys (uniform random words) do not: start at the top.
  int hb = KB - 1;                         // highest bit where kmin and kmax differ
  K kmin = 0;
  if (sizeof(K) == 4) {
    K kmax;
    key_range<NT, U, K>(src, n, &kmin, &kmax, s_scratch);
    if (kmin >= kmax) {                    // one distinct key: the lowest-index `want`
      *thr_out = kmin;
      *neq_out = want;
      return;
    }
    while (!(((kmin ^ kmax) >> hb) & K(1))) --hb;
  }
  K mask = (hb == KB - 1) ? K(0) : ~((K(2) << hb) - K(1));
  K prefix = kmin & mask;
  int remaining = want;
  bool done = false;
  int* my_hist = s_hist + 256 * ((tid / kWave) % kSelHistCopies);
  for (int top = hb; top >= 0 && !done;) {
    const int width = top + 1 < 8 ? top + 1 : 8;
    const int shift = top + 1 - width;
    const K dmask = K((1u << width) - 1u);
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
        hist_add(my_hist, int((key[u] >> shift) & dmask), ok[u] && (key[u] & mask) == prefix);
    }
    __syncthreads();
    if (tid < kWave) {
      const int l = tid;
      if (l == 0) {
        s_bc[0] = 0;
        s_bc[1] = 0;
        s_bc[2] = 0;
      }
      int c[4], tot = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        c[b] = 0;
#pragma unroll
        for (int h = 0; h < kSelHistCopies; ++h) c[b] += s_hist[256 * h + 4 * l + b];
        tot += c[b];
      }
      int sfx = tot;  // inclusive suffix sum over lanes l..63
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_down(sfx, o, kWave);
        if (l + o < kWave) sfx += t;
      }
      const int above = sfx - tot;
      if (above < remaining && remaining <= sfx) {
        int cum = above, digit = 4 * l, at = above;
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
    mask |= dmask << shift;
    remaining -= at;
    done = bucket == remaining;        // the whole bucket is taken: stop early
    top = shift - 1;
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
