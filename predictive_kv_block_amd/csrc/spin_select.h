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

namespace spin {

// ------------------------------------------------------------------------
// Register-resident selection: a workgroup of NT threads holds NPL keys per
// thread, element e(w, i, l) = w * (NPL * 64) + i * 64 + l (wave w owns a
// contiguous segment, in lane order within each step i), with a validity bit
// per element.  The `want` largest valid keys (ties to the lower element) are
// keys > T, or == T for the first n_eq valid elements holding T.

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts within
// each 16-lane row, then the row broadcasts of lanes 15 and 31).  Every lane
// of the wave must be active.
__device__ __forceinline__ int wave_prefix_sum(int x) {
  int s = x;
  s += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // x[l-1]
  s += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // x[l-2]
  s += __builtin_amdgcn_update_dpp(0, x, 0x113, 0xF, 0xF, true);   // x[l-3]
  s += __builtin_amdgcn_update_dpp(0, s, 0x114, 0xF, 0xE, false);  // lanes 4..15 of a row
  s += __builtin_amdgcn_update_dpp(0, s, 0x118, 0xF, 0xC, false);  // lanes 8..15 of a row
  s += __builtin_amdgcn_update_dpp(0, s, 0x142, 0xA, 0xF, false);  // rows 1, 3: + lane 15
  s += __builtin_amdgcn_update_dpp(0, s, 0x143, 0xC, 0xF, false);  // rows 2, 3: + lane 31
  return s;
}

// LDS of the register-resident threshold search: two histograms, used in turn
// by successive passes, each held as kSelCopies copies (lane l adds to copy
// l % kSelCopies; the copies of a digit are adjacent words in distinct
// banks), so that lanes sharing a digit rarely hit one address; and two
// broadcast words.
constexpr int kSelCopies = 8;
struct RegsSelectShared {
  __attribute__((aligned(16))) int hist[2][kSelHist * kSelCopies];
  int bc[2][4];
};

// Clears the first histogram; a barrier must follow before the first search.
template <int NT>
__device__ __forceinline__ void regs_select_init(RegsSelectShared& sh) {
  for (int i = threadIdx.x; i < kSelHist * kSelCopies; i += NT) sh.hist[0][i] = 0;
}

// Threshold of the `want` largest valid keys, 0 < want < number valid: MSB
// first radix digits of up to 8 bits, stopping once the threshold bucket is
// taken whole (then n_eq is unbounded, 0x7fffffff).  Given the smallest and
// largest valid key, the digits start below the bits those two share (all
// keys share them); all keys equal gives the first `want` valid elements.
// Pass p (counted over every search of the workgroup in `pass`) fills
// hist[p & 1]; wave 0 then scans it while the other waves clear
// hist[(p + 1) & 1] for the next pass.
template <int NT, int NPL, typename K>
__device__ void regs_threshold(const K (&key)[NPL], uint32_t valid, int want,
                               RegsSelectShared& sh, int& pass, K* thr_out, int* neq_out,
                               K kmin = K(0), K kmax = ~K(0)) {
  static_assert(NT > kWave, "one wave scans while the others clear");
  static_assert(NPL <= 32, "one validity bit per key");
  constexpr int kBits = int(sizeof(K)) * 8;
  const int tid = threadIdx.x, l = lane_id();
  const int copy = l & (kSelCopies - 1);
  if (kmin == kmax) {
    *thr_out = kmin;
    *neq_out = want;
    return;
  }
  const K diff = kmin ^ kmax;
  const int hb = kBits - 1 - (kBits == 64 ? __clzll(static_cast<long long>(diff))
                                          : __clz(static_cast<int>(diff)));
  K mask = hb == kBits - 1 ? K(0) : ~((K(2) << hb) - K(1));   // the shared high bits
  K prefix = kmin & mask;
  int remaining = want;
  bool done = false;
  for (int top = hb; top >= 0 && !done; ++pass) {
    const int width = top + 1 < 8 ? top + 1 : 8;
    const int shift = top + 1 - width;
    const K dmask = (K(1) << width) - K(1);
    int* h = sh.hist[pass & 1];
    int* bc = sh.bc[pass & 1];
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if ((valid >> i & 1u) != 0 && (key[i] & mask) == prefix)
        atomicAdd(&h[int((key[i] >> shift) & dmask) * kSelCopies + copy], 1);
    __syncthreads();
    if (tid < kWave) {
      // lane l holds digits 255 - 4 l .. 252 - 4 l: a prefix sum over lanes is
      // the count of keys at or above a digit
      int c[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int4* hv = reinterpret_cast<const int4*>(h + (255 - 4 * l - k) * kSelCopies);
        int t = 0;
#pragma unroll
        for (int q = 0; q < kSelCopies / 4; ++q) {
          const int4 v4 = hv[q];
          t += v4.x + v4.y + v4.z + v4.w;
        }
        c[k] = t;
      }
      const int tot = c[0] + c[1] + c[2] + c[3];
      const int incl = wave_prefix_sum(tot);
      const int above = incl - tot;
      const uint64_t hit = __ballot(above < remaining && remaining <= incl);
      const int at = __ffsll(static_cast<unsigned long long>(hit)) - 1;   // exactly one lane
      const int a1 = above + c[0], a2 = a1 + c[1], a3 = a2 + c[2];
      const int k = (a1 < remaining ? 1 : 0) + (a2 < remaining ? 1 : 0) + (a3 < remaining ? 1 : 0);
      const int cum = k == 0 ? above : (k == 1 ? a1 : (k == 2 ? a2 : a3));
      const int cnt = k == 0 ? c[0] : (k == 1 ? c[1] : (k == 2 ? c[2] : c[3]));
      if (l == at) {
        bc[0] = 255 - 4 * l - k;
        bc[1] = cum;
        bc[2] = cnt;
      }
    } else {
      int* hn = sh.hist[(pass + 1) & 1];
      for (int i = tid - kWave; i < kSelHist * kSelCopies; i += NT - kWave) hn[i] = 0;
    }
    __syncthreads();
    remaining -= bc[1];
    prefix |= K(bc[0]) << shift;
    mask |= dmask << shift;
    done = bc[2] == remaining;
    top = shift - 1;
  }
  *thr_out = prefix;
  *neq_out = done ? 0x7fffffff : remaining;
}

// Bits of the selected elements (key > thr, or == thr among the first n_eq
// valid holders of thr in element order).  s_i: NT / 64 ints.
template <int NT, int NPL, typename K>
__device__ uint32_t regs_selected(const K (&key)[NPL], uint32_t valid, K thr, int n_eq, int* s_i) {
  uint32_t sel = 0;
  if (n_eq == 0x7fffffff) {
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if ((valid >> i & 1u) && key[i] >= thr) sel |= 1u << i;
    return sel;
  }
  const int w = threadIdx.x / kWave, l = lane_id();
  int eq = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) eq += ((valid >> i & 1u) && key[i] == thr) ? 1 : 0;
  eq = wave_sum(eq);
  __syncthreads();
  if (l == 0) s_i[w] = eq;
  __syncthreads();
  int eq_base = 0;
  for (int i = 0; i < w; ++i) eq_base += s_i[i];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const bool is_eq = (valid >> i & 1u) && key[i] == thr;
    const uint64_t eqb = __ballot(is_eq);
    if (((valid >> i & 1u) && key[i] > thr) || (is_eq && eq_base + ballot_rank(eqb) < n_eq))
      sel |= 1u << i;
    eq_base += __popcll(eqb);
  }
  __syncthreads();
  return sel;
}

}  // namespace spin
