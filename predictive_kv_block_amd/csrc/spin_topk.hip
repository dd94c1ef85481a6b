// Per-row top-k over the kept-order indexer scores, and the miss measurement.
//
// Candidates of a row are the kept slots at or before its position, in kept
// order (= ascending position).  The selection is exact, with ties to the
// lower position.
//
// With the indexer's per-page quarter maxima (the largest score of each
// 16-slot quarter of a page), k_topk_fused answers every row in one launch
// (one workgroup per row): t1 = the K-th largest of the pages' top quarter
// maxima.  Those are scores of distinct slots, so the row's K-th largest score
// is >= t1 and every score < t1 can be dropped; only 16-slot quarters whose
// maximum is >= t1 can hold such scores.  Those quarters are read, their
// scores >= t1 gathered in position order and ranked exactly.  A row that does not fit
// those buffers is walked in chunks by the same workgroup, keeping a running
// top-K.
//
// Without page maxima, the chunked levels (k_topk_level):
// 1. level 0: the row is cut into chunks of kChunk; each chunk's candidates
//    are held in registers (wave w owns a contiguous segment, lane l every
//    64th element of it).  If at most K survive, all of them pass on;
//    otherwise the chunk's local top-K is found by an MSB-first radix select
//    over LDS histograms.  Every element of the row's top-K is in its chunk's
//    local top-K, so nothing of the answer is lost.  Survivors are written in
//    position order, K slots per chunk.
// 2. Further levels repeat this over the survivors until one chunk remains;
//    that level writes the answer ascending, padded with -1.
//
// k_miss: share of an all-keep top-k that falls in skipped blocks.
#include <atomic>

#include "spin_device.h"
#include "spin_internal.h"
#include "spin_select.h"

namespace spin {
namespace {

constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kSeg = kChunk / kTopkWaves;            // 2048 keys per wave
constexpr int kPerLane = kSeg / kWave;               // 32 keys per lane

struct LevelArgs {
  spin_batch bt;
  int K;
  // level 0 input
  const float* scores;
  const int32_t* kept;
  const int32_t* kept_count;
  // later levels' input: survivors of the previous level
  const uint32_t* in_keys;    // [rows][in_chunks * K]
  const int32_t* in_pos;      // [rows][in_chunks * K]
  const int32_t* in_counts;   // [rows][in_chunks]
  int in_chunks;
  // output
  uint32_t* out_keys;         // [rows][out_chunks * K]
  int32_t* out_pos;
  int32_t* out_counts;        // [rows][out_chunks]
  int out_chunks;
  int32_t* topk_out;          // final level: [rows][K]
};

constexpr int kMaxWaves = 16;

struct TopkShared {
  RegsSelectShared sel;
  int wave_a[kMaxWaves], wave_b[kMaxWaves];
  uint32_t wave_min[kMaxWaves], wave_max[kMaxWaves];
  int bc[4];
};

// Workgroup totals over register-held keys (0 = not a candidate): the number
// of candidates and their smallest and largest key.  NT threads, NPL keys each.
template <int NT, int NPL>
__device__ void block_key_stats(const uint32_t* key, TopkShared& sh, int* total, uint32_t* kmin,
                                uint32_t* kmax) {
  constexpr int NW = NT / kWave;
  const int w = threadIdx.x / kWave, l = lane_id();
  int n = 0;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    n += key[i] != 0u;
    if (key[i] != 0u) {
      lo = min(lo, key[i]);
      hi = max(hi, key[i]);
    }
  }
  n = wave_sum(n);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, uint32_t(__shfl_xor(int(lo), o, kWave)));
    hi = max(hi, uint32_t(__shfl_xor(int(hi), o, kWave)));
  }
  __syncthreads();
  if (l == 0) {
    sh.wave_a[w] = n;
    sh.wave_min[w] = lo;
    sh.wave_max[w] = hi;
  }
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    t += sh.wave_a[i];
    lo = min(lo, sh.wave_min[i]);
    hi = max(hi, sh.wave_max[i]);
  }
  *total = t;
  *kmin = lo;
  *kmax = hi;
}

// Threshold of the `want` largest register-held keys (0 < want < total, key 0
// = not a candidate): selected = key > thr, or key == thr for the first n_eq
// in index order (n_eq unbounded when the whole threshold bucket is taken).
// kmin and kmax are the smallest and largest candidate keys.
template <int NT, int NPL>
__device__ void radix_select_regs(const uint32_t* key, int want, uint32_t kmin, uint32_t kmax,
                                  TopkShared& sh, uint32_t* thr_out, int* n_eq_out) {
  uint32_t k[NPL];
  uint32_t valid = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    k[i] = key[i];
    valid |= (key[i] != 0u) ? (1u << i) : 0u;
  }
  int pass = 0;
  __syncthreads();                       // earlier readers of the histograms are done
  regs_select_init<NT>(sh.sel);
  __syncthreads();
  regs_threshold<NT, NPL, uint32_t>(k, valid, want, sh.sel, pass, thr_out, n_eq_out, kmin, kmax);
}

// ---------------------------------------------------------------- fused row
constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / kWave;
constexpr int kFusedPageLanes = 16;                          // page maxima per lane
constexpr int kFusedMaxPages = kFusedThreads * kFusedPageLanes;   // 16384
constexpr int kFusedCandQ = 8192;
                            // listed candidate quarters
constexpr int kFusedCap = 8192;                              // survivors held in LDS
constexpr int kFusedPerLane = kFusedCap / kFusedThreads;     // 8

constexpr int kFusedBatch = 256;                             // quarters per wave step
static_assert(kFusedBatch % 16 == 0 && kFusedBatch <= 256, "16 quarters per load");

struct FusedShared {
  TopkShared t;
  int cq[kFusedCandQ];            // candidate quarters (4 kept index + quarter), ascending
  int qcount[kFusedCandQ];        // survivors per candidate quarter, then their offsets
  uint32_t skey[kFusedCap];       // survivors in position order
  int spos[kFusedCap];
  int scan[kFusedWaves];
  int wcount[kFusedWaves];        // survivors found by each wave
};

// Inverse of ord_key for keys of non-NaN floats (the key of +0 gives +0).
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Inclusive prefix sum within each 16-lane row of the wave (DPP row shifts;
// lanes shifted in from outside the row read 0).
__device__ __forceinline__ int row_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  return x;
}

// Inclusive prefix sum over the 64 lanes of the wave in lane order: the row
// sums, then the last lane of row 0 added into rows 1 and 3 and the last lane
// of row 1 into rows 2 and 3 (DPP row broadcasts; lanes of other rows add 0).
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x = row_inclusive_sum(x);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return x;
}

// Exclusive prefix sum over n <= kFusedCandQ ints in LDS; returns the total.
__device__ __forceinline__ int block_exclusive_scan(int* v, int n, int* wave_tot) {
  constexpr int per = kFusedCandQ / kFusedThreads;             // 8
  const int tid = threadIdx.x, w = tid / kWave, l = lane_id();
  int loc[per], sum = 0;
#pragma unroll
  for (int k = 0; k < per; ++k) {
    const int i = tid * per + k;
    loc[k] = (i < n) ? v[i] : 0;
    sum += loc[k];
  }
  int inc = sum;                                               // inclusive scan in the wave
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(inc, o, kWave);
    if (l >= o) inc += t;
  }
  __syncthreads();
  if (l == kWave - 1) wave_tot[w] = inc;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kFusedWaves; ++i) {
    before += (i < w) ? wave_tot[i] : 0;
    total += wave_tot[i];
  }
  int run = before + inc - sum;
#pragma unroll
  for (int k = 0; k < per; ++k) {
    const int i = tid * per + k;
    if (i < n) v[i] = run;
    run += loc[k];
  }
  __syncthreads();
  return total;
}

// Top-min(K, live) of the entries sh.skey/spos[0..n) in position order, of
// which `live` have a key > 0 (key 0 marks an empty entry), ties to the lower
// index.  With `out`, their positions are written to out[0..K) ascending and
// padded with -1; without, they are compacted in place into
// sh.skey/spos[0..min(K, live)).  n <= kFusedCap.  Returns min(K, live).
// Bounds lo <= hi on the live keys, when known (lo > 0), save the workgroup
// reduction that finds them.
__device__ __forceinline__ int lds_topk(FusedShared& sh, int n, int live, int K, int32_t* out,
                        uint32_t lo = 0u, uint32_t hi = 0u) {
  const int tid = threadIdx.x, w = tid / kWave, l = lane_id();
  uint32_t key[kFusedPerLane];
  int pos[kFusedPerLane];
#pragma unroll
  for (int i = 0; i < kFusedPerLane; ++i) {      // element s = w*512 + i*64 + l
    const int s = w * (kFusedPerLane * kWave) + i * kWave + l;
    key[i] = (s < n) ? sh.skey[s] : 0u;
    pos[i] = (s < n) ? sh.spos[s] : 0;
  }
  uint32_t thr = 0;                              // live <= K: every entry
  int n_eq = 0;
  if (live > K) {
    uint32_t smin = lo, smax = hi;
    if (lo == 0u) {
      int tot;
      block_key_stats<kFusedThreads, kFusedPerLane>(key, sh.t, &tot, &smin, &smax);
    }
    radix_select_regs<kFusedThreads, kFusedPerLane>(key, K, smin, smax, sh.t, &thr, &n_eq);
  }
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < kFusedPerLane; ++i) {
    gt += (key[i] != 0u && key[i] > thr) ? 1 : 0;
    eq += (key[i] != 0u && key[i] == thr) ? 1 : 0;
  }
  gt = wave_sum(gt);
  eq = wave_sum(eq);
  __syncthreads();                               // also: every read of sh above is done
  if (l == 0) {
    sh.t.wave_a[w] = gt;
    sh.t.wave_b[w] = eq;
  }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
#pragma unroll
  for (int i = 0; i < kFusedWaves; ++i) {
    gt_before += (i < w) ? sh.t.wave_a[i] : 0;
    eq_before += (i < w) ? sh.t.wave_b[i] : 0;
  }
  int eq_base = eq_before;
  int out_base = gt_before + min(n_eq, eq_before);
#pragma unroll
  for (int i = 0; i < kFusedPerLane; ++i) {
    const bool is_eq = key[i] != 0u && key[i] == thr;
    const uint64_t eqb = __ballot(is_eq);
    const bool sel = (key[i] != 0u && key[i] > thr) || (is_eq && eq_base + ballot_rank(eqb) < n_eq);
    const uint64_t selb = __ballot(sel);
    const int rank = out_base + ballot_rank(selb);
    if (sel && rank < K) {
      if (out) {
        out[rank] = pos[i];
      } else {
        sh.skey[rank] = key[i];
        sh.spos[rank] = pos[i];
      }
    }
    eq_base += __popcll(eqb);
    out_base += __popcll(selb);
  }
  const int m = min(live, K);
  if (out)
    for (int i = m + tid; i < K; i += kFusedThreads) out[i] = -1;
  __syncthreads();
  return m;
}

// grid (rows), 1024 threads: the whole top-k of a row.
// Fast path (at most 16384 kept pages and at least K finite quarter maxima
// among the ones used): t1 = the K-th largest of the pages' top-m quarter
// maxima (m = 1, 2 or 4); only 16-slot quarters whose maximum is >= t1 can
// hold scores >= t1, and those scores (at least K of them) are collected in
// position order and ranked exactly.
// Fallback (fewer than K finite quarter maxima, more than kFusedCandQ
// candidate quarters or more than kFusedCap survivors): the row is walked in
// chunks of 16384 slots (wave w: pages 16w .. 16w+15 of the chunk, lane l:
// slot l); each chunk's top-K (scores >= t1 when t1 is known) is appended in
// position order to the running result in LDS, which is cut back to its top K
// whenever it holds more.  Every element of the answer is in its chunk's
// top-K, so nothing of it is lost.
__device__ __forceinline__ void topk_row(FusedShared& sh, int row, const spin_batch& bt, int K,
                         const float* scores, const float* page_qmax, const int32_t* kept,
                         const int32_t* kept_count, int32_t* topk_out) {
  const int b = row / bt.R, r = row % bt.R;
  const int tid = threadIdx.x, w = tid / kWave, l = lane_id();
  const size_t mb = size_t(bt.max_blocks);
  int cnt = kept_count[b];
  cnt = cnt < 0 ? 0 : (cnt > bt.max_blocks ? bt.max_blocks : cnt);
  const int qr = bt.qpos[b] + r;
  const float* sc = scores + size_t(row) * mb * kBlock;
  const int32_t* kb = kept + size_t(b) * mb;
  int32_t* out = topk_out + size_t(row) * K;
  uint32_t lowest = 1u;                          // smallest key that can be in the answer

  if (page_qmax && cnt >= K / 4 && cnt <= kFusedMaxPages) {
    const float* pq = page_qmax + size_t(row) * mb * 4;
    // 1. t1 = the K-th largest of the pages' top-m quarter maxima, m = 1, 2 or
    // 4: the smallest with m * cnt >= 2K that fits 16 values per lane (value
    // e = w*1024 + i*64 + l: page e/m, rank e%m).  They are scores of
    // distinct slots, so at least K slots score >= t1.
    int lm = 0;
    while (lm < 2 && (cnt << lm) < 2 * K && (cnt << (lm + 1)) <= kFusedMaxPages) ++lm;
    // (every lane loads, page 0 past the count, so that the loads are issued
    // together rather than one branch and wait each)
    float4 xq[kFusedPageLanes];
#pragma unroll
    for (int i = 0; i < kFusedPageLanes; ++i) {
      const int p = (w * (kFusedPageLanes * kWave) + i * kWave + l) >> lm;
      xq[i] = *reinterpret_cast<const float4*>(pq + size_t(p < cnt ? p : 0) * 4);
    }
    uint32_t pk[kFusedPageLanes];
#pragma unroll
    for (int i = 0; i < kFusedPageLanes; ++i) {
      const int e = w * (kFusedPageLanes * kWave) + i * kWave + l;
      const int p = e >> lm, t = e & ((1 << lm) - 1);
      const float4 x = xq[i];
      float v;
      if (lm == 2) {
        v = t == 0 ? x.x : t == 1 ? x.y : t == 2 ? x.z : x.w;
      } else {
        const float a = fmaxf(x.x, x.y), b2 = fminf(x.x, x.y);
        const float c = fmaxf(x.z, x.w), d = fminf(x.z, x.w);
        const float top1 = fmaxf(a, c);
        const float top2 = fmaxf(fminf(a, c), fmaxf(b2, d));
        v = (lm == 1 && t == 1) ? top2 : top1;
      }
      pk[i] = (p < cnt && v > -INFINITY) ? ord_key(v) : 0u;
    }
    int nvals;
    uint32_t kmin, kmax;
    block_key_stats<kFusedThreads, kFusedPageLanes>(pk, sh.t, &nvals, &kmin, &kmax);
    if (nvals >= K) {
      uint32_t t1 = kmin;
      if (nvals > K) {
        int n_eq;
        radix_select_regs<kFusedThreads, kFusedPageLanes>(pk, K, kmin, kmax, sh.t, &t1, &n_eq);
      }
      lowest = max(t1, 1u);

      // 2. candidate quarters (quarter maximum >= t1), listed in ascending
      // position order: lane l of wave w checks the 16 consecutive pages
      // p = 1024 w + 16 l + i, and each page's quarters c with a maximum
      // >= t1 become entries 4p + c, so one scan of the lanes' counts places
      // every lane's entries.  Only those quarters can hold scores >= t1.
      const float f1 = key_to_float(t1);
      const int p_first = w * (kFusedPageLanes * kWave) + kFusedPageLanes * l;
      int qbits[kFusedPageLanes];
      int mine = 0;
#pragma unroll
      for (int i = 0; i < kFusedPageLanes; ++i) {
        const int p = p_first + i;
        xq[i] = *reinterpret_cast<const float4*>(pq + size_t(p < cnt ? p : 0) * 4);
      }
#pragma unroll
      for (int i = 0; i < kFusedPageLanes; ++i) {
        const float4 x = xq[i];
        qbits[i] = p_first + i < cnt ? int(x.x >= f1) | (int(x.y >= f1) << 1) |
                                           (int(x.z >= f1) << 2) | (int(x.w >= f1) << 3)
                                     : 0;
        mine += __popc(qbits[i]);
      }
      const int incl = wave_inclusive_sum(mine);
      __syncthreads();
      if (l == kWave - 1) sh.scan[w] = incl;
      __syncthreads();
      int before = 0, ncand = 0;
#pragma unroll
      for (int i = 0; i < kFusedWaves; ++i) {
        before += (i < w) ? sh.scan[i] : 0;
        ncand += sh.scan[i];
      }
      if (ncand <= kFusedCandQ) {
        int o = before + incl - mine;
        // the lane's flags as one 64-bit mask (bit 4 i + c: quarter c of page
        // p_first + i), walked set bit by set bit: entry 4 p_first + bit
        uint64_t fm = 0;
#pragma unroll
        for (int i = 0; i < kFusedPageLanes; ++i) fm |= uint64_t(qbits[i]) << (4 * i);
        while (fm != 0) {
          const int bit = __ffsll(static_cast<unsigned long long>(fm)) - 1;
          sh.cq[o++] = 4 * p_first + bit;
          fm &= fm - 1;
        }
        __syncthreads();

        // 3. survivors per candidate quarter.  Wave w scans the contiguous
        // candidate range [c_lo, c_hi), kFusedBatch quarters per step; each
        // group of 4 lanes takes one quarter per load (lane l: slots
        // 4(l%4) .. 4(l%4)+3 of it as one 16-byte load), so one load
        // instruction covers 16 quarters.  A slot survives if it is valid,
        // causal and its score is >= t1 (compared as floats: the key order
        // and the float order agree, with -0 = +0).
        const int per_wave = (ncand + kFusedWaves - 1) / kFusedWaves;
        const int c_lo = min(ncand, w * per_wave), c_hi = min(ncand, c_lo + per_wave);
        const int sub = 4 * (l & 3);
        constexpr int kLoads = kFusedBatch / 16;
        // lane's survivor flags (4 bits) for load i of the batch at c0, with
        // the slot of its first element
        auto survivors = [&](int c0, int i, const float4& v, int j, int* c_out, int* s_out) {
          const int c = c0 + 16 * i + (l >> 2);
          *c_out = c;
          const int e = (c < c_hi) ? sh.cq[c] : 0;
          const int slot = j * kBlock + 16 * (e & 3) + sub;
          *s_out = slot;
          const int lim = (c < c_hi && j >= 0 && j < bt.max_blocks) ? qr - slot : -1;
          return int(v.x >= f1 && lim >= 0) | (int(v.y >= f1 && lim >= 1) << 1) |
                 (int(v.z >= f1 && lim >= 2) << 2) | (int(v.w >= f1 && lim >= 3) << 3);
        };
        // scores and kept entries of a batch, all loads issued together
        auto load_batch = [&](int c0, float4* v, int* jv) {
#pragma unroll
          for (int i = 0; i < kLoads; ++i) {
            const int c = c0 + 16 * i + (l >> 2);
            const int e = (c < c_hi) ? sh.cq[c] : 0;
            v[i] = *reinterpret_cast<const float4*>(sc + size_t(e >> 2) * kBlock + 16 * (e & 3) + sub);
            jv[i] = kb[e >> 2];
          }
        };
        // One pass counts each quarter's survivors and appends the survivors
        // to the wave's slice sh.skey/spos[kSlice w, kSlice (w + 1)) in
        // position order (lanes are in position order within a load, loads
        // and batches ascend, and wave ranges follow one another), as long
        // as they fit.  Gaps left in the slices hold key 0, which lds_topk
        // reads as empty.
        constexpr int kSlice = kFusedCap / kFusedWaves;              // 512
        int wave_n = 0;                                              // this wave's survivors so far
        for (int c0 = c_lo; c0 < c_hi; c0 += kFusedBatch) {
          float4 v[kLoads];
          int jv[kLoads];
          load_batch(c0, v, jv);
          // loads of 16 quarters wholly past the wave's range hold nothing: their
          // processing is skipped (a wave-uniform test; the loads themselves are
          // issued regardless, so that they go out together)
          const int live_loads = __builtin_amdgcn_readfirstlane((c_hi - c0 + 15) / 16);
#pragma unroll
          for (int i = 0; i < kLoads; ++i) {
            if (i < live_loads) {
              int c, slot;
              const int f = survivors(c0, i, v[i], jv[i], &c, &slot);
              const int n = __popc(f);
              const int incl = wave_inclusive_sum(n);
              int o = wave_n + incl - n;
              const float vals[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                if (f & (1 << k)) {
                  if (o < kSlice) {
                    sh.skey[kSlice * w + o] = ord_key(vals[k]);
                    sh.spos[kSlice * w + o] = slot + k;
                  }
                  ++o;
                }
              }
              wave_n += __builtin_amdgcn_readlane(incl, kWave - 1);
            }
          }
        }
        if (l == 0) sh.wcount[w] = wave_n;
        __syncthreads();
        int nsurv = 0;
        bool spilled = false;
#pragma unroll
        for (int i = 0; i < kFusedWaves; ++i) {
          nsurv += sh.wcount[i];
          spilled = spilled || sh.wcount[i] > kSlice;
        }
        if (nsurv <= kFusedCap && nsurv >= K) {
          if (!spilled) {
            // 4. empty the rest of each slice, then rank the slices' entries
            for (int x = wave_n + l; x < kSlice; x += kWave) {
              sh.skey[kSlice * w + x] = 0u;
              sh.spos[kSlice * w + x] = 0;
            }
            __syncthreads();
            lds_topk(sh, kFusedCap, nsurv, K, out, lowest, max(kmax, lowest));
            return;
          }
          // 4'. a wave found more than its slice holds: a second read counts
          // each quarter's survivors, and after a scan of those counts a third
          // collects the survivors packed
          for (int c0 = c_lo; c0 < c_hi; c0 += kFusedBatch) {
            float4 v[kLoads];
            int jv[kLoads];
            load_batch(c0, v, jv);
#pragma unroll
            for (int i = 0; i < kLoads; ++i) {
              int c, slot;
              const int n = __popc(survivors(c0, i, v[i], jv[i], &c, &slot));
              // survivors of the quarter: sum over its 4 lanes (quad DPP)
              int q = n + __builtin_amdgcn_update_dpp(0, n, kDppXor1, 0xF, 0xF, false);
              q += __builtin_amdgcn_update_dpp(0, q, kDppXor2, 0xF, 0xF, false);
              if ((l & 3) == 3 && c < c_hi) sh.qcount[c] = q;
            }
          }
          __syncthreads();
          block_exclusive_scan(sh.qcount, ncand, sh.scan);
          for (int c0 = c_lo; c0 < c_hi; c0 += kFusedBatch) {
            float4 v[kLoads];
            int jv[kLoads];
            load_batch(c0, v, jv);
#pragma unroll
            for (int i = 0; i < kLoads; ++i) {
              int c, slot;
              const int f = survivors(c0, i, v[i], jv[i], &c, &slot);
              const int n = __popc(f);
              // survivors of the earlier lanes of the same quarter (the DPP
              // reads run on every lane, then each lane keeps its own terms)
              const int d1 = __builtin_amdgcn_update_dpp(0, n, 0x111, 0xF, 0xF, true);  // row_shr:1
              const int d2 = __builtin_amdgcn_update_dpp(0, n, 0x112, 0xF, 0xF, true);  // row_shr:2
              const int d3 = __builtin_amdgcn_update_dpp(0, n, 0x113, 0xF, 0xF, true);  // row_shr:3
              const int qi = l & 3;
              const int pre = (qi >= 1 ? d1 : 0) + (qi >= 2 ? d2 : 0) + (qi == 3 ? d3 : 0);
              int o = pre + ((c < c_hi) ? sh.qcount[c] : 0);
              const float vals[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                if (f & (1 << k)) {
                  sh.skey[o] = ord_key(vals[k]);
                  sh.spos[o] = slot + k;
                  ++o;
                }
              }
            }
          }
          __syncthreads();
          // 5. exact top-K of the survivors, written ascending
          lds_topk(sh, nsurv, nsurv, K, out, lowest, max(kmax, lowest));
          return;
        }
      }
    }
  }

  // ---------------------------------------------------------------- fallback
  constexpr int kChunkPages = kFusedThreads * kFusedPageLanes / kBlock;   // 256
  int n_run = 0;                                 // running result in sh.skey/spos[0..n_run)
  for (int p0 = 0; p0 < cnt; p0 += kChunkPages) {
    const int pw = p0 + w * kFusedPageLanes;     // this wave's first page
    const int my_j = (l < kFusedPageLanes && pw + l < cnt) ? kb[pw + l] : -1;
    float v[kFusedPageLanes];
#pragma unroll
    for (int i = 0; i < kFusedPageLanes; ++i)
      v[i] = (pw + i < cnt) ? sc[size_t(pw + i) * kBlock + l] : -INFINITY;
    uint32_t key[kFusedPageLanes];
#pragma unroll
    for (int i = 0; i < kFusedPageLanes; ++i) {
      const int j = __builtin_amdgcn_readlane(my_j, i);
      const bool ok = j >= 0 && j < bt.max_blocks && j * kBlock + l <= qr;
      const uint32_t kk = ord_key(v[i]);
      key[i] = (ok && kk >= lowest) ? kk : 0u;
    }
    int total;
    uint32_t kmin, kmax;
    block_key_stats<kFusedThreads, kFusedPageLanes>(key, sh.t, &total, &kmin, &kmax);
    if (total == 0) continue;
    const int want = min(K, total);
    uint32_t thr = 0;
    int n_eq = 0;
    if (want < total)
      radix_select_regs<kFusedThreads, kFusedPageLanes>(key, want, kmin, kmax, sh.t, &thr, &n_eq);
    // append the chunk's selection in position order after the running result
    int gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < kFusedPageLanes; ++i) {
      gt += (key[i] != 0u && key[i] > thr) ? 1 : 0;
      eq += (key[i] != 0u && key[i] == thr) ? 1 : 0;
    }
    gt = wave_sum(gt);
    eq = wave_sum(eq);
    __syncthreads();
    if (l == 0) {
      sh.t.wave_a[w] = gt;
      sh.t.wave_b[w] = eq;
    }
    __syncthreads();
    int gt_before = 0, eq_before = 0;
#pragma unroll
    for (int i = 0; i < kFusedWaves; ++i) {
      gt_before += (i < w) ? sh.t.wave_a[i] : 0;
      eq_before += (i < w) ? sh.t.wave_b[i] : 0;
    }
    int eq_base = eq_before;
    int out_base = n_run + gt_before + min(n_eq, eq_before);
#pragma unroll
    for (int i = 0; i < kFusedPageLanes; ++i) {
      const bool is_eq = key[i] != 0u && key[i] == thr;
      const uint64_t eqb = __ballot(is_eq);
      const bool sel =
          (key[i] != 0u && key[i] > thr) || (is_eq && eq_base + ballot_rank(eqb) < n_eq);
      const uint64_t selb = __ballot(sel);
      const int rank = out_base + ballot_rank(selb);
      if (sel && rank < n_run + want) {
        sh.skey[rank] = key[i];
        sh.spos[rank] = __builtin_amdgcn_readlane(my_j, i) * kBlock + l;
      }
      eq_base += __popcll(eqb);
      out_base += __popcll(selb);
    }
    __syncthreads();
    n_run += want;
    if (n_run > K) n_run = lds_topk(sh, n_run, n_run, K, nullptr);
  }
  lds_topk(sh, n_run, n_run, K, out);
}

// grid (rows), 1024 threads: the whole top-k of row blockIdx.x.  With
// `arrivals`, each workgroup first adds 1 to it (the gate of the round's
// tail waits for every one of them).
__global__ void __launch_bounds__(kFusedThreads)
k_topk_fused(spin_batch bt, int K, const float* scores, const float* page_qmax,
             const int32_t* kept, const int32_t* kept_count, int32_t* topk_out,
             unsigned long long* arrivals) {
  // An empty asm that clobbers v127 makes the kernel allocate 128 registers per
  // thread: its 16 waves then fill the CU's register files (4 waves x 128 of
  // 512 per SIMD), so no workgroup of the kernel beside the top-k (the EMA
  // update: 34 registers, 104 replaying) lands on a top-k CU and takes its
  // issue slots; the two then share only HBM.  (Without it the kernel
  // allocates 123 as compiled now; the clobber keeps the bound whatever the
  // compiler does.)
  asm volatile("" ::: "v127");
  __shared__ FusedShared sh;
  if (arrivals && threadIdx.x == 0)
    __hip_atomic_fetch_add(arrivals, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  topk_row(sh, blockIdx.x, bt, K, scores, page_qmax, kept, kept_count, topk_out);
}

// One wave that waits until `arrivals` reaches `target` (every workgroup of
// the gated top-k launch has started), polling the device-scope counter with
// vector loads, or until max_ticks of the 100 MHz device clock have passed;
// the update queued behind it on another stream then never takes the CUs
// the top-k needs.  The wait is bounded, so a top-k that cannot start only
// delays the update.
__global__ void __launch_bounds__(kWave)
k_gate(const unsigned long long* arrivals, unsigned long long target, uint64_t max_ticks) {
  if (threadIdx.x != 0) return;
  const uint64_t t0 = wall_clock64();
  while (__hip_atomic_load(arrivals, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    if (wall_clock64() - t0 > max_ticks) break;
    __builtin_amdgcn_s_sleep(1);
  }
}

// grid (rows, chunks of this level).
template <bool FIRST, bool FINAL>
__global__ void __launch_bounds__(kTopkThreads) k_topk_level(LevelArgs a) {
  __shared__ TopkShared sh;
  const int row = blockIdx.x;           // b * R + r
  const int c = blockIdx.y;             // chunk of this level
  const int b = row / a.bt.R, r = row % a.bt.R;
  const int tid = threadIdx.x, w = tid / kWave, l = lane_id();
  const int K = a.K;
  const size_t mb = size_t(a.bt.max_blocks);
  const int seg = c * kChunk + w * kSeg;  // first candidate of this wave

  uint32_t key[kPerLane];
  int my_kept = -1;                       // level 0: kept entry of block i (lane i)
  if (FIRST) {
    int cnt = a.kept_count[b];
    cnt = cnt < 0 ? 0 : (cnt > a.bt.max_blocks ? a.bt.max_blocks : cnt);
    const int n = cnt * kBlock;
    if (c * kChunk >= n) {                // the whole chunk is past the kept list
      if (!FINAL && tid == 0) a.out_counts[size_t(row) * a.out_chunks + c] = 0;
      if (FINAL)
        for (int i = tid; i < K; i += kTopkThreads) a.topk_out[size_t(row) * K + i] = -1;
      return;
    }
    const int qr = a.bt.qpos[b] + r;
    const float* s = a.scores + size_t(row) * mb * kBlock;
    if (l < kPerLane && seg + l * kBlock < n) my_kept = a.kept[size_t(b) * mb + seg / kBlock + l];
    float v[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int x = seg + i * kBlock + l;
      v[i] = (x < n) ? s[x] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int j = __builtin_amdgcn_readlane(my_kept, i);
      const bool ok = j >= 0 && j < a.bt.max_blocks && j * kBlock + l <= qr;
      const uint32_t kk = ord_key(v[i]);
      key[i] = ok ? kk : 0u;
    }
  } else {
    const uint32_t* ik = a.in_keys + size_t(row) * a.in_chunks * K;
    const int32_t* ic = a.in_counts + size_t(row) * a.in_chunks;
    // survivor slot sidx = g * K + within, advanced by 64 per step (no division)
    int g = (seg + l) / K, within = (seg + l) - g * K;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int sidx = seg + i * kBlock + l;
      const int cnt = (g < a.in_chunks) ? ic[g] : 0;
      key[i] = (within < cnt) ? ik[sidx] : 0u;
      within += kBlock;
      while (within >= K) {
        within -= K;
        ++g;
      }
    }
  }

  int total_valid;
  uint32_t kmin, kmax;
  block_key_stats<kTopkThreads, kPerLane>(key, sh, &total_valid, &kmin, &kmax);
  const int want = min(K, total_valid);
  uint32_t thr = 0;                       // select-all: every key > 0
  int n_eq = 0;
  if (want > 0 && want < total_valid)
    radix_select_regs<kTopkThreads, kPerLane>(key, want, kmin, kmax, sh, &thr, &n_eq);

  // ---- ordered emission ----
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    gt += (key[i] != 0u && key[i] > thr) ? 1 : 0;
    eq += (key[i] != 0u && key[i] == thr) ? 1 : 0;
  }
  gt = wave_sum(gt);
  eq = wave_sum(eq);
  __syncthreads();
  if (l == 0) {
    sh.wave_a[w] = gt;
    sh.wave_b[w] = eq;
  }
  __syncthreads();
  int gt_before = 0, eq_before = 0, gt_all = 0, eq_all = 0;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) {
    gt_before += (i < w) ? sh.wave_a[i] : 0;
    eq_before += (i < w) ? sh.wave_b[i] : 0;
    gt_all += sh.wave_a[i];
    eq_all += sh.wave_b[i];
  }
  const int total = want > 0 ? gt_all + min(n_eq, eq_all) : 0;
  int eq_base = eq_before;
  int out_base = gt_before + min(n_eq, eq_before);
  int rk[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const bool is_eq = key[i] != 0u && key[i] == thr;
    const uint64_t eqb = __ballot(is_eq);
    const bool sel = want > 0 &&
        ((key[i] != 0u && key[i] > thr) || (is_eq && eq_base + ballot_rank(eqb) < n_eq));
    const uint64_t selb = __ballot(sel);
    rk[i] = sel ? out_base + ballot_rank(selb) : -1;
    eq_base += __popcll(eqb);
    out_base += __popcll(selb);
  }
  const int32_t* ip = FIRST ? nullptr : a.in_pos + size_t(row) * a.in_chunks * K;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int rank = rk[i];
    if (rank >= 0 && rank < K) {
      const int pos = FIRST ? __builtin_amdgcn_readlane(my_kept, i) * kBlock + l
                            : ip[seg + i * kBlock + l];
      if (FINAL) {
        a.topk_out[size_t(row) * K + rank] = pos;
      } else {
        const size_t o = size_t(row) * a.out_chunks * K + size_t(c) * K + rank;
        a.out_keys[o] = key[i];
        a.out_pos[o] = pos;
      }
    }
  }
  if (FINAL) {
    for (int i = min(total, K) + tid; i < K; i += kTopkThreads) a.topk_out[size_t(row) * K + i] = -1;
  } else if (tid == 0) {
    a.out_counts[size_t(row) * a.out_chunks + c] = min(total, K);
  }
}

__global__ void __launch_bounds__(256)
k_miss(spin_batch bt, int K, const int32_t* full, const uint8_t* flags, float* miss) {
  __shared__ int s_t[4], s_m[4];
  const int b = blockIdx.x / bt.R;
  const int32_t* f = full + size_t(blockIdx.x) * K;
  const uint8_t* fl = flags + size_t(b) * bt.max_blocks;
  int tot = 0, mis = 0;
  for (int e = threadIdx.x; e < K; e += blockDim.x) {
    const int pos = f[e];
    if (pos >= 0) {
      ++tot;
      const int blk = pos / kBlock;
      if (blk >= bt.max_blocks || fl[blk] == 0) ++mis;
    }
  }
  tot = wave_sum(tot);
  mis = wave_sum(mis);
  if (lane_id() == 0) {
    s_t[threadIdx.x / kWave] = tot;
    s_m[threadIdx.x / kWave] = mis;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int t = s_t[0] + s_t[1] + s_t[2] + s_t[3];
    const int m = s_m[0] + s_m[1] + s_m[2] + s_m[3];
    miss[blockIdx.x] = t > 0 ? float(m) / float(t) : 0.0f;
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Device scratch of spin_topk_scores_noalloc (the chunked levels' survivor
// buffers), for callers that cannot allocate.  Each device holds its own copy
// for the life of the process.  In host code `scratch` only names the array:
// its device address comes from hipGetSymbolAddress, per device.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

}  // namespace

// Device address of this device's `scratch`, looked up on the first call on
// each device (with that device current) and kept.
hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  *bytes = kNoAllocScratchBytes;
  return hipSuccess;
}

TopkPlan topk_plan(int rows, int max_blocks, int K) {
  TopkPlan p;
  p.rows = rows;
  p.K = K;
  p.levels = 0;
  int64_t n = int64_t(max_blocks) * kBlock;
  int64_t widest = 0;
  while (true) {
    const int64_t chunks = (n + kChunk - 1) / kChunk;
    p.chunks[p.levels++] = int(chunks);
    if (chunks <= 1) break;
    if (chunks > widest) widest = chunks;
    n = chunks * K;
  }
  p.buf_elems = size_t(rows) * size_t(widest) * size_t(K);
  p.count_elems = size_t(rows) * size_t(widest);
  p.bytes = 2 * (align256(p.buf_elems * 4) * 2 + align256(p.count_elems * 4)) + 256;
  return p;
}

hipError_t launch_topk(const spin_batch& bt, int topk, const float* scores, const float* page_qmax,
                       const int32_t* kept, const int32_t* kept_count, int32_t* out, void* ws,
                       hipStream_t s) {
  const int rows = bt.B * bt.R;
  const TopkPlan p = topk_plan(rows, bt.max_blocks, topk);
  char* base = static_cast<char*>(ws);
  uint32_t* keys[2] = {nullptr, nullptr};
  int32_t* pos[2] = {nullptr, nullptr};
  int32_t* cnts[2] = {nullptr, nullptr};
  if (base) {
    size_t off = 0;
    for (int i = 0; i < 2; ++i) {
      keys[i] = reinterpret_cast<uint32_t*>(base + off);
      off += align256(p.buf_elems * 4);
      pos[i] = reinterpret_cast<int32_t*>(base + off);
      off += align256(p.buf_elems * 4);
      cnts[i] = reinterpret_cast<int32_t*>(base + off);
      off += align256(p.count_elems * 4);
    }
  }
  if (page_qmax) {
    hipLaunchKernelGGL(k_topk_fused, dim3(rows), dim3(kFusedThreads), 0, s, bt, topk, scores,
                       page_qmax, kept, kept_count, out, nullptr);
    return hipGetLastError();
  }
  LevelArgs a;
  a.bt = bt;
  a.K = topk;
  a.scores = scores;
  a.kept = kept;
  a.kept_count = kept_count;
  a.topk_out = out;
  for (int lv = 0; lv < p.levels; ++lv) {
    const bool first = lv == 0, final = lv == p.levels - 1;
    a.in_keys = first ? nullptr : keys[(lv - 1) & 1];
    a.in_pos = first ? nullptr : pos[(lv - 1) & 1];
    a.in_counts = first ? nullptr : cnts[(lv - 1) & 1];
    a.in_chunks = first ? 0 : p.chunks[lv - 1];
    a.out_keys = keys[lv & 1];
    a.out_pos = pos[lv & 1];
    a.out_counts = cnts[lv & 1];
    a.out_chunks = p.chunks[lv];
    const dim3 grid(unsigned(rows), unsigned(p.chunks[lv]));
    if (first && final)
      hipLaunchKernelGGL((k_topk_level<true, true>), grid, dim3(kTopkThreads), 0, s, a);
    else if (first)
      hipLaunchKernelGGL((k_topk_level<true, false>), grid, dim3(kTopkThreads), 0, s, a);
    else if (final)
      hipLaunchKernelGGL((k_topk_level<false, true>), grid, dim3(kTopkThreads), 0, s, a);
    else
      hipLaunchKernelGGL((k_topk_level<false, false>), grid, dim3(kTopkThreads), 0, s, a);
    const hipError_t e = hipGetLastError();     // a failed level stops the chain
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_topk_gated(const spin_batch& bt, int topk, const float* scores,
                             const float* page_qmax, const int32_t* kept,
                             const int32_t* kept_count, int32_t* out,
                             unsigned long long* arrivals, hipStream_t s) {
  hipLaunchKernelGGL(k_topk_fused, dim3(bt.B * bt.R), dim3(kFusedThreads), 0, s, bt, topk,
                     scores, page_qmax, kept, kept_count, out, arrivals);
  return hipGetLastError();
}

hipError_t launch_gate(const unsigned long long* arrivals, unsigned long long target,
                       hipStream_t s) {
  // at most 2 ms of the 100 MHz device clock
  hipLaunchKernelGGL(k_gate, dim3(1), dim3(kWave), 0, s, arrivals, target, uint64_t(200000));
  return hipGetLastError();
}

hipError_t launch_miss(const spin_batch& bt, int topk, const int32_t* full_topk,
                       const uint8_t* flags, float* miss, hipStream_t s) {
  hipLaunchKernelGGL(k_miss, dim3(bt.B * bt.R), dim3(256), 0, s, bt, topk, full_topk, flags,
                     miss);
  return hipGetLastError();
}

}  // namespace spin
