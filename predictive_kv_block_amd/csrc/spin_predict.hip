// SPIN block predictor: z = max(V, D), block max-pool, budgeted top-P block
// selection, Philox exploration and the MTP row union.
//
// Two kernels per call (three when several rows build their own masks):
//   k_block_scores  (B x R x block-chunks workgroups, streams D and VB, 128
//                    blocks per wave, the next batch's loads in flight while
//                    the current one is reduced)
//       S_j = max over existing slots i of block j of max(V_i, D_{q-i}).
//       For a block wholly at or before q this equals max(VB_j, max of the
//       D window), where VB_j (the block max of V) is kept exact by the update
//       kernel; the partial last block reads V directly.  The row-0
//       workgroups also write the request's Philox exploration words (ALU work
//       under the D loads).
//   k_select_regs   (one 1024-thread workgroup per request, or per (request,
//                    row) under the union policy; up to 16384 blocks)
//       each thread holds NPL blocks' keys in registers: radix-select of the
//       top-P blocks (ties -> lower j), radix-select of the n_exp explored
//       blocks with the smallest Philox words among the rest, ballot
//       compaction of the kept list.  k_select does the same from global
//       memory for longer contexts.
//   k_select_union  (union policy only: one workgroup per request) ORs the
//                    rows' flags and compacts the kept list.
#include "spin_device.h"
#include "spin_internal.h"
#include "spin_select.h"

namespace spin {
namespace {

constexpr int kScoreWaves = 4;        // waves per workgroup in k_block_scores
constexpr int kScoreBatch = 16;       // blocks per load batch (one D load per lane per block)
constexpr int kScoreBatchesPerWave = 8;
constexpr int kScoreBlocksPerWave = kScoreBatch * kScoreBatchesPerWave;   // 128
static_assert(kScoreBatchesPerWave % 2 == 0, "double-buffered batches");
constexpr int kSelectThreads = 1024;
constexpr int kSelectRegsMax = 16 * kSelectThreads;   // blocks the register-resident selection holds

__device__ __forceinline__ void budget(int keep_bp, int n, int explore_bp, int* kb, int* nexp) {
  const int k = int((int64_t(keep_bp) * n + 9999) / 10000);
  *kb = k;
  *nexp = int((int64_t(explore_bp) * k) / 10000);
}

// True when the request's arguments are usable; otherwise the selection
// kernel reports the error.
__device__ __forceinline__ bool request_ok(const SpinView& v, const spin_batch& bt, int s, int q0) {
  return s >= 0 && s < v.S && q0 >= 0 && q0 + bt.R - 1 < v.max_ctx &&
         num_blocks_of(q0 + bt.R - 1) <= bt.max_blocks && bt.max_blocks <= v.max_blocks;
}

// Exploration words, shared by every row of a request:
// u_j = Philox(counter (j/4, step, request id, 0), key (seed, layer)) word j%4,
// for j < n_last.  A wave writes blocks [j0, j0 + count) (j0 and count
// multiples of 4), lane g taking group j0/4 + g.
__device__ __forceinline__ void explore_words(const SpinView& v, int layer, int b, int s, int step,
                                              int j0, int count, int n_last) {
  const int g = j0 / 4 + lane_id();
  if (lane_id() >= count / 4 || 4 * g >= n_last) return;
  const Philox4x64 p = philox4x64_10(uint64_t(g), uint64_t(step), v.rid[s], 0ull, v.seed,
                                     uint64_t(layer));
  uint64_t* u = v.ukey + size_t(b) * v.max_blocks;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (4 * g + k < n_last) u[4 * g + k] = p.w[k];
}

// grid (ceil(max_blocks / (W * kScoreBlocksPerWave)), B, R), W waves: wave w
// of workgroup x scores the kScoreBlocksPerWave consecutive blocks from
// (x*W + w) * kScoreBlocksPerWave, in batches of kScoreBatch with the next
// batch's loads in flight while the current one is reduced.  Every batch
// issues the same loads (blocks past the last full one are masked).  The
// partial block holding q (if any) is scored apart from V and D directly.
// Row-0 waves also write the exploration words of their blocks.
__global__ void __launch_bounds__(kScoreWaves * kWave)
k_block_scores(SpinView v, int layer, spin_batch bt, int keep_bp) {
  const int b = blockIdx.y, r = blockIdx.z;
  const int s = bt.slot[b];
  const int q0 = bt.qpos[b];
  if (!request_ok(v, bt, s, q0) || keep_bp >= 10000) return;
  const size_t row = size_t(layer) * v.S + s;
  const int step = v.step[row];             // waited for only after the first loads
  const int q = q0 + r;
  const int n = num_blocks_of(q);
  const int n_last = num_blocks_of(q0 + bt.R - 1);
  int kb, nexp;
  budget(keep_bp, n, v.explore_bp, &kb, &nexp);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int jw = (blockIdx.x * kScoreWaves + wave) * kScoreBlocksPerWave;
  const bool words = r == 0 && v.explore_bp > 0 && jw < n_last;
  if (kb >= n || jw >= n) {
    if (words && step >= v.warmup) explore_words(v, layer, b, s, step, jw, kScoreBlocksPerWave, n_last);
    return;
  }

  const float* V = v.V + row * v.max_ctx;
  const float* D = v.D + row * v.max_ctx;
  const float* VB = v.VB + row * v.max_blocks;
  float* out = v.bscore + (size_t(b) * v.max_rows + r) * v.max_blocks;
  const int l = lane_id();
  const int nfull = (q + 1) / kBlock;          // blocks wholly at or before q

  // Group g of a batch is blocks jb + 4g .. jb + 4g + 3, whose D windows are the
  // 256 consecutive offsets from q - 64 (jb + 4g) - 255: lane l loads 4 of them
  // (16 bytes, 4-byte aligned), so 16-lane row k holds block jb + 4g + 3 - k.
  // Rows of blocks that are not full may reach below offset 0; those lanes
  // read offset 0 instead and their row is never stored.
  constexpr int kGroups = kScoreBatch / 4;
  float4 dbuf[2][kGroups];
  float vbuf[2][kGroups];
  const int row_k = l >> 4;
  auto issue = [&](int u, int t) {
    const int jb = jw + t * kScoreBatch;
#pragma unroll
    for (int gq = 0; gq < kGroups; ++gq) {
      const int o = q - kBlock * (jb + 4 * gq) - (4 * kBlock - 1) + 4 * l;
      __builtin_memcpy(&dbuf[u][gq], D + (o > 0 ? o : 0), sizeof(float4));
      const int j = jb + 4 * gq + 3 - row_k;
      vbuf[u][gq] = VB[j < nfull ? j : 0];
    }
  };
  auto reduce = [&](int u, int t) {
    const int jb = jw + t * kScoreBatch;
#pragma unroll
    for (int gq = 0; gq < kGroups; ++gq) {
      const float4 x = dbuf[u][gq];
      float m = fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w));
      // max over the 16-lane row: row shifts 1, 2, 4, 8 (lanes shifted in from
      // outside the row contribute -inf); lane 16k + 15 ends with the row's max
      m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(
                       __float_as_int(-INFINITY), __float_as_int(m), 0x111, 0xF, 0xF, false)));
      m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(
                       __float_as_int(-INFINITY), __float_as_int(m), 0x112, 0xF, 0xF, false)));
      m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(
                       __float_as_int(-INFINITY), __float_as_int(m), 0x114, 0xF, 0xF, false)));
      m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(
                       __float_as_int(-INFINITY), __float_as_int(m), 0x118, 0xF, 0xF, false)));
      const int j = jb + 4 * gq + 3 - row_k;
      if ((l & 15) == 15 && j < nfull) out[j] = fmaxf(m, vbuf[u][gq]);
    }
  };
  // the first batch's loads go out before the step count is known: a request
  // still warming up (its selection keeps every block) drops them unused
  issue(0, 0);
  if (step < v.warmup) return;
#pragma unroll
  for (int t = 0; t < kScoreBatchesPerWave; t += 2) {
    issue(1, t + 1);
    // the exploration words while the first two batches are in flight
    if (t == 0 && words) explore_words(v, layer, b, s, step, jw, kScoreBlocksPerWave, n_last);
    reduce(0, t);
    if (t + 2 < kScoreBatchesPerWave) issue(0, t + 2);
    reduce(1, t + 1);
  }

  // the partial block (slots 64 nfull .. q), owned by the wave whose range holds it
  if (nfull < n && nfull >= jw && nfull < jw + kScoreBlocksPerWave) {
    const int i = nfull * kBlock + l;
    const float z = (i <= q) ? fmaxf(V[i], D[q - i]) : -INFINITY;
    const float sj = wave_max(z);
    if (l == 0) out[nfull] = sj;
  }
}

// Sum over the wave (DPP, as wave_max).
__device__ __forceinline__ float wave_sum_f(float v) {
  int x = __float_as_int(v);
  x = __float_as_int(__int_as_float(x) + __int_as_float(dpp<kDppXor1, 0xF>(x)));
  x = __float_as_int(__int_as_float(x) + __int_as_float(dpp<kDppXor2, 0xF>(x)));
  x = __float_as_int(__int_as_float(x) + __int_as_float(dpp<kDppRowHalfMirror, 0xF>(x)));
  x = __float_as_int(__int_as_float(x) + __int_as_float(dpp<kDppRowMirror, 0xF>(x)));
  x = __float_as_int(__int_as_float(x) + __int_as_float(dpp<kDppRowBcast15, 0xA>(x)));
  x = __float_as_int(__int_as_float(x) + __int_as_float(dpp<kDppRowBcast31, 0xC>(x)));
  return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}

constexpr int kPoolBlocksPerWave = 16;

// Mean / Top-4 block pooling (the ablation variants): z per slot from V and D
// directly, one wave per block, lane t = slot 64 j + t; fp32 sums.
// grid (ceil(max_blocks / (W * kPoolBlocksPerWave)), B, rows), W waves.
template <int POOL>
__global__ void __launch_bounds__(kScoreWaves * kWave)
k_block_scores_pool(SpinView v, int layer, spin_batch bt, int keep_bp) {
  const int b = blockIdx.y, r = blockIdx.z;
  const int s = bt.slot[b];
  const int q0 = bt.qpos[b];
  if (!request_ok(v, bt, s, q0)) return;
  const size_t row = size_t(layer) * v.S + s;
  const int step = v.step[row];
  if (step < v.warmup || keep_bp >= 10000) return;
  const int q = q0 + r;
  const int n = num_blocks_of(q);
  const int n_last = num_blocks_of(q0 + bt.R - 1);
  const int jw = (blockIdx.x * kScoreWaves + threadIdx.x / kWave) * kPoolBlocksPerWave;
  if (r == 0 && v.explore_bp > 0 && jw < n_last)
    explore_words(v, layer, b, s, step, jw, kPoolBlocksPerWave, n_last);
  int kb, nexp;
  budget(keep_bp, n, v.explore_bp, &kb, &nexp);
  if (kb >= n) return;
  const float* V = v.V + row * v.max_ctx;
  const float* D = v.D + row * v.max_ctx;
  float* out = v.bscore + (size_t(b) * v.max_rows + r) * v.max_blocks;
  const int l = lane_id();
  for (int m = 0; m < kPoolBlocksPerWave; ++m) {
    const int j = jw + m;
    if (j >= n) break;
    const int i = j * kBlock + l;
    const float z = (i <= q) ? fmaxf(V[i], D[q - i]) : -INFINITY;
    const bool fin = z > -INFINITY;
    float sj;
    if (POOL == int(SPIN_POOL_MEAN)) {
      const int c = wave_sum(fin ? 1 : 0);
      const float sum = wave_sum_f(fin ? z : 0.0f);
      sj = c > 0 ? sum / float(c) : -INFINITY;
    } else {
      // the 4 largest: take the maximum, retire the lowest lane holding it
      float x = z, sum = 0.0f;
      int c = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float t = wave_max(x);
        if (t > -INFINITY) {
          sum += t;
          ++c;
        }
        const uint64_t at = __ballot(x == t);
        if (l == __ffsll(static_cast<unsigned long long>(at)) - 1) x = -INFINITY;
      }
      sj = c > 0 ? sum / float(c) : -INFINITY;
    }
    if (l == 0) out[j] = sj + 0.0f;            // -0 -> +0
  }
}

struct BlockScoreSrc {
  const float* S;
  __device__ bool get(int j, uint32_t& key) const {
    key = ord_key(S[j]);
    return true;
  }
};

struct ExploreSrc {
  const uint64_t* u;
  const uint8_t* flags;
  __device__ bool get(int j, uint64_t& key) const {
    if (flags[j] & 4) return false;      // predicted by this row
    key = ~u[j];                         // smallest word first
    return true;
  }
};

struct KeptSrc {
  const uint8_t* flags;
  __device__ bool get(int j, uint32_t& key) const {
    key = 0;
    return (flags[j] & 3) != 0;
  }
};

// Invalid request arguments: the whole-request workgroup clears its outputs
// and flags the error (the per-row workgroups leave that to k_select_union).
__device__ bool reject_request(const SpinView& v, const spin_batch& bt, int s, int q0,
                               int per_row, uint8_t* fo, int32_t* kept_count, int b) {
  if (request_ok(v, bt, s, q0)) return false;
  if (per_row) return true;
  for (int j = threadIdx.x; j < bt.max_blocks; j += blockDim.x) fo[j] = 0;
  if (threadIdx.x == 0) {
    kept_count[b] = 0;
    flag_error(v.err, (s < 0 || s >= v.S) ? SPIN_ERR_SLOT : SPIN_ERR_QPOS);
  }
  return true;
}

// The `want` largest valid keys of a register-resident selection (0 < want <
// number valid), ties to the lower element; returns this thread's bits.
template <int NPL, typename K>
__device__ uint32_t select_largest(const K (&key)[NPL], uint32_t valid, int want,
                                   RegsSelectShared& sh, int& pass, int* s_i) {
  K thr;
  int neq;
  regs_threshold<kSelectThreads, NPL, K>(key, valid, want, sh, pass, &thr, &neq);
  return regs_selected<kSelectThreads, NPL, K>(key, valid, thr, neq, s_i);
}

// Register-resident selection of one row, 1024 threads, max_blocks <=
// 1024 * NPL.  Thread (wave w, lane l) holds blocks j = w * 64 NPL + 64 i + l,
// i < NPL: their block scores for the top-P pass, then the exploration words
// of the blocks not predicted.  grid (B) with per_row = 0: one row (row 0;
// under the row-0 mask the blocks only the later rows reach are added as
// predicted), flags and the kept list written.  grid (B, R) with per_row = 1:
// workgroup (b, r) selects row r and leaves its flags (bit 0 predicted, bit 1
// explored; 0 past the row's last block) as bytes in the row's block-score
// workspace, which it has finished reading; k_select_union forms the union.
template <int NPL>
__global__ void __launch_bounds__(kSelectThreads)
k_select_regs(SpinView v, int layer, spin_batch bt, int keep_bp, int32_t* kept,
              int32_t* kept_count, uint8_t* flags_out, int per_row) {
  constexpr int NW = kSelectThreads / kWave;
  __shared__ RegsSelectShared sh;
  __shared__ int s_i[NW];      // tie counts of the selections
  __shared__ int s_c[NW];      // kept counts of the compaction
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid / kWave, l = lane_id();
  const int r = per_row ? int(blockIdx.y) : 0;
  const int e0 = w * (NPL * kWave) + l;        // block of step i: e0 + 64 i
  // The row's block scores and exploration words are loaded first, every
  // lane from block 0 past max_blocks: their addresses need neither the
  // request's slot, position nor step count, so the loads go out together at
  // once, and a request that turns out to be invalid or still warming up
  // leaves them unused.  (A conditional load per element had made the
  // compiler put each one behind its own branch and wait.)  With 16 blocks per
  // thread, registers allow neither that nor holding the words through the
  // top-P search: the scores are loaded after the request checks and the words
  // after the top-P search.
  constexpr bool kEarly = NPL <= 8;
  const uint64_t* u = v.ukey + size_t(b) * v.max_blocks;
  const float* S_row = v.bscore + (size_t(b) * v.max_rows + r) * v.max_blocks;
  auto block_of = [&](int i) { return e0 + kWave * i < bt.max_blocks ? e0 + kWave * i : 0; };
  float xs[NPL];
  uint64_t xu[NPL];
  if (kEarly) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      xu[i] = u[block_of(i)];
      xs[i] = S_row[block_of(i)];
    }
  }
  const int s = bt.slot[b];
  const int q0 = bt.qpos[b];
  uint8_t* fo = flags_out + size_t(b) * bt.max_blocks;
  if (reject_request(v, bt, s, q0, per_row, fo, kept_count, b)) return;
  if (!kEarly) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) xs[i] = S_row[block_of(i)];
  }
  const size_t row = size_t(layer) * v.S + s;
  const int step = v.step[row];
  const int n = num_blocks_of(q0 + r);
  const int n_last = num_blocks_of(q0 + bt.R - 1);
  uint32_t in_row = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) in_row |= (e0 + kWave * i < n) ? (1u << i) : 0u;
  int kb, nexp;
  budget(keep_bp, n, v.explore_bp, &kb, &nexp);
  const int pcount = kb - nexp;
  const bool budgeted = keep_bp < 10000 && kb < n;
  regs_select_init<kSelectThreads>(sh);
  __syncthreads();

  uint32_t pred = 0, expl = 0;
  if (!budgeted || step < v.warmup) {
    pred = in_row;
  } else {
    int pass = 0;
    if (pcount > 0) {
      uint32_t key[NPL];
#pragma unroll
      for (int i = 0; i < NPL; ++i) key[i] = ord_key(xs[i]) & (0u - (in_row >> i & 1u));
      pred = select_largest<NPL, uint32_t>(key, in_row, pcount, sh, pass, s_i);
    }
    if (nexp > 0) {    // smallest word first among the blocks not predicted (nexp < their count)
      if (!kEarly) {
#pragma unroll
        for (int i = 0; i < NPL; ++i) xu[i] = u[block_of(i)];
      }
      const uint32_t cand = in_row & ~pred;
      uint64_t ukey[NPL];
#pragma unroll
      for (int i = 0; i < NPL; ++i) ukey[i] = ~xu[i] & (uint64_t(0) - uint64_t(cand >> i & 1u));
      expl = select_largest<NPL, uint64_t>(ukey, cand, nexp, sh, pass, s_i);
    }
  }

  if (per_row) {
    uint8_t* rf = reinterpret_cast<uint8_t*>(v.bscore + (size_t(b) * v.max_rows + r) *
                                                            v.max_blocks);
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int j = e0 + kWave * i;
      if (j < n_last) rf[j] = uint8_t((pred >> i & 1u) | ((expl >> i & 1u) << 1));
    }
    return;
  }
  if (v.mask_row0) {     // blocks only the later rows reach (the draft positions)
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int j = e0 + kWave * i;
      if (j >= n && j < n_last) pred |= 1u << i;
    }
  }
  const uint32_t keep = pred | expl;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = e0 + kWave * i;
    if (j < bt.max_blocks)
      fo[j] = (pred >> i & 1u) ? uint8_t(1) : ((expl >> i & 1u) ? uint8_t(2) : uint8_t(0));
  }
  // ascending compaction: per-wave counts, then ballot ranks
  const int mine = wave_sum(__popc(keep));
  if (l == 0) s_c[w] = mine;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int x = 0; x < NW; ++x) {
    base += x < w ? s_c[x] : 0;
    total += s_c[x];
  }
  int32_t* ko = kept + size_t(b) * bt.max_blocks;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const bool k = (keep >> i & 1u) != 0;
    const uint64_t kb_ = __ballot(k);
    if (k) ko[base + ballot_rank(kb_)] = e0 + kWave * i;
    base += __popcll(kb_);
  }
  if (tid == 0) kept_count[b] = total;
}

// Flags in LDS (dynamic, max_blocks bytes): bit 0 predicted by some row, bit
// 1 explored by some row, bit 2 predicted by the current row; block scores and
// exploration words read from the state's workspace.  For requests longer than
// the register-resident selection holds; grid and per_row as k_select_regs.
__global__ void __launch_bounds__(kSelectThreads)
k_select(SpinView v, int layer, spin_batch bt, int keep_bp, int32_t* kept, int32_t* kept_count,
         uint8_t* flags_out, int per_row) {
  extern __shared__ __attribute__((aligned(16))) uint8_t s_flags[];
  __shared__ int s_scr[kSelectScratchInts];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int s = bt.slot[b];
  const int q0 = bt.qpos[b];
  uint8_t* fo = flags_out + size_t(b) * bt.max_blocks;
  int32_t* ko = kept + size_t(b) * bt.max_blocks;
  if (reject_request(v, bt, s, q0, per_row, fo, kept_count, b)) return;
  const size_t row = size_t(layer) * v.S + s;
  const bool warm = v.step[row] < v.warmup || keep_bp >= 10000;
  const int n_last = num_blocks_of(q0 + bt.R - 1);
  for (int j = tid; j < n_last; j += kSelectThreads) s_flags[j] = 0;
  __syncthreads();

  const int r = per_row ? int(blockIdx.y) : 0;
  const int n = num_blocks_of(q0 + r);
  int kb, nexp;
  budget(keep_bp, n, v.explore_bp, &kb, &nexp);
  if (warm || kb >= n) {
    for (int j = tid; j < n; j += kSelectThreads) s_flags[j] |= 1;
  } else {
    const int pcount = kb - nexp;
    if (pcount > 0) {
      BlockScoreSrc src{v.bscore + (size_t(b) * v.max_rows + r) * v.max_blocks};
      uint32_t thr;
      int neq;
      radix_threshold<kSelectThreads, 4, uint32_t>(src, n, pcount, &thr, &neq, s_scr);
      if (neq == 0x7fffffff)
        mark_at_least<kSelectThreads, 4, uint32_t>(src, n, thr, [&](int j) { s_flags[j] |= 5; });
      else
        ordered_emit<kSelectThreads, 2, uint32_t>(
            src, n, thr, neq, [&](int j, int) { s_flags[j] |= 5; }, s_scr);
    }
    if (nexp > 0) {
      ExploreSrc src{v.ukey + size_t(b) * v.max_blocks, s_flags};
      uint64_t thr;
      int neq;
      radix_threshold<kSelectThreads, 4, uint64_t>(src, n, nexp, &thr, &neq, s_scr);
      if (neq == 0x7fffffff)
        mark_at_least<kSelectThreads, 4, uint64_t>(src, n, thr, [&](int j) { s_flags[j] |= 2; });
      else
        ordered_emit<kSelectThreads, 2, uint64_t>(
            src, n, thr, neq, [&](int j, int) { s_flags[j] |= 2; }, s_scr);
    }
  }
  __syncthreads();

  if (per_row) {
    uint8_t* rf = reinterpret_cast<uint8_t*>(v.bscore + (size_t(b) * v.max_rows + r) *
                                                            v.max_blocks);
    for (int j = tid; j < n_last; j += kSelectThreads) rf[j] = s_flags[j] & 3;
    return;
  }
  if (v.mask_row0)      // blocks only the later rows reach (the draft positions)
    for (int j = n + tid; j < n_last; j += kSelectThreads) s_flags[j] |= 1;
  __syncthreads();
  for (int j = tid; j < bt.max_blocks; j += kSelectThreads) {
    uint8_t f = 0;
    if (j < n_last) f = (s_flags[j] & 1) ? 1 : ((s_flags[j] & 2) ? 2 : 0);
    fo[j] = f;
  }
  KeptSrc ksrc{s_flags};
  const int total = ordered_emit<kSelectThreads, 2, uint32_t>(
      ksrc, n_last, 0u, 0x7fffffff,
      [&](int j, int rank) {
        if (rank < bt.max_blocks) ko[rank] = j;
      },
      s_scr);
  if (tid == 0) kept_count[b] = min(total, bt.max_blocks);
}

// grid (B), kSelectThreads threads, dynamic LDS = max_blocks bytes: the union
// of the R rows' flags left by k_select in per-row mode (bit 0 predicted by
// some row, else bit 1 explored), written as the block flags, and the kept
// list compacted in ascending block order.
__global__ void __launch_bounds__(kSelectThreads)
k_select_union(SpinView v, spin_batch bt, int32_t* kept, int32_t* kept_count,
               uint8_t* flags_out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t s_flags[];
  __shared__ int s_scr[kSelectScratchInts];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int s = bt.slot[b];
  const int q0 = bt.qpos[b];
  uint8_t* fo = flags_out + size_t(b) * bt.max_blocks;
  int32_t* ko = kept + size_t(b) * bt.max_blocks;
  if (!request_ok(v, bt, s, q0)) {
    for (int j = tid; j < bt.max_blocks; j += kSelectThreads) fo[j] = 0;
    if (tid == 0) {
      kept_count[b] = 0;
      flag_error(v.err, (s < 0 || s >= v.S) ? SPIN_ERR_SLOT : SPIN_ERR_QPOS);
    }
    return;
  }
  const int n_last = num_blocks_of(q0 + bt.R - 1);
  const uint8_t* rf = reinterpret_cast<const uint8_t*>(v.bscore + size_t(b) * v.max_rows *
                                                                      v.max_blocks);
  const size_t rstride = size_t(v.max_blocks) * 4;     // bytes between rows
  for (int j = tid; j < n_last; j += kSelectThreads) {
    uint8_t f = 0;
    for (int r = 0; r < bt.R; ++r) f |= rf[r * rstride + j];
    s_flags[j] = f;
  }
  __syncthreads();
  for (int j = tid; j < bt.max_blocks; j += kSelectThreads) {
    uint8_t f = 0;
    if (j < n_last) f = (s_flags[j] & 1) ? 1 : ((s_flags[j] & 2) ? 2 : 0);
    fo[j] = f;
  }
  KeptSrc ksrc{s_flags};
  const int total = ordered_emit<kSelectThreads, 2, uint32_t>(
      ksrc, n_last, 0u, 0x7fffffff,
      [&](int j, int rank) {
        if (rank < bt.max_blocks) ko[rank] = j;
      },
      s_scr);
  if (tid == 0) kept_count[b] = min(total, bt.max_blocks);
}

}  // namespace

hipError_t launch_predict(const SpinView& v, int layer, const spin_batch& bt, int keep_bp,
                          int32_t* kept, int32_t* kept_count, uint8_t* flags, hipStream_t s) {
  const int per_wg = kScoreWaves * kScoreBlocksPerWave;
  const unsigned chunks = unsigned((bt.max_blocks + per_wg - 1) / per_wg);
  const unsigned rows = v.mask_row0 ? 1u : unsigned(bt.R);
  if (keep_bp < 10000) {
    if (v.pooling == int(SPIN_POOL_MAX)) {
      hipLaunchKernelGGL(k_block_scores, dim3(chunks, bt.B, rows), dim3(kScoreWaves * kWave), 0,
                         s, v, layer, bt, keep_bp);
    } else {
      const int per = kScoreWaves * kPoolBlocksPerWave;
      const dim3 grid(unsigned((bt.max_blocks + per - 1) / per), bt.B, rows);
      if (v.pooling == int(SPIN_POOL_MEAN))
        hipLaunchKernelGGL(k_block_scores_pool<int(SPIN_POOL_MEAN)>, grid,
                           dim3(kScoreWaves * kWave), 0, s, v, layer, bt, keep_bp);
      else
        hipLaunchKernelGGL(k_block_scores_pool<int(SPIN_POOL_TOP4)>, grid,
                           dim3(kScoreWaves * kWave), 0, s, v, layer, bt, keep_bp);
    }
  }
  // Several rows building their own masks (the union policy) run as one
  // workgroup per (request, row), then one per request forms the union.
  const int per_row = (!v.mask_row0 && bt.R > 1) ? 1 : 0;
  const dim3 grid(unsigned(bt.B), per_row ? unsigned(bt.R) : 1u);
  const dim3 block(kSelectThreads);
  if (bt.max_blocks <= 2 * kSelectThreads)
    hipLaunchKernelGGL(k_select_regs<2>, grid, block, 0, s, v, layer, bt, keep_bp, kept,
                       kept_count, flags, per_row);
  else if (bt.max_blocks <= 4 * kSelectThreads)
    hipLaunchKernelGGL(k_select_regs<4>, grid, block, 0, s, v, layer, bt, keep_bp, kept,
                       kept_count, flags, per_row);
  else if (bt.max_blocks <= 8 * kSelectThreads)
    hipLaunchKernelGGL(k_select_regs<8>, grid, block, 0, s, v, layer, bt, keep_bp, kept,
                       kept_count, flags, per_row);
  else if (bt.max_blocks <= kSelectRegsMax)
    hipLaunchKernelGGL(k_select_regs<16>, grid, block, 0, s, v, layer, bt, keep_bp, kept,
                       kept_count, flags, per_row);
  else
    hipLaunchKernelGGL(k_select, grid, block, size_t(bt.max_blocks), s, v, layer, bt, keep_bp,
                       kept, kept_count, flags, per_row);
  if (per_row) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_select_union, dim3(bt.B), dim3(kSelectThreads), size_t(bt.max_blocks),
                       s, v, bt, kept, kept_count, flags);
  }
  return hipGetLastError();
}

}  // namespace spin
