// Query quantisation and the gather-indexer over the kept KV pages.
//
// k_quantize: per (request, row, head) the exponent e = smallest integer with
//   max|q| * 2^-e <= 448, codes = RNE e4m3fn(q * 2^-e) (exact scaling), and
//   wq = w * 2^e, so sum_h wq_h ReLU(q8_h . k) equals the bf16-query score up
//   to the rounding of q to e4m3fn.
// k_indexer: one wave per kept page (64 tokens x 128 fp8 = 8 KB, contiguous in
//   the pool); optionally also, per row, the maxima of the page's four 16-slot
//   quarters, which let the top-k discard most candidates before ranking them.  Heads form the M side of v_mfma_scale_f32_16x16x128_f8f6f4 and
//   tokens the N side, so one MFMA does 16 heads x 16 tokens over the whole
//   head dim; a page is 4 head tiles x 4 token tiles per row.  ReLU, the head
//   weights and the head sum run on the accumulator registers (the epilogue of
//   one head tile beside the MFMAs of the next), the 4 lane groups are folded
//   with permlane swaps, and every lane then holds the score of token `lane`;
//   rows are staged in LDS and written in bursts.
#include <atomic>

#include "spin_device.h"
#include "spin_internal.h"

namespace spin {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kHeads = 64;
constexpr int kDim = 128;
constexpr int kPagesPerWave = 32;    // pages each wave takes in turn, one query row
constexpr int kPagesPerWaveMR = 16;  // the same with several query rows (more workgroups)
constexpr int kIdxWaves = 4;         // waves per workgroup
constexpr int kStages1 = 2;          // key ring depth: pages in flight + the one on the MFMAs
constexpr int kStagesMR = 2;         // the same with several rows (more compute per page)
// LDS row stride of the staged queries: 16 bytes of padding after each head
// row move the 16 head rows that one operand read touches onto different banks.
constexpr int kQStride = kDim + 16;
constexpr int kFlushRows = 32;       // page-rows of scores staged per wave before a burst write
constexpr int kFlushRowsMR = 8;      // the same with several rows (small: 3 workgroups per CU)
constexpr int kIdxMinPagesPerWg = 16;  // smallest share of the batch's pages a workgroup takes
constexpr int kIdxRounds = 4;        // dispatch rounds of resident workgroups per launch
template <int R>
constexpr int pages_per_wave() { return R == 1 ? kPagesPerWave : kPagesPerWaveMR; }
static_assert(kStages1 >= 2 && kStagesMR >= 2 && kPagesPerWave + kStages1 <= kWave &&
                  kPagesPerWaveMR + kStagesMR <= kWave,
              "indexer pipeline shape");
static_assert(kQStride % 16 == 0, "16-byte aligned query rows");

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Smallest e with amax * 2^-e <= 448.  amax = f * 2^x with f in [0.5, 1):
// f * 2^9 <= 448 iff f <= 0.875, so e = x - 9 then, else x - 8.
__device__ __forceinline__ int q_exponent(float amax) {
  if (amax == 0.0f) return 0;
  int x;
  const float f = frexpf(amax, &x);
  return x - (f <= 0.875f ? 9 : 8);
}

// grid (B, R, 16), 256 threads; wave w handles head 4z + w; lane l the
// elements 2l and 2l+1 of the head.
__global__ void __launch_bounds__(256)
k_quantize(SpinView v, spin_batch bt, const uint16_t* q, const float* w) {
  const int b = blockIdx.x, r = blockIdx.y;
  const int l = lane_id();
  const size_t in_row = size_t(b) * bt.R + r;
  const size_t ws_row = size_t(b) * v.max_rows + r;
  {
    const int h = blockIdx.z * 4 + threadIdx.x / kWave;
    const uint32_t pair =
        *reinterpret_cast<const uint32_t*>(q + (in_row * kHeads + h) * kDim + 2 * l);
    const float x0 = bf16_bits_to_f32(pair & 0xFFFFu), x1 = bf16_bits_to_f32(pair >> 16);
    const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    const int e = q_exponent(amax);
    const float y0 = ldexpf(x0, -e), y1 = ldexpf(x1, -e);
    const uint32_t packed = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false));
    *reinterpret_cast<uint16_t*>(v.q8 + (ws_row * kHeads + h) * kDim + 2 * l) =
        uint16_t(packed & 0xFFFFu);
    if (l == 0) {
      v.wq[ws_row * kHeads + h] = ldexpf(w[in_row * kHeads + h], e);
      v.qexp[ws_row * kHeads + h] = e;
    }
  }
}

// 32 contiguous key bytes.
__device__ __forceinline__ v8i load32(const uint8_t* p) {
  return *reinterpret_cast<const v8i*>(p);
}

// One page of keys in MFMA B-operand layout: tile tt holds tokens 16tt..16tt+15,
// lane (g, n16) the 32 bytes g*32.. of token 16tt + n16.
struct PageRegs {
  v8i t[4];
};

// Issues the 8 loads of page p, or, when `live` is false, 8 loads that all hit
// the pool's first 32 bytes: the ring then issues the same number of loads on
// every path, so the waits before the MFMAs stay partial (a conditional load
// would force a full drain of the load queue).
__device__ __forceinline__ void load_page(PageRegs& dst, const uint8_t* k_pool, int p, bool live,
                                          int lane_off) {
  const uint8_t* base = k_pool + (live ? size_t(p) * (kBlock * kDim) + lane_off : 0);
  const int step = live ? 16 * kDim : 0;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) dst.t[tt] = load32(base + tt * step);
}

// 2 max(x, 0) as x + |x|: one add with an abs source modifier, exact for finite
// x (fmaxf would cost a second, NaN-quieting max in IEEE mode).  The head
// weights are staged halved, so (w/2)(x + |x|) is bit-identical to w max(x, 0).
__device__ __forceinline__ float relu2(float x) { return x + fabsf(x); }

// Sum of the four lane groups' partials for token `lane`: lane group g
// (lanes 16g..16g+15) holds, for each token tile tt, its partial sum of token
// 16 tt + (lane & 15); the result of lane l is the full sum for token l.  Two
// half-wave swaps (lanes l and l + 32) fold tiles (0, 2) and (1, 3), then one
// row swap (lanes l and l + 16 within each half) folds the rest: three
// permlane swaps and three adds, no LDS traffic.
__device__ __forceinline__ float fold_lane_groups(const float (&p)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]),
                                                  false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]),
                                                  false, false);
  // lanes 0..31: tiles 0 and 1; lanes 32..63: tiles 2 and 3
  const float x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float y = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false,
                                                  false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Raw (unscaled) scores of token `lane` of one page for every query row r:
// 4R steps of (row, head tile), each 4 MFMAs (one per token tile) into one of
// two accumulator sets, software-pipelined so that the ReLU / head-weight
// epilogue of step i - 1 (32 VALU operations on the other set) issues while
// the MFMAs of step i run.  ReLU is x + |x| against halved head weights (s_w),
// bit-identical to w max(x, 0).
template <int R>
__device__ __forceinline__ void page_scores(const PageRegs& kb, const uint8_t* s_q,
                                            const float* s_w, int g, int n16, float (&res)[R]) {
  constexpr int T = 4 * R;
  float part[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) part[r][tt] = 0.0f;
  v4f acc[2][4];
  v8i qa[2];
  float4 wv[2];
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // query operand of step i: row i / 4, head tile i % 4
  auto q_of = [&](int i) {
    return *reinterpret_cast<const v8i*>(s_q + ((i / 4) * kHeads + (i % 4) * 16 + n16) * kQStride +
                                         g * 32);
  };
  auto w_of = [&](int i) {
    return *reinterpret_cast<const float4*>(s_w + (i / 4) * kHeads + (i % 4) * 16 + g * 4);
  };
  // With several rows the LDS operands are read one step ahead (the next
  // step's query tile, this step's head weights for its epilogue in the next
  // step), so the MFMAs do not wait on LDS; with one row the kernel is bound
  // by HBM and keeps the registers instead (3 waves per SIMD either way).
  constexpr bool kAhead = R > 1;
  if (kAhead) qa[0] = q_of(0);
#pragma unroll
  for (int i = 0; i <= T; ++i) {
    if (i < T) {
      if (kAhead) {
        if (i + 1 < T) qa[(i + 1) & 1] = q_of(i + 1);
      } else {
        qa[i & 1] = q_of(i);
      }
      wv[i & 1] = w_of(i);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        acc[i & 1][tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[i & 1], kb.t[tt], zero,
                                                                          0, 0, 0, 127, 0, 127);
    }
    if (i > 0) {
      const int r = (i - 1) / 4;
      const float4 w = wv[(i - 1) & 1];
      const v4f* a = acc[(i - 1) & 1];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        part[r][tt] = fmaf(w.x, relu2(a[tt][0]), part[r][tt]);
        part[r][tt] = fmaf(w.y, relu2(a[tt][1]), part[r][tt]);
        part[r][tt] = fmaf(w.z, relu2(a[tt][2]), part[r][tt]);
        part[r][tt] = fmaf(w.w, relu2(a[tt][3]), part[r][tt]);
        // keep this step's epilogue inside its scheduling region (beside the
        // next step's MFMAs) instead of letting it sink to the end of the page
        asm volatile("" : "+v"(part[r][tt]));
      }
    }
    if (i < T) {
      // the LDS reads first, then one MFMA and 8 epilogue operations, four times
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) res[r] = fold_lane_groups(part[r]);
}

// Count of kept pages of row b as the kernels use it: negative counts read as
// 0 and counts above max_blocks as max_blocks (both are reported as errors).
__device__ __forceinline__ int kept_pages_of(const int32_t* kept_count, int b, int max_blocks) {
  const int c = kept_count[b];
  return c < 0 ? 0 : (c > max_blocks ? max_blocks : c);
}

// 64-bit value of lane `src` (wave-uniform result).
__device__ __forceinline__ int64_t readlane64(int64_t x, int src) {
  const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(uint64_t(x)), src);
  const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(uint64_t(x) >> 32), src);
  return int64_t((uint64_t(hi) << 32) | lo);
}

// Balanced split.  The batch's kept pages, taken row after row in kept order,
// form one sequence of T pages; the workgroups used (whole dispatch rounds of
// the resident workgroups, or one partial round for a small batch) take equal
// consecutive shares of it, so every workgroup finishes at about the same
// time whatever the kept counts are (per-row chunks of fixed size leave a
// partial last dispatch round that costs a full one).  A share that crosses a row boundary is processed
// one row segment at a time: the segment's queries are staged in LDS and its
// pages split into 4 consecutive wave ranges.  Every wave walks the counts
// itself, so the workgroup's barriers are uniform.
//
// Within a wave range, page metadata (kept entry -> block table -> scale) for
// up to P pages sits in lanes 0..P-1 and is read back with scalar lane reads,
// so every branch on it is wave-uniform.  Keys stream through a ring of
// kStages register buffers: while page m is on the MFMAs, pages m+1 ..
// m+kStages-1 are in flight.  Score rows are staged in LDS and written
// kFlushRows pages (one row) or kFlushRowsMR/R pages (R rows) at a time as one
// contiguous burst per row: single 256-byte rows, each written long after its
// neighbours, reach HBM as scattered partial-row writes that stall the key
// stream far more than their share of the bytes.
template <int R>
__global__ void __launch_bounds__(kIdxWaves * kWave)
    __attribute__((amdgpu_waves_per_eu(3)))   // register budget for 3 waves per SIMD
k_indexer(SpinView v, spin_batch bt, const uint8_t* __restrict__ k_pool,
          const float* __restrict__ k_scale, int64_t pool_pages, const int32_t* table,
          const int32_t* kept, const int32_t* kept_count, float* scores, float* page_qmax,
          int resident) {
  constexpr int kPagesPerWaveR = pages_per_wave<R>();
  constexpr int F = (R == 1 ? kFlushRows : kFlushRowsMR) / R > 0
                        ? (R == 1 ? kFlushRows : kFlushRowsMR) / R : 1;   // pages per flush
  constexpr int kStages = R == 1 ? kStages1 : kStagesMR;
  __shared__ __attribute__((aligned(16))) uint8_t s_q[R * kHeads * kQStride];
  __shared__ float s_w[R * kHeads];
  __shared__ __attribute__((aligned(16))) float s_out[kIdxWaves * R * F * kBlock];
  __shared__ int s_seg[3 * kWave];
  __shared__ __attribute__((aligned(16))) float s_qm[R == 1 ? kIdxWaves * F * 4 : 4];

  const int l = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const size_t mb = size_t(bt.max_blocks);

  // Total kept pages T (per lane the low and high parts of its counts, so the
  // wave sums stay within int).
  int64_t total = 0;
  for (int r0 = 0; r0 < bt.B; r0 += kWave) {
    int c = 0;
    if (r0 + l < bt.B) {
      const int raw = kept_count[r0 + l];
      c = kept_pages_of(kept_count, r0 + l, bt.max_blocks);
      if (raw != c && blockIdx.x == 0 && wave == 0) flag_error(v.err, SPIN_ERR_KEPT);
    }
    total += (int64_t(wave_sum(c >> 12)) << 12) + wave_sum(c & 4095);
  }
  // Workgroups used: whole dispatch rounds of the `resident` workgroups while
  // each gets at least 32 R pages (up to kIdxRounds rounds), else one partial
  // round of shares of at least kIdxMinPagesPerWg pages.
  int64_t rounds = total / (int64_t(resident) * 32 * R);
  if (rounds > kIdxRounds) rounds = kIdxRounds;
  int64_t groups = rounds > 0 ? rounds * resident
                              : (total + kIdxMinPagesPerWg - 1) / kIdxMinPagesPerWg;
  if (rounds == 0 && groups > resident) groups = resident;
  if (groups > int64_t(gridDim.x)) groups = gridDim.x;
  if (int64_t(blockIdx.x) >= groups) return;
  const int64_t g0 = int64_t(blockIdx.x) * total / groups;
  const int64_t g1 = (int64_t(blockIdx.x) + 1) * total / groups;

  const int g = l >> 4;       // lane group: K chunk of the operands, M rows of the result
  const int n16 = l & 15;     // M row of A / N column of B
  const int lane_off = n16 * kDim + g * 32;
  float* my_out = s_out + wave * (R * F * kBlock);
  float* my_qm = s_qm + wave * (R * F * 4);

  // Walk the rows 64 at a time: lane l holds row r0 + l, its pages [start, end)
  // in the sequence; rows meeting [g0, g1) are this workgroup's segments.
  // Wave 0 lists them in LDS (row, first and end kept position), so that no
  // per-lane walk state stays live while pages are scored.
  int64_t base = 0;
  for (int r0 = 0; r0 < bt.B && base < g1; r0 += kWave) {
    int nseg;
    {
      const int c = (r0 + l < bt.B) ? kept_pages_of(kept_count, r0 + l, bt.max_blocks) : 0;
      int64_t incl = c;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int64_t t = __shfl_up(incl, o, kWave);
        if (l >= o) incl += t;
      }
      const int64_t end = base + incl, start = end - c;
      const bool on = c > 0 && start < g1 && end > g0;
      const uint64_t hit = __ballot(on);
      nseg = __popcll(hit);
      __syncthreads();     // the previous list and staged queries are no longer read
      if (wave == 0 && on) {
        const int at = ballot_rank(hit);
        s_seg[3 * at] = r0 + l;
        s_seg[3 * at + 1] = int((g0 > start ? g0 : start) - start);
        s_seg[3 * at + 2] = int((g1 < end ? g1 : end) - start);
      }
      base += readlane64(incl, kWave - 1);
      __syncthreads();
    }
    for (int si = 0; si < nseg; ++si) {
      const int b = __builtin_amdgcn_readfirstlane(s_seg[3 * si]);
      const int k0 = __builtin_amdgcn_readfirstlane(s_seg[3 * si + 1]);
      const int k1 = __builtin_amdgcn_readfirstlane(s_seg[3 * si + 2]);

      // Stage this row's quantised queries and halved head weights in LDS.
      if (si > 0) __syncthreads();
      const uint8_t* q8 = v.q8 + size_t(b) * v.max_rows * kHeads * kDim;
      const float* wq = v.wq + size_t(b) * v.max_rows * kHeads;
      for (int x = threadIdx.x; x < R * kHeads * kDim / 16; x += kIdxWaves * kWave)
        *reinterpret_cast<uint4*>(s_q + (x / (kDim / 16)) * kQStride + (x % (kDim / 16)) * 16) =
            reinterpret_cast<const uint4*>(q8)[x];
      for (int x = threadIdx.x; x < R * kHeads; x += kIdxWaves * kWave) s_w[x] = 0.5f * wq[x];
      __syncthreads();

      const int q0 = bt.qpos[b];
      const int n = k1 - k0;
      const int wa = k0 + int(int64_t(n) * wave / kIdxWaves);
      const int we = k0 + int(int64_t(n) * (wave + 1) / kIdxWaves);
      for (int kw = wa; kw < we; kw += kPagesPerWaveR) {
        const int npages = min(kPagesPerWaveR, we - kw);

        // Page metadata of this batch, lane m holding page m (j = -1: invalid).
        int my_j = -1, my_p = 0;
        float my_sc = 0.0f;
        if (l < npages) {
          const int j = kept[size_t(b) * mb + kw + l];
          if (j < 0 || j >= bt.max_blocks) {
            flag_error(v.err, SPIN_ERR_KEPT);
          } else {
            const int p = table[size_t(b) * mb + j];
            if (p < 0 || int64_t(p) >= pool_pages) {
              flag_error(v.err, SPIN_ERR_PAGE);
            } else {
              my_j = j;
              my_p = p;
              my_sc = k_scale[p];
            }
          }
        }

        // Invalid pages (flagged above) read page 0 and are written as -inf.
        PageRegs ring[kStages];
#pragma unroll
        for (int f = 0; f + 1 < kStages; ++f)
          load_page(ring[f], k_pool, __builtin_amdgcn_readlane(my_p, f), f < npages, lane_off);

        for (int m0 = 0; m0 < npages; m0 += kStages) {
#pragma unroll
          for (int u = 0; u < kStages; ++u) {
            const int m = m0 + u;
            if (m >= npages) break;
            load_page(ring[(u + kStages - 1) % kStages], k_pool,
                      __builtin_amdgcn_readlane(my_p, m + kStages - 1), m + kStages - 1 < npages,
                      lane_off);
            const int j = __builtin_amdgcn_readlane(my_j, m);
            const float sc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_sc), m));
            const int mf = m % F;
            float val[R];
            if (j >= 0) page_scores<R>(ring[u], s_q, s_w, g, n16, val);
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const float out = (j >= 0 && j * kBlock + l <= q0 + r) ? val[r] * sc : -INFINITY;
              my_out[(r * F + mf) * kBlock + l] = out;
              if (page_qmax) {
                // maxima of the page's four 16-slot quarters (DPP row reduction;
                // lane 16c + 15 holds quarter c), one 16-byte row (staged in LDS
                // with one query row)
                float x = out;
                x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(
                                 __float_as_int(-INFINITY), __float_as_int(x), 0x111, 0xF, 0xF, false)));
                x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(
                                 __float_as_int(-INFINITY), __float_as_int(x), 0x112, 0xF, 0xF, false)));
                x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(
                                 __float_as_int(-INFINITY), __float_as_int(x), 0x114, 0xF, 0xF, false)));
                x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(
                                 __float_as_int(-INFINITY), __float_as_int(x), 0x118, 0xF, 0xF, false)));
                if ((l & 15) == 15) {
                  if (R == 1)
                    my_qm[(r * F + mf) * 4 + (l >> 4)] = x;
                  else
                    page_qmax[((size_t(b) * R + r) * mb + kw + m) * 4 + (l >> 4)] = x;
                }
              }
            }
            if (mf == F - 1 || m + 1 == npages) {
              // Flush pages m-mf .. m of every row: LDS -> one contiguous burst of
              // scores and one of quarter maxima.
              __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
              __builtin_amdgcn_wave_barrier();
              __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
              const int n4 = (mf + 1) * (kBlock / 4);
#pragma unroll
              for (int r = 0; r < R; ++r) {
                v4f* dst = reinterpret_cast<v4f*>(scores + (size_t(b) * R + r) * mb * kBlock +
                                                  size_t(kw + m - mf) * kBlock);
                const v4f* src = reinterpret_cast<const v4f*>(my_out + r * F * kBlock);
#pragma unroll
                for (int i0 = 0; i0 < F * (kBlock / 4); i0 += kWave) {
                  const int x = i0 + l;
                  if (x < n4) {
                    __builtin_nontemporal_store(src[x], dst + x);   // streaming
                  }
                }
                if (R == 1 && page_qmax && l <= mf) {
                  // the pages' quarter maxima, one 16-byte row per page, written
                  // together: with one query row, single 16-byte rows stored page
                  // by page cost the key stream about 2% more (with several rows
                  // the flushes come every few pages and the rows go out directly)
                  v4f* qd = reinterpret_cast<v4f*>(page_qmax +
                                                   ((size_t(b) * R + r) * mb + kw + m - mf) * 4);
                  qd[l] = reinterpret_cast<const v4f*>(my_qm + r * F * 4)[l];
                }
              }
              __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
              __builtin_amdgcn_wave_barrier();
              __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
          }
        }
      }
    }
  }
}
}  // namespace

hipError_t launch_quantize(const SpinView& v, const spin_batch& bt, const void* q_bf16,
                           const float* w, hipStream_t s) {
  hipLaunchKernelGGL(k_quantize, dim3(bt.B, bt.R, kHeads / 4), dim3(256), 0, s, v, bt,
                     reinterpret_cast<const uint16_t*>(q_bf16), w);
  return hipGetLastError();
}

// Workgroups of one indexer launch: kIdxRounds dispatch rounds of the
// device's resident k_indexer<R> workgroups (occupancy x compute units, taken
// once per device), and no more than shares of kIdxMinPagesPerWg pages need;
// the kernel uses as many of them as the batch's kept pages call for.
template <int R>
hipError_t indexer_groups(const spin_batch& bt, unsigned* groups, int* resident_out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> resident[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cap = (dev >= 0 && dev < kMaxDevices) ? resident[dev].load(std::memory_order_relaxed) : 0;
  if (cap <= 0) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_indexer<R>, kIdxWaves * kWave, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cap = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
    if (dev >= 0 && dev < kMaxDevices) resident[dev].store(cap, std::memory_order_relaxed);
  }
  const int64_t most =
      (int64_t(bt.B) * bt.max_blocks + kIdxMinPagesPerWg - 1) / kIdxMinPagesPerWg;
  int64_t g = int64_t(cap) * kIdxRounds;
  if (g > most) g = most;
  *groups = unsigned(g > 0 ? g : 1);
  *resident_out = cap;
  return hipSuccess;
}

hipError_t launch_indexer(const SpinView& v, const spin_batch& bt, const uint8_t* k_pool,
                          const float* k_scale, int64_t pool_pages, const int32_t* table,
                          const int32_t* kept, const int32_t* kept_count, float* scores,
                          float* page_qmax, hipStream_t s) {
  const dim3 block(kIdxWaves * kWave);
  unsigned groups = 1;
  int resident = 1;
  hipError_t e = hipSuccess;
  switch (bt.R) {
    case 1:
      if ((e = indexer_groups<1>(bt, &groups, &resident)) != hipSuccess) return e;
      hipLaunchKernelGGL(k_indexer<1>, dim3(groups), block, 0, s, v, bt, k_pool, k_scale,
                         pool_pages, table, kept, kept_count, scores, page_qmax, resident);
      break;
    case 2:
      if ((e = indexer_groups<2>(bt, &groups, &resident)) != hipSuccess) return e;
      hipLaunchKernelGGL(k_indexer<2>, dim3(groups), block, 0, s, v, bt, k_pool, k_scale,
                         pool_pages, table, kept, kept_count, scores, page_qmax, resident);
      break;
    case 3:
      if ((e = indexer_groups<3>(bt, &groups, &resident)) != hipSuccess) return e;
      hipLaunchKernelGGL(k_indexer<3>, dim3(groups), block, 0, s, v, bt, k_pool, k_scale,
                         pool_pages, table, kept, kept_count, scores, page_qmax, resident);
      break;
    case 4:
      if ((e = indexer_groups<4>(bt, &groups, &resident)) != hipSuccess) return e;
      hipLaunchKernelGGL(k_indexer<4>, dim3(groups), block, 0, s, v, bt, k_pool, k_scale,
                         pool_pages, table, kept, kept_count, scores, page_qmax, resident);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace spin
