// Query quantisation and the gather-indexer over the kept KV pages.
//
// k_quantize: per (request, row, head) the exponent e = smallest integer with
//   max|q| * 2^-e <= 448, codes = RNE e4m3fn(q * 2^-e) (exact scaling), and
//   wq = w * 2^e, so sum_h wq_h ReLU(q8_h . k) equals the bf16-query score up
//   to the rounding of q to e4m3fn.
// k_indexer: one wave per kept page (64 tokens x 128 fp8 = 8 KB, contiguous in
//   the pool); optionally also the page's maximum score per row, which lets
//   the top-k discard most candidates before ranking them.  Heads form the M side of v_mfma_scale_f32_16x16x128_f8f6f4 and
//   tokens the N side, so one MFMA does 16 heads x 16 tokens over the whole
//   head dim; a page is 4 head tiles x 4 token tiles per row.  ReLU, the head
//   weights and the head sum run on the accumulator registers, the 4 lane
//   groups are folded with two cross-lane adds, and every lane then holds the
//   score of token `lane`, stored as one coalesced 256-byte row.
#include "spin_device.h"
#include "spin_internal.h"

namespace spin {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kHeads = 64;
constexpr int kDim = 128;
#ifndef SPIN_IDX_PAGES_PER_WAVE
#define SPIN_IDX_PAGES_PER_WAVE 16
#endif
#ifndef SPIN_IDX_WAVES
#define SPIN_IDX_WAVES 4
#endif
#ifndef SPIN_IDX_NONTEMPORAL
#define SPIN_IDX_NONTEMPORAL 0
#endif
#ifndef SPIN_IDX_PREFETCH
#define SPIN_IDX_PREFETCH 1            // pages in flight ahead of the one on the MFMAs
#endif
#ifndef SPIN_IDX_NT_STORE
#define SPIN_IDX_NT_STORE 0            // streaming (non-temporal) score stores
#endif
#ifndef SPIN_IDX_WAVES_PER_EU
#define SPIN_IDX_WAVES_PER_EU 0        // occupancy target for the register allocator (0: none)
#endif
#if SPIN_IDX_WAVES_PER_EU > 0
#define SPIN_IDX_OCCUPANCY __attribute__((amdgpu_waves_per_eu(SPIN_IDX_WAVES_PER_EU)))
#else
#define SPIN_IDX_OCCUPANCY
#endif
constexpr int kIdxWaves = SPIN_IDX_WAVES;
constexpr int kPagesPerWave = SPIN_IDX_PAGES_PER_WAVE;

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

// 32 contiguous key bytes; keys are streamed once, so optionally non-temporal.
__device__ __forceinline__ v8i load32(const uint8_t* p) {
#if SPIN_IDX_NONTEMPORAL
  return __builtin_nontemporal_load(reinterpret_cast<const v8i*>(p));
#else
  return *reinterpret_cast<const v8i*>(p);
#endif
}

// grid (ceil(max_blocks / (4 * kPagesPerWave)), B), 256 threads.
// Wave w of workgroup x handles kept pages x*4*P + w + 4m, m < P = kPagesPerWave.
// The page metadata chain (kept entry -> block table -> scale) is issued first
// and overlaps the staging of the queries in LDS; the keys of page m+1 are in
// flight while page m runs on the MFMAs.
template <int R>
__global__ void __launch_bounds__(kIdxWaves * kWave) SPIN_IDX_OCCUPANCY
k_indexer(SpinView v, spin_batch bt, const uint8_t* __restrict__ k_pool,
          const float* __restrict__ k_scale, int64_t pool_pages, const int32_t* table,
          const int32_t* kept, const int32_t* kept_count, float* scores, float* page_max) {
  __shared__ __attribute__((aligned(16))) uint8_t s_q[R * kHeads * kDim];
  __shared__ float s_w[R * kHeads];
  const int b = blockIdx.y;
  int cnt = kept_count[b];
  if (cnt < 0 || cnt > bt.max_blocks) {
    if (blockIdx.x == 0 && threadIdx.x == 0) flag_error(v.err, SPIN_ERR_KEPT);
    cnt = cnt < 0 ? 0 : bt.max_blocks;
  }
  const int first = blockIdx.x * (kIdxWaves * kPagesPerWave);
  if (first >= cnt) return;

  const int l = lane_id();
  const int wave = threadIdx.x / kWave;
  const size_t mb = size_t(bt.max_blocks);

  // Page metadata for this wave's pages, lane m holding page m.
  int my_j = -1, my_p = -1;
  float my_sc = 0.0f;
  if (l < kPagesPerWave) {
    const int k = first + wave + kIdxWaves * l;
    if (k < cnt) {
      const int j = kept[size_t(b) * mb + k];
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
  }

  // Stage this request's quantised queries and head weights in LDS.
  const uint8_t* q8 = v.q8 + size_t(b) * v.max_rows * kHeads * kDim;
  const float* wq = v.wq + size_t(b) * v.max_rows * kHeads;
  for (int i = threadIdx.x; i < R * kHeads * kDim / 16; i += kIdxWaves * kWave)
    reinterpret_cast<uint4*>(s_q)[i] = reinterpret_cast<const uint4*>(q8)[i];
  for (int i = threadIdx.x; i < R * kHeads; i += kIdxWaves * kWave) s_w[i] = wq[i];

  const int q0 = bt.qpos[b];
  const int g = l >> 4;       // lane group: K chunk of the operands, M rows of the result
  const int n16 = l & 15;     // M row of A / N column of B
  const int npages = min(kPagesPerWave, (cnt - first - wave + kIdxWaves - 1) / kIdxWaves);

  constexpr int PF = SPIN_IDX_PREFETCH > 0 ? SPIN_IDX_PREFETCH : 1;
  constexpr bool kPrefetch = SPIN_IDX_PREFETCH > 0;
  v8i kb[4], kn[PF][4];
  auto load_page = [&](v8i* dst, int p) {
    const uint8_t* base = k_pool + size_t(p) * (kBlock * kDim) + g * 32;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) dst[tt] = load32(base + (tt * 16 + n16) * kDim);
  };
  if (kPrefetch) {
#pragma unroll
    for (int f = 0; f < PF; ++f) {
      const int pf = __builtin_amdgcn_readlane(my_p, f);
      if (f < npages && pf >= 0) load_page(kn[f], pf);
    }
  }
  __syncthreads();

#pragma unroll 1
  for (int m = 0; m < npages; ++m) {
    const int k = first + wave + kIdxWaves * m;
    const int j = __shfl(my_j, m, kWave);
    const float sc = __shfl(my_sc, m, kWave);
    if (kPrefetch) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) kb[tt] = kn[0][tt];
#pragma unroll
      for (int f = 0; f + 1 < PF; ++f)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) kn[f][tt] = kn[f + 1][tt];
      if (m + PF < npages) {
        const int pn = __shfl(my_p, m + PF, kWave);
        if (pn >= 0) load_page(kn[PF - 1], pn);
      }
    } else {
      const int pc = __shfl(my_p, m, kWave);
      if (pc >= 0) load_page(kb, pc);
    }
    if (j < 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        scores[(size_t(b) * R + r) * mb * kBlock + size_t(k) * kBlock + l] = -INFINITY;
        if (page_max && l == 0) page_max[(size_t(b) * R + r) * mb + k] = -INFINITY;
      }
      continue;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        const v8i qa = *reinterpret_cast<const v8i*>(s_q + ((r * kHeads + ht * 16 + n16) * kDim) + g * 32);
        const float4 wv = *reinterpret_cast<const float4*>(s_w + r * kHeads + ht * 16 + g * 4);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          v4f acc = {0.f, 0.f, 0.f, 0.f};
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa, kb[tt], acc, 0, 0, 0, 127, 0, 127);
          part[tt] += wv.x * fmaxf(acc[0], 0.f) + wv.y * fmaxf(acc[1], 0.f) +
                      wv.z * fmaxf(acc[2], 0.f) + wv.w * fmaxf(acc[3], 0.f);
        }
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        part[tt] += __shfl_xor(part[tt], 16, kWave);
        part[tt] += __shfl_xor(part[tt], 32, kWave);
      }
      const float val = g == 0 ? part[0] : g == 1 ? part[1] : g == 2 ? part[2] : part[3];
      const int slot = j * kBlock + l;
      const float out = (slot <= q0 + r) ? val * sc : -INFINITY;
      float* dst = scores + (size_t(b) * R + r) * mb * kBlock + size_t(k) * kBlock + l;
#if SPIN_IDX_NT_STORE
      __builtin_nontemporal_store(out, dst);
#else
      *dst = out;
#endif
      if (page_max) {
        const float m = wave_max(out);
        if (l == 0) page_max[(size_t(b) * R + r) * mb + k] = m;
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

hipError_t launch_indexer(const SpinView& v, const spin_batch& bt, const uint8_t* k_pool,
                          const float* k_scale, int64_t pool_pages, const int32_t* table,
                          const int32_t* kept, const int32_t* kept_count, float* scores,
                          float* page_max, hipStream_t s) {
  const int per_wg = kIdxWaves * kPagesPerWave;
  const dim3 grid(unsigned((bt.max_blocks + per_wg - 1) / per_wg), unsigned(bt.B));
  const dim3 block(kIdxWaves * kWave);
  switch (bt.R) {
    case 1:
      hipLaunchKernelGGL(k_indexer<1>, grid, block, 0, s, v, bt, k_pool, k_scale, pool_pages,
                         table, kept, kept_count, scores, page_max);
      break;
    case 2:
      hipLaunchKernelGGL(k_indexer<2>, grid, block, 0, s, v, bt, k_pool, k_scale, pool_pages,
                         table, kept, kept_count, scores, page_max);
      break;
    case 3:
      hipLaunchKernelGGL(k_indexer<3>, grid, block, 0, s, v, bt, k_pool, k_scale, pool_pages,
                         table, kept, kept_count, scores, page_max);
      break;
    case 4:
      hipLaunchKernelGGL(k_indexer<4>, grid, block, 0, s, v, bt, k_pool, k_scale, pool_pages,
                         table, kept, kept_count, scores, page_max);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace spin
