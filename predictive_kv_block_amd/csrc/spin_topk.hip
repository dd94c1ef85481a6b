// Per-row top-k over the kept-order indexer scores, and the miss measurement.
//
// k_topk: one 1024-thread workgroup per (request, row).  Candidates are the
//   kept slots at or before the row's position.  The K-th largest key is found
//   by MSB-first 8-bit radix passes over an LDS histogram; the selected slots
//   (key above the threshold, or equal to it and among the first n_eq such
//   slots) are emitted by a per-wave ordered ballot pass.  Kept order is
//   ascending in position, so the output comes out sorted and ties go to the
//   lower position.
// k_miss: share of an all-keep top-k that falls in skipped blocks.
#include "spin_device.h"
#include "spin_internal.h"
#include "spin_select.h"

namespace spin {
namespace {

constexpr int kTopkThreads = 1024;

struct ScoreRowSrc {
  const float* s;
  const int32_t* kept;
  int qr;
  int max_blocks;
  __device__ bool get(int x, uint32_t& key) const {
    const int j = kept[x >> 6];
    const int slot = j * kBlock + (x & 63);
    if (j < 0 || j >= max_blocks || slot > qr) return false;
    key = ord_key(s[x]);
    return true;
  }
};

__global__ void __launch_bounds__(kTopkThreads)
k_topk(spin_batch bt, int K, const float* scores, const int32_t* kept,
       const int32_t* kept_count, int32_t* out) {
  __shared__ int s_scr[kSelectScratchInts];
  const int b = blockIdx.x / bt.R, r = blockIdx.x % bt.R;
  const size_t mb = size_t(bt.max_blocks);
  int cnt = kept_count[b];
  cnt = cnt < 0 ? 0 : (cnt > bt.max_blocks ? bt.max_blocks : cnt);
  const int n = cnt * kBlock;
  const int32_t* kb = kept + size_t(b) * mb;
  ScoreRowSrc src{scores + (size_t(b) * bt.R + r) * mb * kBlock, kb, bt.qpos[b] + r,
                  bt.max_blocks};
  int32_t* o = out + (size_t(b) * bt.R + r) * K;

  const int nvalid = count_valid<kTopkThreads, 8, uint32_t>(src, n, s_scr);
  const int want = min(K, nvalid);
  uint32_t thr = 0;
  int neq = 0x7fffffff;
  if (want > 0 && want < nvalid)
    radix_threshold<kTopkThreads, 8, uint32_t>(src, n, want, &thr, &neq, s_scr);
  int total = 0;
  if (want > 0)
    total = ordered_emit<kTopkThreads, 4, uint32_t>(
        src, n, thr, neq,
        [&](int x, int rank) {
          if (rank < K) o[rank] = kb[x >> 6] * kBlock + (x & 63);
        },
        s_scr);
  for (int i = min(total, K) + threadIdx.x; i < K; i += kTopkThreads) o[i] = -1;
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

}  // namespace

hipError_t launch_topk(const spin_batch& bt, int topk, const float* scores, const int32_t* kept,
                       const int32_t* kept_count, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_topk, dim3(bt.B * bt.R), dim3(kTopkThreads), 0, s, bt, topk, scores, kept,
                     kept_count, out);
  return hipGetLastError();
}

hipError_t launch_miss(const spin_batch& bt, int topk, const int32_t* full_topk,
                       const uint8_t* flags, float* miss, hipStream_t s) {
  hipLaunchKernelGGL(k_miss, dim3(bt.B * bt.R), dim3(256), 0, s, bt, topk, full_topk, flags,
                     miss);
  return hipGetLastError();
}

}  // namespace spin
