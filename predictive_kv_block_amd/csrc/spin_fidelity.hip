// Selection fidelity on the device: the predicted slot scores themselves, an
// online miss estimate from the exploration blocks' top-k hits, and the
// quality of a slot predictor against the indexer (Pearson correlation and
// top-k recall, the two columns of Table 1 of the v1 listing "SPIN: Shadow
// Predictive Indexer for Sparse Attention").  None of these is on the
// decode round's path; they measure it.
#include "spin_device.h"
#include "spin_fidelity.h"

namespace spin {
namespace {

constexpr int kSlotThreads = 256;
constexpr int kSlotsPerThread = 4;
constexpr int kEstThreads = 1024;
constexpr int kFidThreads = 1024;

// z_i = max(V_i, D_{q+r-i}) for i <= q + r, -inf for the rest of the row.
// grid (ceil(max_blocks * 64 / 1024), B, R); out rows are max_blocks * 64 long.
__global__ void __launch_bounds__(kSlotThreads)
k_slot_scores(SpinView v, int layer, spin_batch bt, float* out) {
  const int b = blockIdx.y, r = blockIdx.z;
  const int s = bt.slot[b];
  const int q0 = bt.qpos[b];
  if (s < 0 || s >= v.S || q0 < 0 || q0 + bt.R - 1 >= v.max_ctx ||
      num_blocks_of(q0 + bt.R - 1) > bt.max_blocks) {
    if (blockIdx.x == 0 && r == 0 && threadIdx.x == 0)
      flag_error(v.err, (s < 0 || s >= v.S) ? SPIN_ERR_SLOT : SPIN_ERR_QPOS);
    return;
  }
  const size_t row = size_t(layer) * v.S + s;
  const float* V = v.V + row * v.max_ctx;
  const float* D = v.D + row * v.max_ctx;
  const int n = bt.max_blocks * kBlock;
  const int q = q0 + r;
  float* o = out + (size_t(b) * bt.R + r) * n;
  const int base = blockIdx.x * (kSlotThreads * kSlotsPerThread) + threadIdx.x;
#pragma unroll
  for (int u = 0; u < kSlotsPerThread; ++u) {
    const int i = base + u * kSlotThreads;
    if (i < n) o[i] = (i <= q) ? fmaxf(V[i], D[q - i]) : -INFINITY;
  }
}

// Sum of three counters over the workgroup; thread 0 gets the totals.
template <int NT>
__device__ void block_sum3(int& a, int& b, int& c, int* s_buf) {
  a = wave_sum(a);
  b = wave_sum(b);
  c = wave_sum(c);
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) {
    s_buf[3 * w] = a;
    s_buf[3 * w + 1] = b;
    s_buf[3 * w + 2] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a = b = c = 0;
    for (int i = 0; i < NT / kWave; ++i) {
      a += s_buf[3 * i];
      b += s_buf[3 * i + 1];
      c += s_buf[3 * i + 2];
    }
  }
}

// Inclusive prefix sum over the workgroup of one int per thread, in thread
// order; s_buf holds NT / 64 ints.
template <int NT>
__device__ int block_inclusive_sum(int x, int* s_buf) {
  const int l = lane_id(), w = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(x, o, kWave);
    if (l >= o) x += t;
  }
  if (l == kWave - 1) s_buf[w] = x;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += s_buf[i];
  __syncthreads();
  return x + before;
}

constexpr int kEstMaxK = 4096;
constexpr int kEstPerThread = kEstMaxK / kEstThreads;

// One workgroup per (request, row).  Skipped / explored blocks among the
// row's N_r blocks; the sparse top-k's entries as 64-bit keys (score order,
// then lower position first, then an explored bit), sorted descending in
// LDS; the weighted walk (|E| per predicted slot, |U| per explored slot,
// target k_r * |E|) stops at the first entry whose running weight reaches the
// target, and the explored entries up to it give the estimate; all explored
// entries give the upper bound.  Ratios in fp64, rounded to fp32.
__global__ void __launch_bounds__(kEstThreads)
k_estimate_miss(spin_batch bt, int K, const float* scores, const int32_t* kept,
                const int32_t* kept_count, const int32_t* topk, const uint8_t* flags,
                float* est) {
  __shared__ uint64_t s_key[kEstMaxK];
  __shared__ int s_buf[3 * (kEstThreads / kWave)];
  __shared__ int s_bc[4];
  const int row = blockIdx.x;
  const int b = row / bt.R, r = row - b * bt.R;
  const int q0 = bt.qpos[b];
  const int tid = threadIdx.x;
  if (q0 < 0 || q0 > bt.max_blocks * kBlock - bt.R) {
    if (tid == 0) est[2 * size_t(row)] = est[2 * size_t(row) + 1] = __builtin_nanf("");
    return;
  }
  const int q = q0 + r;
  const int n = num_blocks_of(q);
  const uint8_t* f = flags + size_t(b) * bt.max_blocks;
  const int32_t* kl = kept + size_t(b) * bt.max_blocks;
  int cnt = kept_count[b];
  cnt = cnt < 0 ? 0 : (cnt > bt.max_blocks ? bt.max_blocks : cnt);
  const float* sc = scores + size_t(row) * bt.max_blocks * kBlock;
  const int32_t* t = topk + size_t(row) * K;

  int skipped = 0, explored = 0, unused = 0;
  for (int j = tid; j < n; j += kEstThreads) {
    const uint8_t x = f[j];
    skipped += x == 0 ? 1 : 0;
    explored += x == 2 ? 1 : 0;
  }
  block_sum3<kEstThreads>(skipped, explored, unused, s_buf);
  if (tid == 0) {
    s_bc[0] = skipped;
    s_bc[1] = explored;
  }
  __syncthreads();
  skipped = s_bc[0];
  explored = s_bc[1];
  if (skipped == 0 || explored == 0) {
    if (tid == 0) est[2 * size_t(row)] = est[2 * size_t(row) + 1] = skipped == 0 ? 0.0f : -1.0f;
    return;
  }

  // keys of the valid entries (0 for the rest, which sort last)
  int np2 = 1;
  while (np2 < K) np2 <<= 1;
  for (int e = tid; e < np2; e += kEstThreads) {
    uint64_t key = 0;
    const int p = e < K ? t[e] : -1;
    if (p >= 0 && p <= q) {
      const int blk = p / kBlock;
      const uint8_t fl = f[blk];
      int lo = 0, hi = cnt;                // first kept index with kl >= blk
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (kl[mid] < blk) lo = mid + 1; else hi = mid;
      }
      if (fl != 0 && lo < cnt && kl[lo] == blk) {
        const float v = sc[size_t(lo) * kBlock + (p & (kBlock - 1))] + 0.0f;
        key = (uint64_t(ord_key(v)) << 32) | (uint64_t(0x3FFFFF - p) << 1) | (fl == 2 ? 1u : 0u);
      }
    }
    s_key[e] = key;
  }
  __syncthreads();
  // bitonic sort, descending
  for (int size = 2; size <= np2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int e = tid; e < np2 / 2; e += kEstThreads) {
        const int lo = 2 * stride * (e / stride) + (e % stride);
        const int hi = lo + stride;
        const bool desc = ((lo & size) == 0);
        const uint64_t a = s_key[lo], c = s_key[hi];
        if ((a < c) == desc) {
          s_key[lo] = c;
          s_key[hi] = a;
        }
      }
      __syncthreads();
    }
  }

  // weighted walk: thread i owns sorted entries [i * PT, i * PT + PT)
  const int n_u = skipped + explored;
  const int k_r = min(K, q + 1);
  const int target = k_r * explored;
  int wsum = 0, esum = 0;
  int wt[kEstPerThread];
  bool ise[kEstPerThread];
#pragma unroll
  for (int u = 0; u < kEstPerThread; ++u) {
    const int e = tid * kEstPerThread + u;
    const uint64_t key = e < np2 ? s_key[e] : 0;
    ise[u] = key != 0 && (key & 1u);
    wt[u] = key == 0 ? 0 : (ise[u] ? n_u : explored);
    wsum += wt[u];
    esum += ise[u] ? 1 : 0;
  }
  if (tid == 0) s_bc[2] = 0x7fffffff;
  const int incl = block_inclusive_sum<kEstThreads>(wsum, s_buf);
  int run = incl - wsum;
#pragma unroll
  for (int u = 0; u < kEstPerThread; ++u) {
    run += wt[u];
    if (wt[u] != 0 && run >= target) {
      atomicMin(&s_bc[2], tid * kEstPerThread + u);
      break;
    }
  }
  __syncthreads();
  const int stop = s_bc[2];
  int c_e = 0;
#pragma unroll
  for (int u = 0; u < kEstPerThread; ++u)
    c_e += (ise[u] && tid * kEstPerThread + u <= stop) ? 1 : 0;
  int h = esum, z = 0;
  block_sum3<kEstThreads>(c_e, h, z, s_buf);
  if (tid == 0) {
    const double den = double(explored) * double(k_r);
    const double a = double(c_e) * double(skipped) / den;
    const double c = double(h) * double(skipped) / den;
    est[2 * size_t(row)] = float(a < 1.0 ? a : 1.0);
    est[2 * size_t(row) + 1] = float(c < 1.0 ? c : 1.0);
  }
}

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

__device__ __forceinline__ float wave_min_f(float x) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) x = fminf(x, __shfl_xor(x, o, kWave));
  return x;
}

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}

// Workgroup sums of N doubles in a fixed order (waves in index order); every
// thread gets the totals.
template <int N>
__device__ void block_sum_d(double (&x)[N], double* s_buf) {
  constexpr int NW = kFidThreads / kWave;
#pragma unroll
  for (int k = 0; k < N; ++k) x[k] = wave_sum_d(x[k]);
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0)
#pragma unroll
    for (int k = 0; k < N; ++k) s_buf[k * NW + w] = x[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < N; ++k) {
    double t = 0.0;
    for (int i = 0; i < NW; ++i) t += s_buf[k * NW + i];
    x[k] = t;
  }
  __syncthreads();
}

// One workgroup per (request, row) over slots 0..q+r where both the
// prediction and the indexer score are finite: Pearson correlation by two
// fp64 passes (means, then centred sums), 0 when fewer than 2 slots remain
// or either side is constant on them; recall = shared entries of the two
// ascending top-k lists over the valid entries of the actual one.
__global__ void __launch_bounds__(kFidThreads)
k_predictor_fidelity(spin_batch bt, int K, const float* pred, const float* actual,
                     const int32_t* pred_topk, const int32_t* actual_topk, double* out) {
  constexpr int NW = kFidThreads / kWave;
  __shared__ double s_d[3 * NW];
  __shared__ float s_f[4 * NW];
  __shared__ int s_i[3 * (kFidThreads / kWave)];
  const int row = blockIdx.x;
  const int b = row / bt.R, r = row - b * bt.R;
  const int q0 = bt.qpos[b];
  if (q0 < 0 || q0 > bt.max_blocks * kBlock - bt.R) {
    if (threadIdx.x == 0) {
      out[2 * size_t(row)] = __builtin_nan("");
      out[2 * size_t(row) + 1] = __builtin_nan("");
    }
    return;
  }
  const int q = q0 + r;
  const size_t n = size_t(bt.max_blocks) * kBlock;
  const float* x = pred + size_t(row) * n;
  const float* y = actual + size_t(row) * n;

  double m1[3] = {0.0, 0.0, 0.0};          // count, sum x, sum y
  float xlo = INFINITY, xhi = -INFINITY, ylo = INFINITY, yhi = -INFINITY;
  for (int i = threadIdx.x; i <= q; i += kFidThreads) {
    const float a = x[i], c = y[i];
    if (__builtin_isfinite(a) && __builtin_isfinite(c)) {
      m1[0] += 1.0;
      m1[1] += double(a);
      m1[2] += double(c);
      xlo = fminf(xlo, a);
      xhi = fmaxf(xhi, a);
      ylo = fminf(ylo, c);
      yhi = fmaxf(yhi, c);
    }
  }
  xlo = wave_min_f(xlo);
  xhi = wave_max_f(xhi);
  ylo = wave_min_f(ylo);
  yhi = wave_max_f(yhi);
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) {
    s_f[w] = xlo;
    s_f[NW + w] = xhi;
    s_f[2 * NW + w] = ylo;
    s_f[3 * NW + w] = yhi;
  }
  block_sum_d(m1, s_d);                    // synchronises, so s_f is complete
  for (int i = 0; i < NW; ++i) {
    xlo = fminf(xlo, s_f[i]);
    xhi = fmaxf(xhi, s_f[NW + i]);
    ylo = fminf(ylo, s_f[2 * NW + i]);
    yhi = fmaxf(yhi, s_f[3 * NW + i]);
  }
  const double cnt = m1[0];
  double corr = 0.0;
  if (cnt >= 2.0 && xlo < xhi && ylo < yhi) {
    const double mx = m1[1] / cnt, my = m1[2] / cnt;
    double m2[3] = {0.0, 0.0, 0.0};        // sum dx^2, sum dy^2, sum dx dy
    for (int i = threadIdx.x; i <= q; i += kFidThreads) {
      const float a = x[i], c = y[i];
      if (__builtin_isfinite(a) && __builtin_isfinite(c)) {
        const double dx = double(a) - mx, dy = double(c) - my;
        m2[0] += dx * dx;
        m2[1] += dy * dy;
        m2[2] += dx * dy;
      }
    }
    block_sum_d(m2, s_d);
    corr = m2[2] / sqrt(m2[0] * m2[1]);
  }

  // recall: the valid entries of an ascending, -1 padded list are its prefix
  const int32_t* tp = pred_topk + size_t(row) * K;
  const int32_t* ta = actual_topk + size_t(row) * K;
  int na = 0, hits = 0, unused = 0;
  for (int e = threadIdx.x; e < K; e += kFidThreads) na += ta[e] >= 0 ? 1 : 0;
  block_sum3<kFidThreads>(na, hits, unused, s_i);
  __syncthreads();
  if (threadIdx.x == 0) s_i[0] = na;
  __syncthreads();
  na = s_i[0];
  __syncthreads();
  for (int e = threadIdx.x; e < K; e += kFidThreads) {
    const int p = tp[e];
    if (p < 0) continue;
    int lo = 0, hi = na;                   // first index with ta >= p
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (ta[mid] < p) lo = mid + 1; else hi = mid;
    }
    hits += (lo < na && ta[lo] == p) ? 1 : 0;
  }
  int z0 = 0, z1 = 0;
  block_sum3<kFidThreads>(hits, z0, z1, s_i);
  if (threadIdx.x == 0) {
    out[2 * size_t(row)] = corr;
    out[2 * size_t(row) + 1] = na > 0 ? double(hits) / double(na) : 0.0;
  }
}

}  // namespace

hipError_t launch_slot_scores(const SpinView& v, int layer, const spin_batch& bt, float* z,
                              hipStream_t s) {
  const int n = bt.max_blocks * kBlock;
  const int per = kSlotThreads * kSlotsPerThread;
  hipLaunchKernelGGL(k_slot_scores, dim3(unsigned((n + per - 1) / per), bt.B, bt.R),
                     dim3(kSlotThreads), 0, s, v, layer, bt, z);
  return hipGetLastError();
}

hipError_t launch_estimate_miss(const spin_batch& bt, int topk, const float* scores,
                                const int32_t* kept, const int32_t* kept_count,
                                const int32_t* topk_out, const uint8_t* flags, float* est,
                                hipStream_t s) {
  if (topk > kEstMaxK) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_estimate_miss, dim3(bt.B * bt.R), dim3(kEstThreads), 0, s, bt, topk,
                     scores, kept, kept_count, topk_out, flags, est);
  return hipGetLastError();
}

hipError_t launch_predictor_fidelity(const spin_batch& bt, int topk, const float* pred,
                                     const float* actual, const int32_t* pred_topk,
                                     const int32_t* actual_topk, double* out, hipStream_t s) {
  hipLaunchKernelGGL(k_predictor_fidelity, dim3(bt.B * bt.R), dim3(kFidThreads), 0, s, bt, topk,
                     pred, actual, pred_topk, actual_topk, out);
  return hipGetLastError();
}

}  // namespace spin
