// HBM probes for the indexer's access pattern, without its arithmetic: a
// gather of whole 8 KB key pages named by a page list, read in the indexer's
// lane layout, optionally with the indexer's write stream (one 256-byte row
// per page).  Measurement only: bench.py --ceilings times them to show what
// this part sustains for a page gather alone and for the same gather with a
// 3% write stream beside it.  Built as its own library, libspin_probe.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kPageBytes = 8192;      // 64 tokens x 128 fp8 keys
constexpr int kLoads = kPageBytes / (kWave * 16);   // 16-byte loads per lane per page
constexpr int kInFlight = 4;          // pages whose loads are issued together

typedef float v4f __attribute__((ext_vector_type(4)));

// grid G x 256 threads: wave gw of the 4G waves takes list entries
// [n gw / 4G, n (gw + 1) / 4G).  Lane l reads bytes 16 l + 1024 i of each page
// (i = 0..7), kInFlight pages at a time.  With `rows`, page m also writes 64
// floats (lane l: one) to rows[64 m + l] with a streaming store; every wave
// writes one float to sink[gw] at the end, so no load can be dropped.  Entries
// outside [0, pool_pages) read page 0.
__global__ void __launch_bounds__(kWaves * kWave)
k_probe_page_read(const uint8_t* __restrict__ pool, int64_t pool_pages,
                  const int32_t* __restrict__ list, int64_t n, float* rows, float* sink) {
  const int l = threadIdx.x & (kWave - 1);
  const int64_t W = int64_t(gridDim.x) * kWaves;
  const int64_t gw = int64_t(blockIdx.x) * kWaves + threadIdx.x / kWave;
  const int64_t m0 = n * gw / W, m1 = n * (gw + 1) / W;
  uint32_t acc = 0;
  for (int64_t m = m0; m < m1; m += kInFlight) {
    uint4 v[kInFlight][kLoads];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      int64_t p = 0;
      if (m + u < m1) {
        const int32_t e = list[m + u];
        p = (e >= 0 && int64_t(e) < pool_pages) ? e : 0;
      }
      const uint8_t* base = pool + p * kPageBytes + 16 * l;
#pragma unroll
      for (int i = 0; i < kLoads; ++i)
        v[u][i] = *reinterpret_cast<const uint4*>(base + i * (kWave * 16));
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      uint32_t x = 0;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) x ^= v[u][i].x ^ v[u][i].y ^ v[u][i].z ^ v[u][i].w;
      if (rows != nullptr && m + u < m1)
        __builtin_nontemporal_store(float(x & 0xFFFF), rows + (m + u) * kWave + l);
      acc ^= x;
    }
  }
  if (l == 0) sink[gw] = float(acc & 0xFFFF);
}

}  // namespace

// Gathers n pages of 8192 bytes from pool (pool_pages of them) in the order of
// list (device int32 [n]); rows (device float [n][64], or null) receives one
// 256-byte row per page; sink (device float, at least the returned number of
// waves) receives one value per wave.  Every pointer is a device pointer the
// caller owns.  Enqueues on `stream` and returns the HIP status; *waves (host)
// gets the number of waves launched.  The grid is 4 dispatch rounds of the
// device's resident workgroups, as the indexer's.
extern "C" int spin_probe_page_read(const void* pool, int64_t pool_pages, const int32_t* list,
                                    int64_t n, float* rows, float* sink, int64_t sink_len,
                                    int64_t* waves, hipStream_t stream) {
  if (pool == nullptr || list == nullptr || sink == nullptr || waves == nullptr || n < 0 ||
      pool_pages < 1)
    return int(hipErrorInvalidValue);
  static std::atomic<int> resident{0};
  int cap = resident.load(std::memory_order_relaxed);
  if (cap <= 0) {
    int per_cu = 0, cus = 0, dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_probe_page_read,
                                                       kWaves * kWave, 0);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return int(e);
    cap = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
    resident.store(cap, std::memory_order_relaxed);
  }
  const int64_t groups = int64_t(cap) * 4;
  *waves = groups * kWaves;
  if (sink_len < *waves) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(k_probe_page_read, dim3(unsigned(groups)), dim3(kWaves * kWave), 0, stream,
                     static_cast<const uint8_t*>(pool), pool_pages, list, n, rows, sink);
  return int(hipGetLastError());
}
