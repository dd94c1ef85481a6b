// State initialisation and slot reset: -inf marks "never observed".
#include "spin_device.h"
#include "spin_internal.h"

namespace spin {
namespace {

__global__ void __launch_bounds__(256) k_fill_f32(float* p, size_t n, float v) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

__global__ void __launch_bounds__(256) k_fill_u32(uint32_t* p, size_t n, uint32_t v) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

// grid: (chunks, n, L).  Each slot's rows of V, D and VB are set to -inf.
__global__ void __launch_bounds__(256) k_reset_slots(SpinView v, int n, const int32_t* slots,
                                                     const uint64_t* rids) {
  const int k = blockIdx.y;
  const int layer = blockIdx.z;
  const int s = slots[k];
  if (s < 0 || s >= v.S) {
    if (blockIdx.x == 0 && layer == 0 && threadIdx.x == 0) flag_error(v.err, SPIN_ERR_SLOT);
    return;
  }
  const size_t row = size_t(layer) * v.S + s;
  float* V = v.V + row * v.max_ctx;
  float* D = v.D + row * v.max_ctx;
  float* VB = v.VB + row * v.max_blocks;
  const int stride = gridDim.x * blockDim.x;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < v.max_ctx; i += stride) {
    V[i] = -INFINITY;
    D[i] = -INFINITY;
  }
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < v.max_blocks; i += stride)
    VB[i] = -INFINITY;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    v.step[row] = 0;
    if (layer == 0) v.rid[s] = rids[k];
  }
}

unsigned grid_for(size_t n) {
  size_t g = (n + 255) / 256;
  if (g > 16384) g = 16384;
  if (g == 0) g = 1;
  return unsigned(g);
}

}  // namespace

hipError_t launch_fill_state(const SpinView& v, hipStream_t s) {
  const size_t nv = size_t(v.L) * v.S * v.max_ctx;
  const size_t nb = size_t(v.L) * v.S * v.max_blocks;
  const size_t ns = size_t(v.L) * v.S;
  hipError_t e;
  hipLaunchKernelGGL(k_fill_f32, dim3(grid_for(nv)), dim3(256), 0, s, v.V, nv, -INFINITY);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_fill_f32, dim3(grid_for(nv)), dim3(256), 0, s, v.D, nv, -INFINITY);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_fill_f32, dim3(grid_for(nb)), dim3(256), 0, s, v.VB, nb, -INFINITY);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(ns)), dim3(256), 0, s,
                     reinterpret_cast<uint32_t*>(v.step), ns, 0u);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(2 * size_t(v.S))), dim3(256), 0, s,
                     reinterpret_cast<uint32_t*>(v.rid), 2 * size_t(v.S), 0u);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(256), 0, s, reinterpret_cast<uint32_t*>(v.err),
                     size_t(1), 0u);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(256), 0, s, reinterpret_cast<uint32_t*>(v.gate),
                     size_t(2), 0u);
  return hipGetLastError();
}

hipError_t launch_reset_slots(const SpinView& v, int n, const int32_t* slots,
                              const uint64_t* rids, hipStream_t s) {
  if (n == 0) return hipSuccess;
  unsigned chunks = unsigned((v.max_ctx + 256 * 16 - 1) / (256 * 16));
  if (chunks == 0) chunks = 1;
  hipLaunchKernelGGL(k_reset_slots, dim3(chunks, n, v.L), dim3(256), 0, s, v, n, slots, rids);
  return hipGetLastError();
}

}  // namespace spin
