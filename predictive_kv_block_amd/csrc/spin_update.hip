// EMA update kernel: one launch over every request's kept list (the per-wave
// work is update_wave in spin_update.h).  The replay variant (acceptances
// given) carries the loads of the later rows; the plain update does not.
#include "spin_update.h"

namespace spin {
namespace {

constexpr int kUpdWaves = 4;
constexpr int kUpdBlocks = 4;     // kept entries per wave

template <bool kReplay>
__global__ void __launch_bounds__(kUpdWaves * kWave)
k_update(SpinView v, int layer, spin_batch bt, const int32_t* accepted, const float* scores,
         const int32_t* kept, const int32_t* kept_count) {
  const int w = threadIdx.x / kWave;
  update_wave<kUpdBlocks, kReplay>(v, layer, bt, accepted, scores, kept, kept_count, blockIdx.y,
                                   (blockIdx.x * kUpdWaves + w) * kUpdBlocks,
                                   blockIdx.x == 0 && threadIdx.x == 0);
}

}  // namespace

hipError_t launch_update(const SpinView& v, int layer, const spin_batch& bt,
                         const int32_t* accepted, const float* scores, const int32_t* kept,
                         const int32_t* kept_count, hipStream_t s) {
  const int per_wg = kUpdWaves * kUpdBlocks;
  const dim3 grid(unsigned((bt.max_blocks + per_wg - 1) / per_wg), unsigned(bt.B));
  if (accepted)
    hipLaunchKernelGGL(k_update<true>, grid, dim3(kUpdWaves * kWave), 0, s, v, layer, bt,
                       accepted, scores, kept, kept_count);
  else
    hipLaunchKernelGGL(k_update<false>, grid, dim3(kUpdWaves * kWave), 0, s, v, layer, bt,
                       accepted, scores, kept, kept_count);
  return hipGetLastError();
}

}  // namespace spin
