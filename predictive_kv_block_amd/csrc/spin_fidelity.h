// Launchers of the selection-fidelity kernels (spin_fidelity.hip).
#pragma once

#include "spin_internal.h"

namespace spin {

hipError_t launch_slot_scores(const SpinView& v, int layer, const spin_batch& bt, float* z,
                              hipStream_t s);
hipError_t launch_estimate_miss(const spin_batch& bt, int topk, const float* scores,
                                const int32_t* kept, const int32_t* kept_count,
                                const int32_t* topk_out, const uint8_t* flags, float* est,
                                hipStream_t s);
hipError_t launch_predictor_fidelity(const spin_batch& bt, int topk, const float* pred,
                                     const float* actual, const int32_t* pred_topk,
                                     const int32_t* actual_topk, double* out, hipStream_t s);

}  // namespace spin
