// Device-side helpers of the SPIN kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spin {

constexpr int kBlock = 64;       // slots per logical KV block (= page)
constexpr int kWave = 64;

// ---------------------------------------------------------------- float keys
// Order-preserving map of fp32 to uint32 (larger float -> larger key), with
// -0.0 folded onto +0.0 so that ReLU zeros of either sign compare equal.
__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------ wave reductions
// DPP data movement within a wave64: quad permutes, row mirrors and the row
// broadcasts of lanes 15 and 31 fold all 64 lanes into lane 63, which is then
// read back as a scalar (no LDS round trips).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;            // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;            // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

__device__ __forceinline__ float wave_max(float v) {
  int x = __float_as_int(v);
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp<kDppXor1, 0xF>(x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp<kDppXor2, 0xF>(x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp<kDppRowHalfMirror, 0xF>(x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp<kDppRowMirror, 0xF>(x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp<kDppRowBcast15, 0xA>(x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp<kDppRowBcast31, 0xC>(x))));
  return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}

__device__ __forceinline__ int wave_sum(int v) {
  v += dpp<kDppXor1, 0xF>(v);
  v += dpp<kDppXor2, 0xF>(v);
  v += dpp<kDppRowHalfMirror, 0xF>(v);
  v += dpp<kDppRowMirror, 0xF>(v);
  v += dpp<kDppRowBcast15, 0xA>(v);
  v += dpp<kDppRowBcast31, 0xC>(v);
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Number of set bits of a 64-lane ballot below this lane (v_mbcnt).
__device__ __forceinline__ int ballot_rank(uint64_t ballot) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(ballot >> 32),
                                   __builtin_amdgcn_mbcnt_lo(uint32_t(ballot), 0u));
}

// ------------------------------------------------------------------- Philox
// Philox4x64-10 counter-based generator, as published by Salmon, Moraes,
// Dror and Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC'11):
// ten rounds, each multiplying words 0 and 2 by fixed odd constants, mixing
// the high halves with the key, and bumping the key by Weyl increments
// between rounds.
struct Philox4x64 {
  uint64_t w[4];
};

__device__ __forceinline__ Philox4x64 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2,
                                                    uint64_t c3, uint64_t k0, uint64_t k1) {
  const uint64_t m0 = 0xD2E7470EE14C6C93ull, m1 = 0xCA5A826395121157ull;
  const uint64_t w0 = 0x9E3779B97F4A7C15ull, w1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round) {
      k0 += w0;
      k1 += w1;
    }
    const uint64_t lo0 = m0 * c0, hi0 = __umul64hi(m0, c0);
    const uint64_t lo1 = m1 * c2, hi1 = __umul64hi(m1, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0;
    const uint64_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  Philox4x64 r;
  r.w[0] = c0;
  r.w[1] = c1;
  r.w[2] = c2;
  r.w[3] = c3;
  return r;
}

// Histogram increment for a wave: every lane with `on` adds 1 to hist[digit].
// When every active lane has the same digit (keys concentrated in one bin),
// one lane adds the whole count; otherwise each lane issues its own LDS atomic.
__device__ __forceinline__ void hist_add(int* hist, int digit, bool on) {
  const uint64_t act = __ballot(on);
  if (act == 0) return;
  const int d0 = __builtin_amdgcn_readlane(digit, __ffsll(static_cast<unsigned long long>(act)) - 1);
  const uint64_t other = __ballot(on && digit != d0);
  if (other == 0) {
    if (lane_id() == __ffsll(static_cast<unsigned long long>(act)) - 1) atomicAdd(&hist[d0], __popcll(act));
  } else if (on) {
    atomicAdd(&hist[digit], 1);
  }
}

// ---------------------------------------------------------------------- misc
__device__ __forceinline__ int num_blocks_of(int qpos) { return (qpos + kBlock) / kBlock; }

__device__ __forceinline__ void flag_error(int32_t* err, int bit) {
  if (err) atomicOr(err, bit);
}

// EMA observation: never-observed (-inf) takes the sample, else
// alpha * x + beta * s in fp32.
__device__ __forceinline__ float ema_observe(float x, float s, float alpha, float beta) {
  return (x == -INFINITY) ? s : fmaf(alpha, x, beta * s);
}

}  // namespace spin
