// Device helpers for the gfx950 kernels of libpagedkv.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pa {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7-i inside each 8
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15-i inside each 16

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N = 4, 8, 16, 32); every lane of the
// group ends with the group's total. Groups of up to 16 lanes stay inside one
// DPP row; 32 adds one cross-row step through the LDS crossbar.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group size");
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  if constexpr (N >= 8) v += dpp<kDppRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kDppRowMirror>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<kDppQuadXor1>(v));
  v = fmaxf(v, dpp<kDppQuadXor2>(v));
  v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp<kDppRowMirror>(v));
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ h2_t as_h2(uint32_t w) { return __builtin_bit_cast(h2_t, w); }

__device__ __forceinline__ float lo_f16(uint32_t w) { return float(as_h2(w).x); }
__device__ __forceinline__ float hi_f16(uint32_t w) { return float(as_h2(w).y); }

// Signed byte k (0..3) of w, as float (exact).
template <int k>
__device__ __forceinline__ float i8_at(uint32_t w) {
  return float(int32_t(w << (24 - 8 * k)) >> 24);
}

__device__ __forceinline__ void flag_error(int32_t* err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

}  // namespace pa
