// Cross-lane moves on gfx950 without an LDS round trip.
//
// v_permlane32_swap exchanges the upper 32 lanes of its first operand with the
// lower 32 lanes of its second; given the same value twice it returns (low half
// in both halves, high half in both halves), whose element sum in a lane is
// v[l] + v[l ^ 32].  v_permlane16_swap does the same for odd and even 16-lane
// rows: v[l] + v[l ^ 16].  (Lane layouts checked on the device.)
#pragma once

#include <hip/hip_runtime.h>

namespace tfb {

__device__ __forceinline__ float lanes_xor32_add(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float lanes_xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float lanes_xor16_add(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float lanes_xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace tfb
