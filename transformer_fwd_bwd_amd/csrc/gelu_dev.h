// GELU of the pages (GPT-2's tanh form), device code shared by the elementwise
// kernels and the few-row products' chunk sums ([GPT2-4, "Common mistakes"]).
#pragma once

#include <hip/hip_runtime.h>

namespace tfb {

// GELU of the pages, 0.5 x (1 + tanh(u)) with u = sqrt(2/pi) (x + 0.044715 x^3), in
// the equivalent form 0.5 (1 + tanh(u)) = s = 1 / (1 + e), e = exp(-2u): one hardware
// exponential and one reciprocal per element instead of a library tanh (these kernels
// are bound by their arithmetic).  With it 1 - tanh(u)^2 = 4 s (1 - s) and 1 - s = e s,
// both without cancellation for large |u|.
constexpr float GELU_C = 0.7978845608028654f;  // sqrt(2/pi)
__device__ __forceinline__ float gelu_s(float x, float& e) {
  const float u = GELU_C * (x + 0.044715f * x * x * x);
  e = __builtin_amdgcn_exp2f(u * -2.8853900817779268f);  // exp(-2u) = 2^(-2u log2 e)
  return __builtin_amdgcn_rcpf(1.f + e);
}

__device__ __forceinline__ float gelu_f(float x) {
  float e;
  return x * gelu_s(x, e);
}

__device__ __forceinline__ float gelu_grad(float x) {
  float e;
  const float s = gelu_s(x, e);
  const float oms = e == INFINITY ? 1.f : e * s;  // 1 - s
  return s + 2.f * x * s * oms * GELU_C * (1.f + 3.f * 0.044715f * x * x);
}

}  // namespace tfb
