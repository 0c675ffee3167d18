// Optimizer steps ([Autograd-1, "The Optimizer: from gradient to a step"]).
// AdamW updates every parameter in one launch: the host splits the parameter
// list into fixed-size chunks once; workgroup i updates chunk i (p, m, v read
// and written once, g read once: 28 bytes per parameter).
#include <algorithm>

#include "kernels.h"

namespace tfb {
namespace {

typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void adam_one(float& p, float g, float& m, float& v, float lr, float b1, float b2,
                                         float eps, float bc1, float bc2, float wd) {
  m = b1 * m + (1.f - b1) * g;
  v = b2 * v + (1.f - b2) * g * g;
  const float mhat = m / bc1, vhat = v / bc2;
  p -= lr * (mhat / (sqrtf(vhat) + eps) + wd * p);
}

__global__ __launch_bounds__(NT) void adamw_k(const AdamSeg* __restrict__ segs, const AdamChunk* __restrict__ chunks,
                                              int64_t chunk_elems, float lr, float b1, float b2, float eps,
                                              float bc1, float bc2) {
  const AdamChunk ch = chunks[blockIdx.x];
  const AdamSeg sg = segs[ch.seg];
  const int64_t end = std::min(sg.n, ch.off + chunk_elems);
  const bool v4 = ((reinterpret_cast<uintptr_t>(sg.p) | reinterpret_cast<uintptr_t>(sg.g) |
                    reinterpret_cast<uintptr_t>(sg.m) | reinterpret_cast<uintptr_t>(sg.v)) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(sg.pbf) & 7) == 0;
  int64_t i = ch.off;
  if (v4) {
    const int64_t end4 = ch.off + ((end - ch.off) / 4) * 4;
    for (int64_t q = ch.off + 4 * (int64_t)threadIdx.x; q < end4; q += 4 * NT) {
      f4 p = *reinterpret_cast<f4*>(sg.p + q);
      const f4 g = *reinterpret_cast<const f4*>(sg.g + q);
      f4 m = *reinterpret_cast<f4*>(sg.m + q);
      f4 v = *reinterpret_cast<f4*>(sg.v + q);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pe = p[e], me = m[e], ve = v[e];
        adam_one(pe, g[e], me, ve, lr, b1, b2, eps, bc1, bc2, sg.wd);
        p[e] = pe;
        m[e] = me;
        v[e] = ve;
      }
      *reinterpret_cast<f4*>(sg.p + q) = p;
      *reinterpret_cast<f4*>(sg.m + q) = m;
      *reinterpret_cast<f4*>(sg.v + q) = v;
      if (sg.pbf) {
        u16x4 b;
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = __builtin_bit_cast(uint16_t, (__bf16)p[e]);
        *reinterpret_cast<u16x4*>(sg.pbf + q) = b;
      }
    }
    i = end4;
  }
  for (int64_t q = i + threadIdx.x; q < end; q += NT) {
    float p = sg.p[q], m = sg.m[q], v = sg.v[q];
    adam_one(p, sg.g[q], m, v, lr, b1, b2, eps, bc1, bc2, sg.wd);
    sg.p[q] = p;
    sg.m[q] = m;
    sg.v[q] = v;
    if (sg.pbf) sg.pbf[q] = __builtin_bit_cast(uint16_t, (__bf16)p);
  }
}

__global__ void sgd_k(float* __restrict__ p, const float* __restrict__ g, float lr, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) p[i] -= lr * g[i];
}

}  // namespace

hipError_t adamw_step(const AdamSeg* segs, const AdamChunk* chunks, int nchunks, int64_t chunk_elems, float lr,
                      float b1, float b2, float eps, float bc1, float bc2, hipStream_t s) {
  if (nchunks <= 0) return hipSuccess;
  run_kernel(adamw_k, dim3(nchunks), dim3(NT), 0, s, segs, chunks, chunk_elems, lr, b1, b2, eps, bc1, bc2);
  return hipGetLastError();
}

hipError_t sgd_step(float* p, const float* g, float lr, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<int64_t>((n + NT - 1) / NT, 65536);
  run_kernel(sgd_k, dim3(blocks), dim3(NT), 0, s, p, g, lr, n);
  return hipGetLastError();
}

}  // namespace tfb
