// Column reductions of per-slab partials (device code shared by the kernels that
// run them one at a time and by the batched launch at the end of a backward pass).
// Each adds the partials of a column in one fixed order, so the result is the same
// whichever way it is launched.  1024 threads per workgroup; bx is the column block.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tfb {

// LayerNorm parameter gradients (and the column sums of dx): part holds np planes of
// C columns per slab (dgamma, dbeta[, dx]); 16 columns x 64 slab groups per workgroup
__device__ inline void ln_reduce_cols(const float* __restrict__ part, int nparts, int np, int C,
                                      float* __restrict__ dgamma, float* __restrict__ dbeta,
                                      float* __restrict__ dxsum, float beta_dg, float beta_db, int bx) {
  // 16 columns x 64 partial groups per workgroup; the groups are added in a fixed order
  __shared__ float sa[64][17], sb[64][17], sd[64][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int c = bx * 16 + tx;
  float a = 0.f, b = 0.f, d = 0.f;
  if (c < C) {
    int p = ty;
    for (; p + 192 < nparts; p += 256) {  // four partials in flight per thread
      float ta[4], tb[4], td[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t o = ((int64_t)(p + 64 * u) * np) * C + c;
        ta[u] = part[o];
        tb[u] = part[o + C];
        td[u] = dxsum ? part[o + 2 * C] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a += ta[u];
        b += tb[u];
        d += td[u];
      }
    }
    for (; p < nparts; p += 64) {
      a += part[((int64_t)p * np) * C + c];
      b += part[((int64_t)p * np + 1) * C + c];
      if (dxsum) d += part[((int64_t)p * np + 2) * C + c];
    }
  }
  sa[ty][tx] = a;
  sb[ty][tx] = b;
  sd[ty][tx] = d;
  __syncthreads();
  if (ty == 0 && c < C) {
    float ra = 0.f, rb = 0.f, rd = 0.f;
#pragma unroll 4
    for (int i = 0; i < 64; ++i) {
      ra += sa[i][tx];
      rb += sb[i][tx];
      rd += sd[i][tx];
    }
    if (beta_dg != 0.f) ra += dgamma[c];
    if (beta_db != 0.f) rb += dbeta[c];
    dgamma[c] = ra;
    dbeta[c] = rb;
    if (dxsum) dxsum[c] = rd;
  }
}

// out[c] = beta * out[c] + the sum over nparts slab partials of column c; 64 columns
// x 16 slab groups per workgroup
__device__ inline void colsum_reduce_cols(const float* __restrict__ partial, int nparts, int64_t cols,
                                          float* __restrict__ out, float beta, int bx) {
  __shared__ float sh[16][65];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t c = (int64_t)bx * 64 + tx;
  float a = 0.f;
  if (c < cols)
    for (int p = ty; p < nparts; p += 16) a += partial[(int64_t)p * cols + c];
  sh[ty][tx] = a;
  __syncthreads();
  if (ty == 0 && c < cols) {
    float r = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) r += sh[i][tx];
    if (beta != 0.f) r += beta * out[c];
    out[c] = r;
  }
}

}  // namespace tfb
