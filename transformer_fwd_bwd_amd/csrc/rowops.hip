// Row reductions: LayerNorm, the causal row softmax and the fused softmax +
// cross-entropy, forward and backward ([Autograd-1, "Ops": SoftmaxCrossEntropy
// and Softmax, the table of ops: LayerNorm, CausalSoftmax; GPT2-4, "The 12
// unused tensors": the causal mask is computed, row r sees r % T + 1 columns]).
// One 64-lane wavefront per row, with the row cached in registers when it fits
// (16 values per lane, rows up to 1024); wave-shuffle reductions; column sums
// (LayerNorm's dgamma, dbeta) are per-block partials reduced in a second pass,
// so every result is deterministic.
#include <algorithm>

#include <type_traits>

#include "kernels.h"
#include "reduce_dev.h"

namespace tfb {
namespace {

typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// bf16 bits of x, rounded to nearest even (the rounding of every bf16 operand copy)
__device__ __forceinline__ uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;
constexpr int WAVES = NT / 64;
constexpr int MAXV = 16;  // cached values per lane -> rows up to 1024

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// The same sum for a wave whose 64 lanes are all active: DPP within each row of
// 16 lanes (quad swaps, then the half-row and row mirrors), then the four row
// sums read as scalars.  No LDS round trips, where the cross-lane shuffles above
// take six dependent ones.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_sum_full(float v) {
  v += dpp_f<0xb1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4e>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror: the other quad of the half-row
  v += dpp_f<0x140>(v);  // row_mirror: the other half of the row
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ float wave_max_full(float v) {
  v = fmaxf(v, dpp_f<0xb1>(v));
  v = fmaxf(v, dpp_f<0x4e>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ------------------------------------------------------------ LayerNorm
template <bool CACHED>
__global__ __launch_bounds__(NT) void ln_fwd_k(const float* __restrict__ x, const float* __restrict__ gamma,
                                               const float* __restrict__ beta, float* __restrict__ y,
                                               uint16_t* __restrict__ ybf, float* __restrict__ mean,
                                               float* __restrict__ rstd, int64_t rows, int C, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * WAVES;
  for (int64_t r = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6); r < rows; r += nw) {
    const float* xr = x + r * C;
    float v[MAXV];
    float s = 0.f;
    if (CACHED) {
#pragma unroll
      for (int j = 0; j < MAXV; ++j) {
        const int c = lane + 64 * j;
        v[j] = c < C ? xr[c] : 0.f;
        s += v[j];
      }
    } else {
      for (int c = lane; c < C; c += 64) s += xr[c];
    }
    const float mu = wave_sum(s) / C;
    float q = 0.f;
    if (CACHED) {
#pragma unroll
      for (int j = 0; j < MAXV; ++j) {
        const int c = lane + 64 * j;
        const float d = c < C ? v[j] - mu : 0.f;
        q += d * d;
      }
    } else {
      for (int c = lane; c < C; c += 64) {
        const float d = xr[c] - mu;
        q += d * d;
      }
    }
    const float rs = rsqrtf(wave_sum(q) / C + eps);
    float* yr = y + r * C;
    if (CACHED) {
#pragma unroll
      for (int j = 0; j < MAXV; ++j) {
        const int c = lane + 64 * j;
        if (c < C) {
          const float o = (v[j] - mu) * rs * gamma[c] + beta[c];
          if (y) yr[c] = o;  // null: the bf16 copy alone
          if (ybf) ybf[r * C + c] = bf16_bits(o);
        }
      }
    } else {
      for (int c = lane; c < C; c += 64) {
        const float o = (xr[c] - mu) * rs * gamma[c] + beta[c];
        if (y) yr[c] = o;
        if (ybf) ybf[r * C + c] = bf16_bits(o);
      }
    }
    if (lane == 0) {
      mean[r] = mu;
      rstd[r] = rs;
    }
  }
}

// float4 variants: rows of C = 4 * 64 * J floats or fewer (C % 4 == 0, C <= 1024),
// lane holds the quads lane + 64 j
template <int J>
__global__ __launch_bounds__(NT) void ln_fwd4_k(const f4* __restrict__ x, const f4* __restrict__ gamma,
                                                const f4* __restrict__ beta, f4* __restrict__ y,
                                                u16x4* __restrict__ ybf, float* __restrict__ mean,
                                                float* __restrict__ rstd, int64_t rows, int C4, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * WAVES;
  const float invC = 1.f / (4 * C4);
  // gamma and beta once per wave, requested with the first row (a column past the
  // row reads column 0 and is not used)
  f4 gm[J], bt[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = lane + 64 * j < C4 ? lane + 64 * j : 0;
    gm[j] = gamma[c];
    bt[j] = beta[c];
  }
  for (int64_t r = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6); r < rows; r += nw) {
    const f4* xr = x + r * C4;
    f4 v[J];
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = lane + 64 * j;
      v[j] = xr[c < C4 ? c : 0];
      if (c >= C4) v[j] = f4{0.f, 0.f, 0.f, 0.f};
      s += (v[j][0] + v[j][1]) + (v[j][2] + v[j][3]);
    }
    const float mu = wave_sum_full(s) * invC;
    float q = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = lane + 64 * j;
      if (c < C4) {
        const f4 d = v[j] - mu;
        q += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
      }
    }
    const float rs = rsqrtf(wave_sum_full(q) * invC + eps);
    f4* yr = y + r * C4;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = lane + 64 * j;
      if (c < C4) {
        const f4 o = (v[j] - mu) * rs * gm[j] + bt[j];
        if (y) yr[c] = o;  // null: the bf16 copy alone
        if (ybf) ybf[r * C4 + c] = u16x4{bf16_bits(o[0]), bf16_bits(o[1]), bf16_bits(o[2]), bf16_bits(o[3])};
      }
    }
    if (lane == 0) {
      mean[r] = mu;
      rstd[r] = rs;
    }
  }
}

// dx per row (one wavefront per row, many rows in flight)
template <bool CACHED>
__global__ __launch_bounds__(NT) void ln_bwd_dx_k(const float* __restrict__ g, const float* __restrict__ x,
                                                  const float* __restrict__ gamma, const float* __restrict__ mean,
                                                  const float* __restrict__ rstd, float* __restrict__ dx, int64_t rows,
                                                  int C, float beta_dx) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * WAVES;
  for (int64_t r = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6); r < rows; r += nw) {
    const float mu = mean[r], rs = rstd[r];
    const float* gr = g + r * C;
    const float* xr = x + r * C;
    float xh[MAXV], dg[MAXV];
    float s1 = 0.f, s2 = 0.f;
    if (CACHED) {
#pragma unroll
      for (int j = 0; j < MAXV; ++j) {
        const int c = lane + 64 * j;
        xh[j] = c < C ? (xr[c] - mu) * rs : 0.f;
        dg[j] = c < C ? gr[c] * gamma[c] : 0.f;
        s1 += dg[j];
        s2 += dg[j] * xh[j];
      }
    } else {
      for (int c = lane; c < C; c += 64) {
        const float xv = (xr[c] - mu) * rs, d = gr[c] * gamma[c];
        s1 += d;
        s2 += d * xv;
      }
    }
    const float m1 = wave_sum(s1) / C, m2 = wave_sum(s2) / C;
    float* dr = dx + r * C;
    if (CACHED) {
#pragma unroll
      for (int j = 0; j < MAXV; ++j) {
        const int c = lane + 64 * j;
        if (c < C) {
          float v = rs * (dg[j] - m1 - xh[j] * m2);
          if (beta_dx != 0.f) v += dr[c];
          dr[c] = v;
        }
      }
    } else {
      for (int c = lane; c < C; c += 64) {
        const float xv = (xr[c] - mu) * rs;
        float v = rs * (gr[c] * gamma[c] - m1 - xv * m2);
        if (beta_dx != 0.f) v += dr[c];
        dr[c] = v;
      }
    }
  }
}

// partial column sums over a slab of rows: part[p][0][c] = sum g*xhat, part[p][1][c] = sum g
// LayerNorm backward over float4 rows, one wavefront per row (the row held in
// registers): dx = rstd (g*gamma - mean(g*gamma) - xhat mean(g*gamma*xhat)),
// plus the dgamma / dbeta column partials of the rows this workgroup handles:
// each lane adds g*xhat and g for its float4 columns into its wave's slice of
// LDS (only that lane touches those entries, so no barrier until the end), the
// 4 waves' slices are added in a fixed order, and part[block][plane][C] receives
// the result (reduced by ln_bwd_reduce).  With SUMDX a third plane holds the
// column sums of the final dx (the bias gradient of a Linear whose output
// gradient this is).  A wave loads its rows two at a time, so two rows' reads
// are in flight; keeping the partials out of registers leaves room for four
// waves per SIMD at C = 768.
__device__ __forceinline__ f4 ld_g4(const f4* p, int64_t i) { return p[i]; }
__device__ __forceinline__ f4 ld_g4(const u16x4* p, int64_t i) {  // exact float values of 4 bf16 numbers
  const u16x4 v = p[i];
  return f4{__uint_as_float((unsigned)v[0] << 16), __uint_as_float((unsigned)v[1] << 16),
            __uint_as_float((unsigned)v[2] << 16), __uint_as_float((unsigned)v[3] << 16)};
}
// the same in two steps: the stored form (held until used), then its float values
__device__ __forceinline__ f4 g4_val(const f4& v) { return v; }
__device__ __forceinline__ f4 g4_val(const u16x4& v) {
  return f4{__uint_as_float((unsigned)v[0] << 16), __uint_as_float((unsigned)v[1] << 16),
            __uint_as_float((unsigned)v[2] << 16), __uint_as_float((unsigned)v[3] << 16)};
}

// GT: f4, or u16x4 for an upstream gradient held as bf16.  FULL: C4 == 64 J (every
// lane has J float4s of every row; no column checks).  The wave index is made
// scalar, so a row's base addresses are scalar and each load is that base plus
// the lane's offset: no per-lane 64-bit addresses to hold.
// Eight waves per workgroup, two workgroups per CU at C = 768 (four waves per
// SIMD): the workgroups, and so the partial rows that the column reduction reads
// afterwards, are half as many as with four-wave workgroups.
constexpr int LNW = 8;
template <int J, bool SUMDX, bool FULL, typename GT = f4>
__global__ __launch_bounds__(LNW * 64, J <= 3 ? 2 : 1) void ln_bwd_fused4_k(
    const GT* __restrict__ g, const f4* __restrict__ x, const f4* __restrict__ gamma, const float* __restrict__ mean,
    const float* __restrict__ rstd, f4* dx, const f4* dx_src, u16x4* __restrict__ dxbf, f4* __restrict__ part,
    int64_t rows, int C4, float beta_dx) {
  constexpr int NP = SUMDX ? 3 : 2;
  __shared__ f4 sh[LNW][NP][64 * J];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * LNW;
  const float invC = 1.f / (4 * C4);
  const auto in = [&](int j) { return FULL || lane + 64 * j < C4; };
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int q = 0; q < NP; ++q) sh[w][q][lane + 64 * j] = f4{0.f, 0.f, 0.f, 0.f};
  for (int64_t r0 = (int64_t)blockIdx.x * LNW + w; r0 < rows; r0 += 2 * nw) {
    // the column partials stay in LDS: without this compiler-only fence the
    // compiler keeps them in registers across rows (nothing else touches them
    // inside the loop), which is what keeping them in LDS is meant to avoid
    asm volatile("" ::: "memory");
    // rows r0 and r0 + nw (the second clamped to an in-range row when past the end,
    // its results then unused); both rows' x and g are loaded before either is used
    const int64_t rr[2] = {r0, r0 + nw < rows ? r0 + nw : r0};
    f4 xv[2][J];
    GT graw[2][J];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const f4* xr = x + rr[u] * C4;
      const GT* gr = g + rr[u] * C4;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = in(j) ? lane + 64 * j : 0;  // an in-range column, its value unused
        xv[u][j] = xr[c];
        graw[u][j] = gr[c];
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && r0 + nw >= rows) break;
      const int64_t r = rr[u];
      const float mu = mean[r], rs = rstd[r];
      f4 xh[J], dg[J];
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = lane + 64 * j;
        const f4 gj = in(j) ? g4_val(graw[u][j]) : f4{0.f, 0.f, 0.f, 0.f};
        xh[j] = in(j) ? (xv[u][j] - mu) * rs : f4{0.f, 0.f, 0.f, 0.f};
        dg[j] = in(j) ? gj * gamma[in(j) ? c : 0] : f4{0.f, 0.f, 0.f, 0.f};
        sh[w][0][c] += gj * xh[j];
        sh[w][1][c] += gj;
        s1 += (dg[j][0] + dg[j][1]) + (dg[j][2] + dg[j][3]);
        const f4 t = dg[j] * xh[j];
        s2 += (t[0] + t[1]) + (t[2] + t[3]);
      }
      // the earlier gradient of an element is read just before that element is
      // stored, by the lane that stores it, so this holds even when dx_src is dx
      f4 sv[J];
      const f4* sr = dx_src + r * C4;
#pragma unroll
      for (int j = 0; j < J; ++j)  // zero when beta_dx == 0
        sv[j] = beta_dx != 0.f ? sr[in(j) ? lane + 64 * j : 0] : f4{0.f, 0.f, 0.f, 0.f};
      const float m1 = wave_sum_full(s1) * invC, m2 = wave_sum_full(s2) * invC;
      f4* dr = dx + r * C4;
      u16x4* dbr = dxbf ? dxbf + r * C4 : nullptr;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = lane + 64 * j;
        if (in(j)) {
          f4 v = rs * (dg[j] - m1 - xh[j] * m2);
          v += sv[j];
          dr[c] = v;
          if constexpr (SUMDX) sh[w][2][c] += v;
          if (dbr) dbr[c] = u16x4{bf16_bits(v[0]), bf16_bits(v[1]), bf16_bits(v[2]), bf16_bits(v[3])};
        }
      }
    }
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = lane + 64 * j;
      if (in(j)) {
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          f4 a = sh[0][q][c];
#pragma unroll
          for (int i = 1; i < LNW; ++i) a += sh[i][q][c];
          part[((int64_t)blockIdx.x * NP + q) * C4 + c] = a;
        }
      }
    }
  }
}

__global__ __launch_bounds__(NT) void ln_bwd_cols_k(const float* __restrict__ g, const float* __restrict__ x,
                                                    const float* __restrict__ mean, const float* __restrict__ rstd,
                                                    float* __restrict__ part, int64_t rows, int C, int64_t rows_per) {
  const int c = blockIdx.x * NT + threadIdx.x;
  if (c >= C) return;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per;
  const int64_t r1 = r0 + rows_per < rows ? r0 + rows_per : rows;
  float a = 0.f, b = 0.f;
  int64_t r = r0;
  for (; r + 4 <= r1; r += 4) {
    float gv[4], xv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      gv[u] = g[(r + u) * C + c];
      xv[u] = x[(r + u) * C + c];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a += gv[u] * (xv[u] - mean[r + u]) * rstd[r + u];
      b += gv[u];
    }
  }
  for (; r < r1; ++r) {
    const float gv = g[r * C + c];
    a += gv * (x[r * C + c] - mean[r]) * rstd[r];
    b += gv;
  }
  part[((int64_t)blockIdx.y * 2) * C + c] = a;
  part[((int64_t)blockIdx.y * 2 + 1) * C + c] = b;
}

// out_a[c] (+)= sum_p part[p][0][c], out_b[c] (+)= sum_p part[p][1][c], and with
// dxsum (np == 3) dxsum[c] = sum_p part[p][2][c]
__global__ __launch_bounds__(1024) void ln_bwd_reduce(const float* __restrict__ part, int nparts, int np, int C,
                                                      float* __restrict__ dgamma, float* __restrict__ dbeta,
                                                      float* __restrict__ dxsum, float beta_dg, float beta_db) {
  ln_reduce_cols(part, nparts, np, C, dgamma, dbeta, dxsum, beta_dg, beta_db, blockIdx.x);
}

__global__ __launch_bounds__(1024) void reduce_batch_k(ReduceJobs jobs) {
  const ReduceJob& j = jobs.j[blockIdx.y];
  const int bx = blockIdx.x;
  if (j.kind == REDUCE_LN) {
    if (bx * 16 < j.cols)
      ln_reduce_cols(j.part, j.nparts, j.np, (int)j.cols, j.out[0], j.out[1], j.out[2], j.beta[0], j.beta[1], bx);
  } else {
    if ((int64_t)bx * 64 < j.cols) colsum_reduce_cols(j.part, j.nparts, j.cols, j.out[0], j.beta[0], bx);
  }
}

int ln_bwd_parts(int64_t rows) {
  return (int)std::max<int64_t>(1, std::min<int64_t>(128, (rows + 31) / 32));
}

// workgroups of the fused LayerNorm backward: at most 512 (two per CU), each
// wave taking two rows per step; the column partials stay a few MB
int64_t ln_fused_blocks(int64_t rows) { return std::max<int64_t>(1, std::min<int64_t>(512, (rows + LNW - 1) / LNW)); }

// ------------------------------------------------------------ causal softmax
template <bool CACHED>
__global__ __launch_bounds__(NT) void csm_fwd_k(const float* __restrict__ x, float* __restrict__ p, int64_t rows,
                                                int T, bool full) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * WAVES;
  for (int64_t r = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6); r < rows; r += nw) {
    const int vis = (int)(r % T) + 1;
    const float* xr = x + r * T;
    float* pr = p + r * T;
    float v[MAXV];
    float mx = -INFINITY;
    if (CACHED) {
#pragma unroll
      for (int j = 0; j < MAXV; ++j) {
        const int c = lane + 64 * j;
        const float t = xr[min(c, vis - 1)];  // every load issued before any is used
        v[j] = c < vis ? t : -INFINITY;
        mx = fmaxf(mx, v[j]);
      }
    } else {
      for (int c = lane; c < vis; c += 64) mx = fmaxf(mx, xr[c]);
    }
    mx = wave_max_full(mx);
    float s = 0.f;
    if (CACHED) {
#pragma unroll
      for (int j = 0; j < MAXV; ++j) {
        const int c = lane + 64 * j;
        v[j] = c < vis ? expf(v[j] - mx) : 0.f;
        s += v[j];
      }
    } else {
      for (int c = lane; c < vis; c += 64) s += expf(xr[c] - mx);
    }
    const float inv = 1.f / wave_sum_full(s);
    if (CACHED) {
#pragma unroll
      for (int j = 0; j < MAXV; ++j) {
        const int c = lane + 64 * j;
        if (c < vis)
          pr[c] = v[j] * inv;
        else if (full && c < T)
          pr[c] = 0.f;
      }
    } else {
      for (int c = lane; c < T; c += 64) {
        if (c < vis)
          pr[c] = expf(xr[c] - mx) * inv;
        else if (full)
          pr[c] = 0.f;
      }
    }
  }
}

template <bool CACHED>
__global__ __launch_bounds__(NT) void csm_bwd_k(const float* __restrict__ g, const float* __restrict__ p,
                                                float* __restrict__ d, int64_t rows, int T, float scale, float beta,
                                                bool full) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * WAVES;
  for (int64_t r = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6); r < rows; r += nw) {
    const int vis = (int)(r % T) + 1;
    const float* gr = g + r * T;
    const float* pr = p + r * T;
    float* dr = d + r * T;
    float gv[MAXV], pv[MAXV];
    float s = 0.f;
    if (CACHED) {
#pragma unroll
      for (int j = 0; j < MAXV; ++j) {
        const int c = lane + 64 * j;
        const float tg = gr[min(c, vis - 1)], tp = pr[min(c, vis - 1)];  // loads issued together
        gv[j] = c < vis ? tg : 0.f;
        pv[j] = c < vis ? tp : 0.f;
        s += gv[j] * pv[j];
      }
    } else {
      for (int c = lane; c < vis; c += 64) s += gr[c] * pr[c];
    }
    s = wave_sum_full(s);
    if (CACHED) {
#pragma unroll
      for (int j = 0; j < MAXV; ++j) {
        const int c = lane + 64 * j;
        if (c < vis) {
          float v = scale * pv[j] * (gv[j] - s);
          if (beta != 0.f) v += dr[c];
          dr[c] = v;
        } else if (full && beta == 0.f && c < T) {
          dr[c] = 0.f;
        }
      }
    } else {
      for (int c = lane; c < T; c += 64) {
        if (c < vis) {
          float v = scale * pr[c] * (gr[c] - s);
          if (beta != 0.f) v += dr[c];
          dr[c] = v;
        } else if (full && beta == 0.f) {
          dr[c] = 0.f;
        }
      }
    }
  }
}

// ------------------------------------------------------------ softmax + cross-entropy
// e^a for the cross-entropy kernels: the hardware 2^x on a * log2(e) (about 2 ulp
// on the softmax terms; 0 for a = -inf).  The forward and backward use it alike,
// so a gradient the forward writes equals the one the backward would.
__device__ __forceinline__ float ce_exp(float a) { return __builtin_amdgcn_exp2f(a * 1.4426950408889634f); }

__device__ __forceinline__ void online_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * ce_exp(m - mn) + s2 * ce_exp(m2 - mn);
  m = mn;
}

// one block per row: lse[r] = log(sum exp(logits)), loss_rows[r] = -log(max(p_target, 1e-30))
__global__ __launch_bounds__(NT) void ce_fwd_k(const float* __restrict__ logits, int64_t ld,
                                               const int32_t* __restrict__ tgt, int64_t V, float* __restrict__ lse,
                                               float* __restrict__ loss_rows) {
  __shared__ float sm[WAVES], ss[WAVES];
  const int64_t r = blockIdx.x;
  const float* lr = logits + r * ld;
  float m = -INFINITY, s = 0.f;
  for (int64_t c = threadIdx.x; c < V; c += NT) {
    const float x = lr[c];
    if (x > m) {
      s = s * ce_exp(m - x) + 1.f;
      m = x;
    } else {
      s += ce_exp(x - m);
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    online_merge(m, s, m2, s2);
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    sm[w] = m;
    ss[w] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = sm[0], S = ss[0];
    for (int i = 1; i < WAVES; ++i) online_merge(M, S, sm[i], ss[i]);
    const float L = M + logf(S);
    lse[r] = L;
    // -log(max(p_t, 1e-30)) with p_t = exp(x_t - L); -log(1e-30) = 69.0775527898...
    // (a target outside [0, V) is a caller error: it yields NaN instead of a stray read)
    const int t = tgt[r];
    loss_rows[r] = (t >= 0 && t < V) ? fminf(L - lr[t], 69.07755278982137f) : NAN;
  }
}

__global__ __launch_bounds__(NT) void mean_k(const float* __restrict__ v, int64_t n, float* __restrict__ out) {
  __shared__ double sh[NT];
  double s = 0.0;
  int64_t i = threadIdx.x;
  for (; i + 7 * NT < n; i += 8 * NT) {  // eight loads in flight, added in index order
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = v[i + u * NT];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += (double)x[u];
  }
  for (; i < n; i += NT) s += (double)v[i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int o = NT / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = (float)(sh[0] / (double)n);
}

__global__ __launch_bounds__(NT) void ce_bwd_k(const float* __restrict__ logits, int64_t ld,
                                               const int32_t* __restrict__ tgt, const float* __restrict__ lse,
                                               const float* __restrict__ gsc, float* __restrict__ dl,
                                               uint16_t* __restrict__ dlbf, int64_t rows, int64_t V, float beta,
                                               int skip_unit) {
  if (skip_unit && gsc[0] == 1.f) return;
  const int64_t r = blockIdx.x;
  const float gn = gsc[0] / (float)rows;
  const float L = lse[r];
  const int t = tgt[r];
  const float* lr = logits + r * ld;
  float* dr = dl ? dl + r * ld : nullptr;  // null: the bf16 copy alone
  uint16_t* br = dlbf ? dlbf + r * ld : nullptr;
  for (int64_t c = threadIdx.x; c < V; c += NT) {
    float v = gn * (ce_exp(lr[c] - L) - (c == t ? 1.f : 0.f));
    if (dr) {
      if (beta != 0.f) v += dr[c];
      dr[c] = v;
    }
    if (br) br[c] = bf16_bits(v);
  }
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

inline unsigned row_blocks(int64_t rows) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>((rows + WAVES - 1) / WAVES, 65536));
}


// The same over float4 (rows 16-byte aligned): 16 logits in flight per thread,
// one max / rescale per 16, then the scalar tail of V % 4 logits.
__global__ __launch_bounds__(NT) void ce_fwd4_k(const float* __restrict__ logits, int64_t ld,
                                                const int32_t* __restrict__ tgt, int64_t V, float* __restrict__ lse,
                                                float* __restrict__ loss_rows) {
  __shared__ float sm[WAVES], ss[WAVES];
  const int64_t r = blockIdx.x;
  const float* lr = logits + r * ld;
  const f4* lr4 = reinterpret_cast<const f4*>(lr);
  const int64_t V4 = V / 4;
  float m = -INFINITY, s = 0.f;
  for (int64_t c = threadIdx.x; c < V4; c += 4 * NT) {
    f4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = c + u * NT;
      x[u] = i < V4 ? lr4[i] : f4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
    float mx = m;
#pragma unroll
    for (int u = 0; u < 4; ++u) mx = fmaxf(mx, fmaxf(fmaxf(x[u][0], x[u][1]), fmaxf(x[u][2], x[u][3])));
    s *= ce_exp(m - mx);  // m = -inf the first time: s is 0 and stays 0
    m = mx;
#pragma unroll
    for (int u = 0; u < 4; ++u) s += (ce_exp(x[u][0] - m) + ce_exp(x[u][1] - m)) + (ce_exp(x[u][2] - m) + ce_exp(x[u][3] - m));
  }
  for (int64_t c = 4 * V4 + threadIdx.x; c < V; c += NT) {
    const float x = lr[c];
    if (x > m) {
      s = s * ce_exp(m - x) + 1.f;
      m = x;
    } else {
      s += ce_exp(x - m);
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    online_merge(m, s, m2, s2);
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    sm[w] = m;
    ss[w] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = sm[0], S = ss[0];
    for (int i = 1; i < WAVES; ++i) online_merge(M, S, sm[i], ss[i]);
    const float L = M + logf(S);
    lse[r] = L;
    const int t = tgt[r];
    loss_rows[r] = (t >= 0 && t < V) ? fminf(L - lr[t], 69.07755278982137f) : NAN;
  }
}


// logits read as float, from fp32 or from bf16 storage
__device__ __forceinline__ float ld_x(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_x(const uint16_t* p, int64_t i) { return __uint_as_float((unsigned)p[i] << 16); }
__device__ __forceinline__ f4 ld_x4(const float* p, int64_t i4) { return reinterpret_cast<const f4*>(p)[i4]; }
__device__ __forceinline__ f4 ld_x4(const uint16_t* p, int64_t i4) {
  const u16x4 v = reinterpret_cast<const u16x4*>(p)[i4];
  return f4{__uint_as_float((unsigned)v[0] << 16), __uint_as_float((unsigned)v[1] << 16),
            __uint_as_float((unsigned)v[2] << 16), __uint_as_float((unsigned)v[3] << 16)};
}

// Cross-entropy forward that also writes the bf16 gradient the backward would
// write for an upstream gradient of 1, (p - onehot) / rows, in the backward's own
// expression: one 1024-thread workgroup per row holds the row in registers (PER
// float4 per thread), so the logits are read once for both passes.
// bf16 logits stay packed in registers (converted at each use): under 64 VGPRs,
// two 1024-thread workgroups share a CU and one's reductions overlap the other's loads
__device__ __forceinline__ f4 cvt4(f4 v) { return v; }
__device__ __forceinline__ f4 cvt4(u16x4 v) {
  return f4{__uint_as_float((unsigned)v[0] << 16), __uint_as_float((unsigned)v[1] << 16),
            __uint_as_float((unsigned)v[2] << 16), __uint_as_float((unsigned)v[3] << 16)};
}
template <int PER, class X>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(sizeof(X) == 2 ? 8 : 1)))
void ce_fwd_grad4_k(const X* __restrict__ logits, int64_t ld,
                                                       const int32_t* __restrict__ tgt, int64_t V,
                                                       float* __restrict__ lse, float* __restrict__ loss_rows,
                                                       uint16_t* __restrict__ dlbf, float gn) {
  constexpr int NW = 16;
  __shared__ float red[NW];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t r = blockIdx.x;
  const X* lr = logits + r * ld;
  const int V4 = (int)(V / 4);
  const int tail = (int)(V - 4 * V4);
  using XS = typename std::conditional<sizeof(X) == 2, u16x4, f4>::type;
  XS xs[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + u * 1024;
    if constexpr (sizeof(X) == 2) {
      // buffer loads over the row's whole groups of 4: one offset register serves
      // every load, and the hardware's range check returns 0 past the end (replaced
      // by -inf below)
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)lr, (short)0, (int)(V4 * 8), 0x00020000);
      const auto raw = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(i * 8), 0, 0);
      const u16x4 ninf = {0xFF80, 0xFF80, 0xFF80, 0xFF80};  // bf16 -inf
      xs[u] = i < V4 ? __builtin_bit_cast(u16x4, raw) : ninf;
    } else {
      xs[u] = i < V4 ? ld_x4(lr, i) : f4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
  }
  // each pass converts the packed values afresh: an empty asm marks them as changed so
  // that the compiler cannot keep the first pass's fp32 copies live instead
  auto refresh = [&]() {
    if constexpr (sizeof(X) == 2) {
#pragma unroll
      for (int u = 0; u < PER; ++u) asm volatile("" : "+v"(xs[u]));
    }
  };
#define x_(u) cvt4(xs[u])
  const float xt = tid < tail ? ld_x(lr, 4 * V4 + tid) : -INFINITY;
  float m = xt;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const f4 x = x_(u);
    m = fmaxf(m, fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  }
  m = wave_max_full(m);
  if (lane == 0) red[w] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) m = fmaxf(m, red[i]);
  __syncthreads();
  float sum = ce_exp(xt - m);
  refresh();
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const f4 x = x_(u);
    sum += (ce_exp(x[0] - m) + ce_exp(x[1] - m)) + (ce_exp(x[2] - m) + ce_exp(x[3] - m));
  }
  sum = wave_sum_full(sum);
  if (lane == 0) red[w] = sum;
  __syncthreads();
  float S = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) S += red[i];
  const float L = m + logf(S);
  const int t = tgt[r];
  if (tid == 0) {
    lse[r] = L;
    loss_rows[r] = (t >= 0 && t < V) ? fminf(L - ld_x(lr, t), 69.07755278982137f) : NAN;
  }
  if (!dlbf) return;  // no gradient wanted
  u16x4* br4 = reinterpret_cast<u16x4*>(dlbf + r * ld);
  refresh();
  __amdgpu_buffer_rsrc_t ws_;
  if constexpr (sizeof(X) == 2)
    ws_ = __builtin_amdgcn_make_buffer_rsrc((void*)br4, (short)0, (int)(V4 * 8), 0x00020000);
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = tid + u * 1024;
    if (i >= V4) break;
    const f4 x = x_(u);
    f4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = gn * (ce_exp(x[e] - L) - (4 * i + e == t ? 1.f : 0.f));
    const u16x4 b = u16x4{bf16_bits(v[0]), bf16_bits(v[1]), bf16_bits(v[2]), bf16_bits(v[3])};
    if constexpr (sizeof(X) == 2) {
      typedef int i32x2 __attribute__((ext_vector_type(2)));
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, b), ws_, (int)(i * 8), 0, 0);
    } else {
      br4[i] = b;
    }
  }
#undef x_
  if (tid < tail) {
    const int64_t c = 4 * V4 + tid;
    dlbf[r * ld + c] = bf16_bits(gn * (ce_exp(xt - L) - (c == t ? 1.f : 0.f)));
  }
}

// float4 form of ce_bwd_k (rows 16-byte aligned): two float4 per thread in flight
template <class X>
__global__ __launch_bounds__(NT) void ce_bwd4_k(const X* __restrict__ logits, int64_t ld,
                                                const int32_t* __restrict__ tgt, const float* __restrict__ lse,
                                                const float* __restrict__ gsc, float* __restrict__ dl,
                                                uint16_t* __restrict__ dlbf, int64_t rows, int64_t V, float beta,
                                                int skip_unit) {
  if (skip_unit && gsc[0] == 1.f) return;  // the forward already wrote this gradient
  const int64_t r = blockIdx.x;
  const float gn = gsc[0] / (float)rows;
  const float L = lse[r];
  const int t = tgt[r];
  const X* lr = logits + r * ld;
  f4* dr4 = dl ? reinterpret_cast<f4*>(dl + r * ld) : nullptr;  // null: the bf16 copy alone
  u16x4* br4 = dlbf ? reinterpret_cast<u16x4*>(dlbf + r * ld) : nullptr;
  const int64_t V4 = V / 4;
  for (int64_t c = threadIdx.x; c < V4; c += 2 * NT) {
    f4 x[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t i = c + u * NT;
      if (i < V4) x[u] = ld_x4(lr, i);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t i = c + u * NT;
      if (i >= V4) continue;
      f4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = gn * (ce_exp(x[u][e] - L) - (4 * i + e == t ? 1.f : 0.f));
      if (dr4) {
        if (beta != 0.f) v += dr4[i];
        dr4[i] = v;
      }
      if (br4) br4[i] = u16x4{bf16_bits(v[0]), bf16_bits(v[1]), bf16_bits(v[2]), bf16_bits(v[3])};
    }
  }
  float* dr = dl ? dl + r * ld : nullptr;
  for (int64_t c = 4 * V4 + threadIdx.x; c < V; c += NT) {
    float v = gn * (ce_exp(ld_x(lr, c) - L) - (c == t ? 1.f : 0.f));
    if (dr) {
      if (beta != 0.f) v += dr[c];
      dr[c] = v;
    }
    if (dlbf) dlbf[r * ld + c] = bf16_bits(v);
  }
}

}  // namespace

hipError_t layernorm_fwd(const float* x, const float* gamma, const float* beta, float* y, uint16_t* ybf, float* mean,
                         float* rstd, int64_t rows, int64_t C, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (C % 4 == 0 && C <= 1024 && aligned16(x) && aligned16(y) && aligned16(gamma) && aligned16(beta) &&
      (reinterpret_cast<uintptr_t>(ybf) & 7) == 0) {
    const int C4 = (int)(C / 4);
    if (C4 <= 64)
      run_kernel(ln_fwd4_k<1>, dim3(row_blocks(rows)), dim3(NT), 0, s, (const f4*)x, (const f4*)gamma,
                         (const f4*)beta, (f4*)y, (u16x4*)ybf, mean, rstd, rows, C4, eps);
    else if (C4 <= 192)
      run_kernel(ln_fwd4_k<3>, dim3(row_blocks(rows)), dim3(NT), 0, s, (const f4*)x, (const f4*)gamma,
                         (const f4*)beta, (f4*)y, (u16x4*)ybf, mean, rstd, rows, C4, eps);
    else
      run_kernel(ln_fwd4_k<4>, dim3(row_blocks(rows)), dim3(NT), 0, s, (const f4*)x, (const f4*)gamma,
                         (const f4*)beta, (f4*)y, (u16x4*)ybf, mean, rstd, rows, C4, eps);
  } else if (C <= 64 * MAXV)
    run_kernel(ln_fwd_k<true>, dim3(row_blocks(rows)), dim3(NT), 0, s, x, gamma, beta, y, ybf, mean, rstd, rows,
                       (int)C, eps);
  else
    run_kernel(ln_fwd_k<false>, dim3(row_blocks(rows)), dim3(NT), 0, s, x, gamma, beta, y, ybf, mean, rstd, rows,
                       (int)C, eps);
  return hipGetLastError();
}

size_t layernorm_bwd_workspace_bytes(int64_t rows, int64_t C) {
  return (size_t)std::max<int64_t>(ln_bwd_parts(rows), ln_fused_blocks(rows)) * 3 * C * sizeof(float);
}

bool layernorm_bwd_bf16_fits(const float* x, const float* dx, const uint16_t* gbf, int64_t rows, int64_t C) {
  return rows > 0 && C % 4 == 0 && C <= 1024 && aligned16(x) && aligned16(dx) &&
         (reinterpret_cast<uintptr_t>(gbf) & 7) == 0;
}

hipError_t layernorm_bwd(const float* g, const float* x, const float* gamma, const float* mean, const float* rstd,
                         float* dx, const float* dx_src, uint16_t* dxbf, float* dgamma, float* dbeta, int64_t rows,
                         int64_t C, float beta_dx, float beta_dg, float beta_db, void* ws, hipStream_t s,
                         float* dxsum, bool* dxsum_written, const uint16_t* gbf, ReduceJob* defer) {
  if (dxsum_written) *dxsum_written = false;
  if (C <= 0) return hipSuccess;
  if (!dx_src) dx_src = dx;
  float* part = static_cast<float*>(ws);
  int parts = 0, np = 2;
  if (gbf && !layernorm_bwd_bf16_fits(x, dx, gbf, rows, C)) return hipErrorInvalidValue;
  if (rows > 0 && C % 4 == 0 && C <= 1024 && (gbf || aligned16(g)) && aligned16(x) && aligned16(gamma) &&
      aligned16(dx) && aligned16(dx_src) && aligned16(part) && (reinterpret_cast<uintptr_t>(dxbf) & 7) == 0 &&
      (reinterpret_cast<uintptr_t>(gbf) & 7) == 0) {
    // dx (and its bf16 copy) and the column partials in one pass over g and x
    const int C4 = (int)(C / 4);
    const int64_t blocks = ln_fused_blocks(rows);
    const dim3 grid((unsigned)blocks), block(LNW * 64);
    const f4 *x4 = (const f4*)x, *gm4 = (const f4*)gamma, *src4 = (const f4*)dx_src;
    auto launch = [&](auto gp) {
      using GT = std::remove_const_t<std::remove_pointer_t<decltype(gp)>>;
      auto go = [&](auto kern) {
        run_kernel(kern, grid, block, 0, s, gp, x4, gm4, mean, rstd, (f4*)dx, src4, (u16x4*)dxbf, (f4*)part, rows, C4,
                   beta_dx);
      };
      if (dxsum) {
        if (C4 <= 64)
          go(ln_bwd_fused4_k<1, true, false, GT>);
        else if (C4 == 192)
          go(ln_bwd_fused4_k<3, true, true, GT>);
        else if (C4 <= 192)
          go(ln_bwd_fused4_k<3, true, false, GT>);
        else
          go(ln_bwd_fused4_k<4, true, false, GT>);
      } else {
        if (C4 <= 64)
          go(ln_bwd_fused4_k<1, false, false, GT>);
        else if (C4 == 192)
          go(ln_bwd_fused4_k<3, false, true, GT>);
        else if (C4 <= 192)
          go(ln_bwd_fused4_k<3, false, false, GT>);
        else
          go(ln_bwd_fused4_k<4, false, false, GT>);
      }
    };
    if (dxsum) np = 3;
    if (gbf)
      launch((const u16x4*)gbf);
    else
      launch((const f4*)g);
    parts = (int)blocks;
  } else {
    if (gbf) return hipErrorInvalidValue;  // the general kernels read fp32 (the caller converts)
    dxsum = nullptr;  // not produced on this path
    if (rows > 0 && beta_dx != 0.f && dx_src != dx) {  // the kernels below accumulate into dx itself
      const hipError_t e = hipMemcpyAsync(dx, dx_src, (size_t)(rows * C) * sizeof(float), hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return e;
    }
    if (rows > 0) {
      if (C <= 64 * MAXV)
        run_kernel(ln_bwd_dx_k<true>, dim3(row_blocks(rows)), dim3(NT), 0, s, g, x, gamma, mean, rstd, dx,
                           rows, (int)C, beta_dx);
      else
        run_kernel(ln_bwd_dx_k<false>, dim3(row_blocks(rows)), dim3(NT), 0, s, g, x, gamma, mean, rstd, dx,
                           rows, (int)C, beta_dx);
    }
    parts = ln_bwd_parts(rows);
    const int64_t rows_per = (rows + parts - 1) / parts;
    run_kernel(ln_bwd_cols_k, dim3((unsigned)((C + NT - 1) / NT), (unsigned)parts), dim3(NT), 0, s, g, x,
                       mean, rstd, part, rows, (int)C, rows_per);
    if (dxbf) {
      const hipError_t e = to_bf16(dx, dxbf, rows * C, s);
      if (e != hipSuccess) return e;
    }
  }
  if (defer) {
    *defer = ReduceJob{};
    defer->kind = REDUCE_LN, defer->part = part, defer->nparts = parts, defer->np = np, defer->cols = C;
    defer->out[0] = dgamma, defer->out[1] = dbeta, defer->out[2] = dxsum;
    defer->beta[0] = beta_dg, defer->beta[1] = beta_db;
  } else {
    run_kernel(ln_bwd_reduce, dim3((unsigned)((C + 15) / 16)), dim3(1024), 0, s, part, parts, np, (int)C,
                       dgamma, dbeta, dxsum, beta_dg, beta_db);
  }
  if (dxsum_written) *dxsum_written = dxsum != nullptr;
  return hipGetLastError();
}

hipError_t reduce_batch(const ReduceJobs& jobs, hipStream_t s) {
  if (jobs.count <= 0) return hipSuccess;
  if (jobs.count > REDUCE_BATCH) return hipErrorInvalidValue;
  int64_t blocks = 1;
  for (int i = 0; i < jobs.count; ++i) {
    const ReduceJob& j = jobs.j[i];
    blocks = std::max<int64_t>(blocks, j.kind == REDUCE_LN ? (j.cols + 15) / 16 : (j.cols + 63) / 64);
  }
  run_kernel(reduce_batch_k, dim3((unsigned)blocks, (unsigned)jobs.count), dim3(1024), 0, s, jobs);
  return hipGetLastError();
}

hipError_t causal_softmax_fwd(const float* x, float* p, int64_t rows, int64_t T, bool full, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (T <= 64 * MAXV)
    run_kernel(csm_fwd_k<true>, dim3(row_blocks(rows)), dim3(NT), 0, s, x, p, rows, (int)T, full);
  else
    run_kernel(csm_fwd_k<false>, dim3(row_blocks(rows)), dim3(NT), 0, s, x, p, rows, (int)T, full);
  return hipGetLastError();
}

hipError_t causal_softmax_bwd(const float* g, const float* p, float* d, int64_t rows, int64_t T, float scale,
                              float beta, bool full, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (T <= 64 * MAXV)
    run_kernel(csm_bwd_k<true>, dim3(row_blocks(rows)), dim3(NT), 0, s, g, p, d, rows, (int)T, scale, beta,
                       full);
  else
    run_kernel(csm_bwd_k<false>, dim3(row_blocks(rows)), dim3(NT), 0, s, g, p, d, rows, (int)T, scale, beta,
                       full);
  return hipGetLastError();
}

size_t softmax_ce_workspace_bytes(int64_t rows) { return (size_t)rows * sizeof(float); }

namespace {
template <class X>
void launch_ce_fwd_grad(const X* logits, int64_t ld, const int32_t* targets, int64_t rows, int64_t V, float* lse,
                        float* loss_rows, uint16_t* dlbf, hipStream_t s) {
  const int64_t per = (V / 4 + 1023) / 1024;
  const float gn = 1.f / (float)rows;  // the backward's g / rows for g = 1
  const dim3 grid((unsigned)rows), block(1024);
  if (per <= 4)
    run_kernel((ce_fwd_grad4_k<4, X>), grid, block, 0, s, logits, ld, targets, V, lse, loss_rows, dlbf, gn);
  else if (per <= 8)
    run_kernel((ce_fwd_grad4_k<8, X>), grid, block, 0, s, logits, ld, targets, V, lse, loss_rows, dlbf, gn);
  else if (per <= 13)
    run_kernel((ce_fwd_grad4_k<13, X>), grid, block, 0, s, logits, ld, targets, V, lse, loss_rows, dlbf, gn);
  else
    run_kernel((ce_fwd_grad4_k<16, X>), grid, block, 0, s, logits, ld, targets, V, lse, loss_rows, dlbf, gn);
}
}  // namespace

bool softmax_ce_bf16_fits(int64_t ld, int64_t V, const uint16_t* logits_bf) {
  const int64_t per = (V / 4 + 1023) / 1024;
  return ld % 4 == 0 && (reinterpret_cast<uintptr_t>(logits_bf) & 7) == 0 && per >= 1 && per <= 16;
}

hipError_t softmax_ce_fwd(const float* logits, int64_t ld, const int32_t* targets, int64_t rows, int64_t V,
                          float* lse, float* loss, void* ws, hipStream_t s, uint16_t* dlbf, bool* dlbf_written,
                          const uint16_t* logits_bf) {
  if (dlbf_written) *dlbf_written = false;
  if (rows <= 0) return hipSuccess;
  float* loss_rows = static_cast<float*>(ws);
  const int64_t per = (V / 4 + 1023) / 1024;
  if (logits_bf) {  // bf16 logits: the one-pass kernel only (the gradient where dlbf is given)
    if (!softmax_ce_bf16_fits(ld, V, logits_bf) || (reinterpret_cast<uintptr_t>(dlbf) & 7) != 0)
      return hipErrorInvalidValue;
    launch_ce_fwd_grad(logits_bf, ld, targets, rows, V, lse, loss_rows, dlbf, s);
    if (dlbf_written) *dlbf_written = dlbf != nullptr;
  } else if (dlbf && ld % 4 == 0 && aligned16(logits) && (reinterpret_cast<uintptr_t>(dlbf) & 7) == 0 && per >= 1 &&
             per <= 16) {
    launch_ce_fwd_grad(logits, ld, targets, rows, V, lse, loss_rows, dlbf, s);
    if (dlbf_written) *dlbf_written = true;
  } else if (ld % 4 == 0 && aligned16(logits))
    run_kernel(ce_fwd4_k, dim3((unsigned)rows), dim3(NT), 0, s, logits, ld, targets, V, lse, loss_rows);
  else
    run_kernel(ce_fwd_k, dim3((unsigned)rows), dim3(NT), 0, s, logits, ld, targets, V, lse, loss_rows);
  run_kernel(mean_k, dim3(1), dim3(NT), 0, s, loss_rows, rows, loss);
  return hipGetLastError();
}

hipError_t softmax_ce_bwd(const float* logits, int64_t ld, const int32_t* targets, const float* lse,
                          const float* g_scalar, float* dl, uint16_t* dlbf, int64_t rows, int64_t V, float beta,
                          hipStream_t s, bool skip_if_unit, const uint16_t* logits_bf) {
  if (rows <= 0) return hipSuccess;
  if (!dl && (!dlbf || beta != 0.f)) return hipErrorInvalidValue;
  if (logits_bf) {
    if (!softmax_ce_bf16_fits(ld, V, logits_bf) || !aligned16(dl) || (reinterpret_cast<uintptr_t>(dlbf) & 7) != 0)
      return hipErrorInvalidValue;
    run_kernel(ce_bwd4_k<uint16_t>, dim3((unsigned)rows), dim3(NT), 0, s, logits_bf, ld, targets, lse, g_scalar,
                       dl, dlbf, rows, V, beta, (int)skip_if_unit);
    return hipGetLastError();
  }
  if (ld % 4 == 0 && aligned16(logits) && aligned16(dl) && (reinterpret_cast<uintptr_t>(dlbf) & 7) == 0)
    run_kernel(ce_bwd4_k<float>, dim3((unsigned)rows), dim3(NT), 0, s, logits, ld, targets, lse, g_scalar, dl, dlbf,
                       rows, V, beta, (int)skip_if_unit);
  else
    run_kernel(ce_bwd_k, dim3((unsigned)rows), dim3(NT), 0, s, logits, ld, targets, lse, g_scalar, dl, dlbf,
                       rows, V, beta, (int)skip_if_unit);
  return hipGetLastError();
}

}  // namespace tfb
