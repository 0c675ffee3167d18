// Bandwidth-bound elementwise and data-movement kernels: Add (with the bias
// broadcast), Mul, Scale, Tanh, GELU (tanh form), Sum, Narrow and the head
// permutations, with their backward rules ([Autograd-1, "Ops" and the table of
// remaining ops; GPT2-4, "Common mistakes": GELU is the tanh approximation]).
// Backward kernels take beta in {0, 1}: 0 overwrites a gradient that has not
// been written yet in this pass, 1 adds to it (the "+=" rule).  Grid-stride
// loops over float4 when the buffers allow it; reductions are two-stage and
// deterministic.
#include <algorithm>

#include <type_traits>

#include "kernels.h"
#include "gelu_dev.h"
#include "reduce_dev.h"

namespace tfb {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;

inline unsigned grid_for(int64_t n, int per_thread = 1) {
  int64_t b = (n + (int64_t)NT * per_thread - 1) / ((int64_t)NT * per_thread);
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(b, 65536));
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <typename F>
__global__ void map1(int64_t n, F f) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) f(i);
}

// bf16 bits of x, rounded to nearest even (the rounding of every bf16 operand copy)
__device__ __forceinline__ uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

__global__ void to_bf16_k(const float* __restrict__ src, uint16_t* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
    const __bf16 b = (__bf16)src[i];
    dst[i] = __builtin_bit_cast(uint16_t, b);
  }
}

typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
__global__ void to_bf16_4_k(const f4* __restrict__ src, u16x4* __restrict__ dst, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n4; i += (int64_t)gridDim.x * NT) {
    const f4 v = src[i];
    u16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __builtin_bit_cast(uint16_t, (__bf16)v[e]);
    dst[i] = o;
  }
}

__global__ void fill_k(float* p, float v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) p[i] = v;
}

__global__ void add_bcast_k(const float* __restrict__ a, const float* __restrict__ b, float* __restrict__ y,
                            int64_t n, int64_t nb) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT)
    y[i] = a[i] + b[i % nb];
}

__global__ void add_bcast4_k(const f4* __restrict__ a, const f4* __restrict__ b, f4* __restrict__ y, int64_t n4,
                             int64_t nb4) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n4; i += (int64_t)gridDim.x * NT)
    y[i] = a[i] + b[i % nb4];
}

__global__ void axpby_k(float* __restrict__ d, const float* __restrict__ s, float alpha, float beta, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
    float v = alpha * s[i];
    if (beta != 0.f) v += beta * d[i];
    d[i] = v;
  }
}

__global__ void axpby_batch_k(AxpbyJobs jobs) {
  const AxpbyJob& j = jobs.j[blockIdx.y];
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < j.n; i += (int64_t)gridDim.x * NT)
    j.dst[i] = j.beta != 0.f ? j.src[i] + j.beta * j.dst[i] : j.src[i];
}

// partial[blockIdx.y * cols + c] = sum of the rows in slab blockIdx.y (4 independent loads in flight)
__global__ void colsum_stage1(const float* __restrict__ g, int64_t rows, int64_t cols, int64_t rows_per,
                              float* __restrict__ partial) {
  const int64_t c = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (c >= cols) return;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per;
  const int64_t r1 = std::min(rows, r0 + rows_per);
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  int64_t r = r0;
  for (; r + 4 <= r1; r += 4) {
    s0 += g[r * cols + c];
    s1 += g[(r + 1) * cols + c];
    s2 += g[(r + 2) * cols + c];
    s3 += g[(r + 3) * cols + c];
  }
  for (; r < r1; ++r) s0 += g[r * cols + c];
  partial[(int64_t)blockIdx.y * cols + c] = (s0 + s1) + (s2 + s3);
}

// The same over float4 columns: a workgroup covers 256 columns (64 lanes x 4)
// and 4 row groups that interleave over the slab's rows, 8 rows in flight per
// thread; the 4 group sums are added in LDS, in a fixed order.
__device__ __forceinline__ f4 load4(const f4* p, int64_t i) { return p[i]; }
__device__ __forceinline__ f4 load4(const u16x4* p, int64_t i) {  // exact float values of 4 bf16 numbers
  const u16x4 b = p[i];
  return f4{__uint_as_float((unsigned)b[0] << 16), __uint_as_float((unsigned)b[1] << 16),
            __uint_as_float((unsigned)b[2] << 16), __uint_as_float((unsigned)b[3] << 16)};
}

template <typename GT>  // f4, or u16x4 for a gradient held as bf16
__global__ __launch_bounds__(NT) void colsum4_stage1(const GT* __restrict__ g, int64_t rows, int64_t cols4,
                                                    int64_t rows_per, f4* __restrict__ partial) {
  __shared__ f4 sh[3][64];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.x * 64 + tx;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per;
  const int64_t r1 = std::min(rows, r0 + rows_per);
  f4 acc[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
  if (c < cols4) {
    int64_t r = r0 + ty;
    for (; r + 28 < r1; r += 32) {
      f4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = load4(g, (r + 4 * u) * cols4 + c);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u & 1] += v[u];
    }
    for (; r < r1; r += 4) acc[0] += load4(g, r * cols4 + c);
  }
  const f4 t = acc[0] + acc[1];
  if (ty > 0) sh[ty - 1][tx] = t;
  __syncthreads();
  if (ty == 0 && c < cols4) partial[(int64_t)blockIdx.y * cols4 + c] = ((t + sh[0][tx]) + sh[1][tx]) + sh[2][tx];
}

// GELU backward over a [rows, cols4] float4 view that also takes the column sums
// of its result (a Linear's bias gradient when this is that Linear's output
// gradient): workgroups as in colsum4_stage1 (256 columns x a slab of rows, 4
// interleaved row groups, 4 rows in flight per thread), each element written once
// and added into its column's slab partial.

// XT: f4 (fp32 input) or u16x4 (the input's bf16 copy); GT likewise for the upstream gradient
template <typename XT, typename GT>
__global__ __launch_bounds__(NT) void gelu_bwd_cols4_k(const GT* __restrict__ g, const XT* __restrict__ x,
                                                      f4* __restrict__ d, u16x4* __restrict__ dbf, float beta,
                                                      int64_t rows, int64_t cols4, int64_t rows_per,
                                                      f4* __restrict__ partial) {
  __shared__ f4 sh[3][64];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.x * 64 + tx;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per;
  const int64_t r1 = std::min(rows, r0 + rows_per);
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  auto one = [&](f4 gv, f4 xv, int64_t i) {
    f4 v = {gv[0] * gelu_grad(xv[0]), gv[1] * gelu_grad(xv[1]), gv[2] * gelu_grad(xv[2]), gv[3] * gelu_grad(xv[3])};
    if (d) {  // null: the bf16 copy alone (beta is 0 then)
      if (beta != 0.f) v += d[i];
      d[i] = v;
    }
    if (dbf) dbf[i] = u16x4{bf16_bits(v[0]), bf16_bits(v[1]), bf16_bits(v[2]), bf16_bits(v[3])};
    acc += v;
  };
  if (c < cols4) {
    int64_t r = r0 + ty;
    for (; r + 12 < r1; r += 16) {
      f4 gv[4], xv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        gv[u] = load4(g, (r + 4 * u) * cols4 + c);
        xv[u] = load4(x, (r + 4 * u) * cols4 + c);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) one(gv[u], xv[u], (r + 4 * u) * cols4 + c);
    }
    for (; r < r1; r += 4) one(load4(g, r * cols4 + c), load4(x, r * cols4 + c), r * cols4 + c);
  }
  if (ty > 0) sh[ty - 1][tx] = acc;
  __syncthreads();
  if (ty == 0 && c < cols4) partial[(int64_t)blockIdx.y * cols4 + c] = ((acc + sh[0][tx]) + sh[1][tx]) + sh[2][tx];
}

// out[c] (+)= sum over the partial rows; 64 columns x 16 partial-groups per workgroup
__global__ __launch_bounds__(1024) void colsum_stage2(const float* __restrict__ partial, int nparts, int64_t cols,
                                                      float* __restrict__ out, float beta) {
  colsum_reduce_cols(partial, nparts, cols, out, beta, blockIdx.x);
}

__device__ __forceinline__ float block_sum(float v) {
  __shared__ float sh[NT / 64];
  for (int o = 32; o > 0; o >>= 1) v += __shfl_down(v, o, 64);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) sh[w] = v;
  __syncthreads();
  float r = 0.f;
  if (threadIdx.x == 0)
    for (int i = 0; i < NT / 64; ++i) r += sh[i];
  __syncthreads();
  return r;
}

__global__ void sum_stage1(const float* __restrict__ a, int64_t n, float* __restrict__ partial) {
  float s = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) s += a[i];
  s = block_sum(s);
  if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

__global__ void sum_stage2(const float* __restrict__ partial, int np, float* __restrict__ out) {
  float s = 0.f;
  for (int i = threadIdx.x; i < np; i += NT) s += partial[i];
  s = block_sum(s);
  if (threadIdx.x == 0) out[0] = s;
}

constexpr int SUM_BLOCKS = 1024;

}  // namespace

hipError_t fill(float* p, float v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  run_kernel(fill_k, dim3(grid_for(n, 4)), dim3(NT), 0, s, p, v, n);
  return hipGetLastError();
}

hipError_t to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 4 == 0 && aligned16(src) && (reinterpret_cast<uintptr_t>(dst) & 7) == 0)
    run_kernel(to_bf16_4_k, dim3(grid_for(n / 4, 2)), dim3(NT), 0, s, (const f4*)src, (u16x4*)dst, n / 4);
  else
    run_kernel(to_bf16_k, dim3(grid_for(n, 4)), dim3(NT), 0, s, src, dst, n);
  return hipGetLastError();
}

hipError_t add_bcast(const float* a, const float* b, float* y, int64_t n, int64_t nb, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (nb % 4 == 0 && aligned16(a) && aligned16(b) && aligned16(y))
    run_kernel(add_bcast4_k, dim3(grid_for(n / 4, 2)), dim3(NT), 0, s, (const f4*)a, (const f4*)b, (f4*)y,
                       n / 4, nb / 4);
  else
    run_kernel(add_bcast_k, dim3(grid_for(n, 4)), dim3(NT), 0, s, a, b, y, n, nb);
  return hipGetLastError();
}

hipError_t axpby(float* dst, const float* src, float alpha, float beta, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  run_kernel(axpby_k, dim3(grid_for(n, 4)), dim3(NT), 0, s, dst, src, alpha, beta, n);
  return hipGetLastError();
}

hipError_t axpby_batch(const AxpbyJobs& jobs, hipStream_t s) {
  if (jobs.count <= 0) return hipSuccess;
  if (jobs.count > AXPBY_BATCH) return hipErrorInvalidValue;
  int64_t nmax = 0;
  for (int i = 0; i < jobs.count; ++i) nmax = std::max(nmax, jobs.j[i].n);
  if (nmax <= 0) return hipSuccess;
  run_kernel(axpby_batch_k, dim3((unsigned)std::min<int64_t>((nmax + NT - 1) / NT, 64), jobs.count),
                     dim3(NT), 0, s, jobs);
  return hipGetLastError();
}

hipError_t copy_pitched(const float* src, int64_t lds, float* dst, int64_t ldd, int64_t rows, int64_t cols,
                        float beta, hipStream_t s) {
  const int64_t n = rows * cols;
  if (n <= 0) return hipSuccess;
  auto f = [=] __device__(int64_t i) {
    const int64_t r = i / cols, c = i % cols;
    float v = src[r * lds + c];
    if (beta != 0.f) v += dst[r * ldd + c];
    dst[r * ldd + c] = v;
  };
  run_kernel(map1<decltype(f)>, dim3(grid_for(n, 4)), dim3(NT), 0, s, n, f);
  return hipGetLastError();
}

hipError_t mul_fwd(const float* a, const float* b, float* y, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  auto f = [=] __device__(int64_t i) { y[i] = a[i] * b[i]; };
  run_kernel(map1<decltype(f)>, dim3(grid_for(n, 4)), dim3(NT), 0, s, n, f);
  return hipGetLastError();
}

hipError_t mul_bwd(const float* g, const float* other, float* d, float beta, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  auto f = [=] __device__(int64_t i) {
    float v = g[i] * other[i];
    if (beta != 0.f) v += d[i];
    d[i] = v;
  };
  run_kernel(map1<decltype(f)>, dim3(grid_for(n, 4)), dim3(NT), 0, s, n, f);
  return hipGetLastError();
}

hipError_t scale_fwd(const float* a, float sc, float* y, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  auto f = [=] __device__(int64_t i) { y[i] = sc * a[i]; };
  run_kernel(map1<decltype(f)>, dim3(grid_for(n, 4)), dim3(NT), 0, s, n, f);
  return hipGetLastError();
}

hipError_t tanh_fwd(const float* a, float* y, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  auto f = [=] __device__(int64_t i) { y[i] = tanhf(a[i]); };
  run_kernel(map1<decltype(f)>, dim3(grid_for(n, 4)), dim3(NT), 0, s, n, f);
  return hipGetLastError();
}

hipError_t tanh_bwd(const float* g, const float* y, float* d, float beta, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  auto f = [=] __device__(int64_t i) {
    const float t = y[i];
    float v = g[i] * (1.f - t * t);
    if (beta != 0.f) v += d[i];
    d[i] = v;
  };
  run_kernel(map1<decltype(f)>, dim3(grid_for(n, 4)), dim3(NT), 0, s, n, f);
  return hipGetLastError();
}

hipError_t to_f32(const uint16_t* src, float* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  auto f = [=] __device__(int64_t i) { dst[i] = __uint_as_float((unsigned)src[i] << 16); };
  run_kernel(map1<decltype(f)>, dim3(grid_for(n, 4)), dim3(NT), 0, s, n, f);
  return hipGetLastError();
}

hipError_t gelu_fwd_bf(const uint16_t* a, float* y, uint16_t* ybf, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 4 == 0 && (reinterpret_cast<uintptr_t>(a) & 7) == 0 && aligned16(y) &&
      (reinterpret_cast<uintptr_t>(ybf) & 7) == 0) {
    const u16x4* a4 = (const u16x4*)a;
    f4* y4 = (f4*)y;
    u16x4* b4 = (u16x4*)ybf;
    auto f = [=] __device__(int64_t i) {
      const f4 v = load4(a4, i);
      const f4 o = {gelu_f(v[0]), gelu_f(v[1]), gelu_f(v[2]), gelu_f(v[3])};
      if (y4) y4[i] = o;
      if (b4) b4[i] = u16x4{bf16_bits(o[0]), bf16_bits(o[1]), bf16_bits(o[2]), bf16_bits(o[3])};
    };
    run_kernel(map1<decltype(f)>, dim3(grid_for(n / 4, 2)), dim3(NT), 0, s, n / 4, f);
  } else {
    auto f = [=] __device__(int64_t i) {
      const float o = gelu_f(__uint_as_float((unsigned)a[i] << 16));
      if (y) y[i] = o;
      if (ybf) ybf[i] = bf16_bits(o);
    };
    run_kernel(map1<decltype(f)>, dim3(grid_for(n, 4)), dim3(NT), 0, s, n, f);
  }
  return hipGetLastError();
}

hipError_t gelu_fwd(const float* a, float* y, uint16_t* ybf, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 4 == 0 && aligned16(a) && aligned16(y) && (reinterpret_cast<uintptr_t>(ybf) & 7) == 0) {
    const f4* a4 = (const f4*)a;
    f4* y4 = (f4*)y;
    u16x4* b4 = (u16x4*)ybf;
    auto f = [=] __device__(int64_t i) {
      f4 v = a4[i];
      const f4 o = {gelu_f(v[0]), gelu_f(v[1]), gelu_f(v[2]), gelu_f(v[3])};
      if (y4) y4[i] = o;  // null: the bf16 copy alone
      if (b4) b4[i] = u16x4{bf16_bits(o[0]), bf16_bits(o[1]), bf16_bits(o[2]), bf16_bits(o[3])};
    };
    run_kernel(map1<decltype(f)>, dim3(grid_for(n / 4, 2)), dim3(NT), 0, s, n / 4, f);
  } else {
    auto f = [=] __device__(int64_t i) {
      const float o = gelu_f(a[i]);
      if (y) y[i] = o;
      if (ybf) ybf[i] = bf16_bits(o);
    };
    run_kernel(map1<decltype(f)>, dim3(grid_for(n, 4)), dim3(NT), 0, s, n, f);
  }
  return hipGetLastError();
}

hipError_t gelu_bwd(const float* g, const float* x, float* d, uint16_t* dbf, float beta, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 4 == 0 && aligned16(g) && aligned16(x) && aligned16(d) && (reinterpret_cast<uintptr_t>(dbf) & 7) == 0) {
    const f4* g4 = (const f4*)g;
    const f4* x4 = (const f4*)x;
    f4* d4 = (f4*)d;
    u16x4* b4 = (u16x4*)dbf;
    auto f = [=] __device__(int64_t i) {
      f4 gv = g4[i], xv = x4[i];
      f4 v = {gv[0] * gelu_grad(xv[0]), gv[1] * gelu_grad(xv[1]), gv[2] * gelu_grad(xv[2]),
              gv[3] * gelu_grad(xv[3])};
      if (beta != 0.f) v += d4[i];
      d4[i] = v;
      if (b4) b4[i] = u16x4{bf16_bits(v[0]), bf16_bits(v[1]), bf16_bits(v[2]), bf16_bits(v[3])};
    };
    run_kernel(map1<decltype(f)>, dim3(grid_for(n / 4, 2)), dim3(NT), 0, s, n / 4, f);
  } else {
    auto f = [=] __device__(int64_t i) {
      float v = g[i] * gelu_grad(x[i]);
      if (beta != 0.f) v += d[i];
      d[i] = v;
      if (dbf) dbf[i] = bf16_bits(v);
    };
    run_kernel(map1<decltype(f)>, dim3(grid_for(n, 4)), dim3(NT), 0, s, n, f);
  }
  return hipGetLastError();
}

static int64_t colsum_parts(int64_t rows, int64_t cols) {
  // enough row slabs to put ~2048 waves in flight, each slab at least 16 rows
  const int64_t col_blocks = (cols + NT - 1) / NT;
  int64_t parts = std::max<int64_t>(1, 512 / std::max<int64_t>(col_blocks, 1));
  parts = std::min<int64_t>(parts, std::max<int64_t>(1, rows / 16));
  return std::min<int64_t>(parts, 256);
}

// float4 path: slabs of at least 128 rows (32 per row group: four rounds of 8 loads in flight)
static int64_t colsum4_parts(int64_t rows) { return std::min<int64_t>(256, std::max<int64_t>(1, rows / 128)); }

size_t colsum_workspace_bytes(int64_t rows, int64_t cols) {
  return (size_t)std::max(colsum_parts(rows, cols), colsum4_parts(rows)) * cols * sizeof(float);
}

bool gelu_bwd_cols_fits(const float* g, const void* x, const float* d, const uint16_t* dbf, int64_t rows,
                        int64_t cols, const void* ws) {
  return rows >= 128 && cols % 4 == 0 && aligned16(g) && (reinterpret_cast<uintptr_t>(x) & 7) == 0 &&
         aligned16(d) && aligned16(ws) && (reinterpret_cast<uintptr_t>(dbf) & 7) == 0;
}

// the column reduction of slab partials: launched now, or described in *defer
static void stage2(const float* partial, int parts, int64_t cols, float* out, float beta, hipStream_t s,
                   ReduceJob* defer) {
  if (defer) {
    *defer = ReduceJob{};
    defer->kind = REDUCE_COLSUM, defer->part = partial, defer->nparts = parts, defer->cols = cols;
    defer->out[0] = out, defer->beta[0] = beta;
    return;
  }
  run_kernel(colsum_stage2, dim3((unsigned)((cols + 63) / 64)), dim3(1024), 0, s, partial, parts, cols, out,
                     beta);
}

hipError_t gelu_bwd_cols(const float* g, const float* x, float* d, uint16_t* dbf, float beta, int64_t rows,
                         int64_t cols, float* dcol, void* ws, hipStream_t s, bool* dcol_written, const uint16_t* xbf,
                         const uint16_t* gbf, ReduceJob* defer) {
  *dcol_written = false;
  if (defer) defer->kind = 0;  // nothing deferred unless the row-slab path runs
  float* partial = static_cast<float*>(ws);
  if (!d && (!dbf || beta != 0.f)) return hipErrorInvalidValue;
  const float* gchk = gbf ? reinterpret_cast<const float*>(gbf) : g;
  if (!gelu_bwd_cols_fits(gchk, xbf ? (const void*)xbf : (const void*)x, d, dbf, rows, cols, ws) ||
      (!xbf && !aligned16(x))) {
    if (xbf || gbf || !d) return hipErrorInvalidValue;  // the caller takes the fp32 forms (converting)
    return gelu_bwd(g, x, d, dbf, beta, rows * cols, s);
  }
  const int64_t parts = colsum4_parts(rows), rows_per = (rows + parts - 1) / parts, cols4 = cols / 4;
  const dim3 grid((unsigned)((cols4 + 63) / 64), (unsigned)parts);
  auto launch = [&](auto gp, auto xp) {
    using GT = std::remove_const_t<std::remove_pointer_t<decltype(gp)>>;
    using XT = std::remove_const_t<std::remove_pointer_t<decltype(xp)>>;
    run_kernel((gelu_bwd_cols4_k<XT, GT>), grid, dim3(NT), 0, s, gp, xp, (f4*)d, (u16x4*)dbf, beta, rows,
                       cols4, rows_per, (f4*)partial);
  };
  if (gbf) {
    if (xbf)
      launch((const u16x4*)gbf, (const u16x4*)xbf);
    else
      launch((const u16x4*)gbf, (const f4*)x);
  } else {
    if (xbf)
      launch((const f4*)g, (const u16x4*)xbf);
    else
      launch((const f4*)g, (const f4*)x);
  }
  stage2(partial, (int)parts, cols, dcol, 0.f, s, defer);
  *dcol_written = true;
  return hipGetLastError();
}

hipError_t colsum(const float* g, int64_t rows, int64_t cols, float* out, float beta, void* ws, hipStream_t s,
                  const uint16_t* gbf, ReduceJob* defer) {
  if (cols <= 0) return hipSuccess;
  float* partial = static_cast<float*>(ws);
  if (gbf) {  // the gradient as bf16: the float4-group path only
    if (cols % 4 != 0 || (reinterpret_cast<uintptr_t>(gbf) & 7) != 0 || !aligned16(partial) || rows <= 0)
      return hipErrorInvalidValue;
    const int64_t parts = colsum4_parts(rows), rows_per = (rows + parts - 1) / parts, cols4 = cols / 4;
    run_kernel(colsum4_stage1<u16x4>, dim3((unsigned)((cols4 + 63) / 64), (unsigned)parts), dim3(NT), 0, s,
                       (const u16x4*)gbf, rows, cols4, rows_per, (f4*)partial);
    stage2(partial, (int)parts, cols, out, beta, s, defer);
    return hipGetLastError();
  }
  if (defer) defer->kind = 0;  // nothing deferred unless the two-stage path runs
  if (rows == 1) return axpby(out, g, 1.f, beta, cols, s);
  const bool vec = cols % 4 == 0 && aligned16(g) && aligned16(partial);
  const int64_t parts = vec ? colsum4_parts(rows) : colsum_parts(rows, cols);
  const int64_t rows_per = (rows + parts - 1) / parts;
  if (vec) {
    const int64_t cols4 = cols / 4;
    dim3 g1((unsigned)((cols4 + 63) / 64), (unsigned)parts);
    if (parts == 1 && beta == 0.f && aligned16(out)) {  // few rows (a broadcast add over the batch): one pass
      run_kernel(colsum4_stage1<f4>, g1, dim3(NT), 0, s, (const f4*)g, rows, cols4, rows_per, (f4*)out);
      return hipGetLastError();
    }
    run_kernel(colsum4_stage1<f4>, g1, dim3(NT), 0, s, (const f4*)g, rows, cols4, rows_per, (f4*)partial);
  } else {
    dim3 g1((unsigned)((cols + NT - 1) / NT), (unsigned)parts);
    run_kernel(colsum_stage1, g1, dim3(NT), 0, s, g, rows, cols, rows_per, partial);
  }
  stage2(partial, (int)parts, cols, out, beta, s, defer);
  return hipGetLastError();
}

size_t sum_workspace_bytes(int64_t) { return SUM_BLOCKS * sizeof(float); }

hipError_t sum_all(const float* a, int64_t n, float* out, void* ws, hipStream_t s) {
  float* partial = static_cast<float*>(ws);
  run_kernel(sum_stage1, dim3(SUM_BLOCKS), dim3(NT), 0, s, a, n, partial);
  run_kernel(sum_stage2, dim3(1), dim3(NT), 0, s, partial, SUM_BLOCKS, out);
  return hipGetLastError();
}

hipError_t bcast_scalar_bwd(const float* gs, float* d, float beta, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  auto f = [=] __device__(int64_t i) {
    float v = gs[0];
    if (beta != 0.f) v += d[i];
    d[i] = v;
  };
  run_kernel(map1<decltype(f)>, dim3(grid_for(n, 4)), dim3(NT), 0, s, n, f);
  return hipGetLastError();
}

hipError_t narrow_fwd(const float* x, float* y, int64_t rows, int64_t cols, int64_t start, int64_t len,
                      hipStream_t s) {
  const int64_t n = rows * len;
  if (n <= 0) return hipSuccess;
  auto f = [=] __device__(int64_t i) {
    const int64_t r = i / len, c = i % len;
    y[i] = x[r * cols + start + c];
  };
  run_kernel(map1<decltype(f)>, dim3(grid_for(n, 4)), dim3(NT), 0, s, n, f);
  return hipGetLastError();
}

hipError_t narrow_bwd(const float* g, float* d, int64_t rows, int64_t cols, int64_t start, int64_t len, float beta,
                      hipStream_t s) {
  const int64_t n = rows * cols;
  if (n <= 0) return hipSuccess;
  auto f = [=] __device__(int64_t i) {
    const int64_t r = i / cols, c = i % cols;
    const bool in = c >= start && c < start + len;
    if (beta != 0.f) {
      if (in) d[i] += g[r * len + c - start];
    } else {
      d[i] = in ? g[r * len + c - start] : 0.f;
    }
  };
  run_kernel(map1<decltype(f)>, dim3(grid_for(n, 4)), dim3(NT), 0, s, n, f);
  return hipGetLastError();
}

hipError_t permute_heads(const float* x, float* y, int64_t B, int64_t T, int64_t H, int64_t hs, bool to_heads,
                         float beta, hipStream_t s) {
  const int64_t n = B * T * H * hs;
  if (n <= 0) return hipSuccess;
  // i indexes the destination
  auto f = [=] __device__(int64_t i) {
    const int64_t d = i % hs;
    int64_t rest = i / hs;
    int64_t src;
    if (to_heads) {  // dst [B, H, T, hs] <- src [B, T, H, hs]
      const int64_t t = rest % T;
      rest /= T;
      const int64_t h = rest % H, b = rest / H;
      src = ((b * T + t) * H + h) * hs + d;
    } else {  // dst [B, T, H, hs] <- src [B, H, T, hs]
      const int64_t h = rest % H;
      rest /= H;
      const int64_t t = rest % T, b = rest / T;
      src = ((b * H + h) * T + t) * hs + d;
    }
    float v = x[src];
    if (beta != 0.f) v += y[i];
    y[i] = v;
  };
  run_kernel(map1<decltype(f)>, dim3(grid_for(n, 4)), dim3(NT), 0, s, n, f);
  return hipGetLastError();
}

}  // namespace tfb
