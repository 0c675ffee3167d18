// Embedding: row gather forward, scatter-add backward ([Autograd-1, table of
// ops: Embedding; GPT2-4, "Generation with KV cache": token and position
// embeddings added]).
//
// The backward is a sorted segment sum, so the result does not depend on
// scheduling: the (id, row) keys are sorted in chunks of CHUNK keys (one
// workgroup bitonic-sorts a chunk in LDS), then for each chunk, in chunk order,
// one wavefront per run of equal ids sums that run's gradient rows in
// ascending row order and adds the sum to the table row.  Runs inside a chunk
// touch distinct table rows, so no atomics are needed.
#include <algorithm>

#include "kernels.h"

namespace tfb {
namespace {

constexpr int NT = 256;
constexpr int CHUNK = 4096;
constexpr int SORT_THREADS = 1024;

typedef float f4 __attribute__((ext_vector_type(4)));

// ids outside [0, rows) are a caller error; they read as a zero row here and
// are skipped by the backward, so a bad id can never touch memory outside the table
__global__ void gather_k(const float* __restrict__ table, int64_t rows, const int32_t* __restrict__ ids,
                         float* __restrict__ y, int64_t n, int64_t C) {
  const int64_t total = n * C;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < total; i += (int64_t)gridDim.x * NT) {
    const int64_t r = i / C, c = i % C;
    const int64_t id = ids[r];
    y[i] = (id >= 0 && id < rows) ? table[id * C + c] : 0.f;
  }
}

__global__ void gather4_k(const f4* __restrict__ table, int64_t rows, const int32_t* __restrict__ ids,
                          f4* __restrict__ y, int64_t n, int64_t C4) {
  const int64_t total = n * C4;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < total; i += (int64_t)gridDim.x * NT) {
    const int64_t r = i / C4, c = i % C4;
    const int64_t id = ids[r];
    y[i] = (id >= 0 && id < rows) ? table[id * C4 + c] : f4{0.f, 0.f, 0.f, 0.f};
  }
}

// sort keys (id << 32 | row) of one chunk; pads with all-ones keys
__global__ __launch_bounds__(SORT_THREADS) void sort_chunks_k(const int32_t* __restrict__ ids, int64_t n,
                                                              uint64_t* __restrict__ keys_out) {
  __shared__ uint64_t k[CHUNK];
  const int64_t base = (int64_t)blockIdx.x * CHUNK;
  for (int i = threadIdx.x; i < CHUNK; i += SORT_THREADS) {
    const int64_t r = base + i;
    k[i] = r < n ? ((uint64_t)(uint32_t)ids[r] << 32) | (uint64_t)(uint32_t)r : ~0ull;
  }
  __syncthreads();
  for (int size = 2; size <= CHUNK; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < CHUNK / 2; i += SORT_THREADS) {
        // i-th compare pair: lo index has a zero at bit `stride`
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t a = k[lo], b = k[hi];
        if ((a > b) == up) {
          k[lo] = b;
          k[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < CHUNK; i += SORT_THREADS) keys_out[base + i] = k[i];
}

// one wavefront per chunk position; positions that start a run sum it.  The
// wave reads keys p-1 .. p+62 at once (lane i holds key p-1+i), finds its run
// with one ballot, takes the run's rows from those lanes, and requests the
// gradient rows two at a time with every column load issued before the first
// is added (out-of-range columns and rows load a valid element and are not
// added; two rather than four keeps four waves a SIMD).  Rows are added in
// ascending order, as the sort left them.
__global__ __launch_bounds__(NT) void segsum_k(const uint64_t* __restrict__ keys, int len, const float* __restrict__ g,
                                               int64_t C, float* __restrict__ dtable, int64_t rows) {
  constexpr int RB = 2;  // rows in flight
  const int p = __builtin_amdgcn_readfirstlane(blockIdx.x * (NT / 64) + (threadIdx.x >> 6));  // uniform per wave
  const int lane = threadIdx.x & 63;
  if (p >= len) return;
  const int kq = p - 1 + lane;
  const uint64_t kv = keys[min(max(kq, 0), len - 1)];
  const uint32_t kid = (uint32_t)(kv >> 32), krow = (uint32_t)kv;
  const uint32_t id = (uint32_t)__builtin_amdgcn_readlane((int)kid, 1);
  if ((int64_t)id >= rows) return;  // negative ids sort as large unsigned values
  if (p > 0 && (uint32_t)__builtin_amdgcn_readlane((int)kid, 0) == id) return;
  // lanes 1.. holding this id, consecutively from lane 1: the run inside the window
  const uint64_t same = __ballot(lane >= 1 && kq < len && kid == id);
  int e = p + (int)__builtin_ctzll(~(same >> 1));
  if (e == p + 63)
    while (e < len && (uint32_t)(keys[e] >> 32) == id) ++e;
  float* dst = dtable + (int64_t)id * C;
  for (int64_t c0 = 0; c0 < C; c0 += 64 * 16) {
    float acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
    for (int q = p; q < e; q += RB) {
      float v[RB][16];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int qi = min(q + i, e - 1);
        const int64_t r = qi - p < 63 ? (int64_t)(uint32_t)__builtin_amdgcn_readlane((int)krow, qi - p + 1)
                                      : (int64_t)(uint32_t)(keys[qi] & 0xffffffffu);
        const float* src = g + r * C;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int64_t c = c0 + lane + 64 * j;
          v[i][j] = src[c < C ? c : 0];
        }
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        if (q + i >= e) break;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (c0 + lane + 64 * j < C) acc[j] += v[i][j];
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t c = c0 + lane + 64 * j;
      if (c < C) dst[c] += acc[j];
    }
  }
}

}  // namespace

hipError_t embedding_fwd(const float* table, int64_t rows, const int32_t* ids, float* y, int64_t n, int64_t C,
                         hipStream_t s) {
  const int64_t total = n * C;
  if (total <= 0) return hipSuccess;
  const bool v4 = C % 4 == 0 && (reinterpret_cast<uintptr_t>(table) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(y) & 15) == 0;
  if (v4) {
    const int64_t t4 = total / 4;
    unsigned blocks = (unsigned)std::min<int64_t>((t4 + NT - 1) / NT, 65536);
    run_kernel(gather4_k, dim3(blocks), dim3(NT), 0, s, (const f4*)table, rows, ids, (f4*)y, n, C / 4);
  } else {
    unsigned blocks = (unsigned)std::min<int64_t>((total + NT - 1) / NT, 65536);
    run_kernel(gather_k, dim3(blocks), dim3(NT), 0, s, table, rows, ids, y, n, C);
  }
  return hipGetLastError();
}

size_t embedding_bwd_workspace_bytes(int64_t n) {
  const int64_t chunks = (n + CHUNK - 1) / CHUNK;
  return (size_t)std::max<int64_t>(chunks, 1) * CHUNK * sizeof(uint64_t);
}

hipError_t embedding_bwd(const float* g, const int32_t* ids, int64_t n, int64_t C, float* dtable, int64_t rows,
                         void* ws, hipStream_t s) {
  if (n <= 0 || C <= 0) return hipSuccess;
  if (n > 0x7fffffff) return hipErrorInvalidValue;
  const int64_t chunks = (n + CHUNK - 1) / CHUNK;
  uint64_t* keys = static_cast<uint64_t*>(ws);
  run_kernel(sort_chunks_k, dim3((unsigned)chunks), dim3(SORT_THREADS), 0, s, ids, n, keys);
  for (int64_t c = 0; c < chunks; ++c) {
    const int len = (int)std::min<int64_t>(CHUNK, n - c * CHUNK);
    const unsigned blocks = (unsigned)((len + (NT / 64) - 1) / (NT / 64));
    run_kernel(segsum_k, dim3(blocks), dim3(NT), 0, s, keys + c * CHUNK, len, g, C, dtable, rows);
  }
  return hipGetLastError();
}

}  // namespace tfb
