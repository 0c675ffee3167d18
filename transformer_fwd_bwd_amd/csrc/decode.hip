// KV-cached inference ([GPT2-4, "Generation with KV cache" and "Temperature
// and Top-k"]).
//
// Cache layout: [L][2][B][Tmax][C] (keys then values of every layer); position
// p of sequence b in layer l is one contiguous row of C values, so a head's slice
// is hs contiguous values.  The values are fp32, or bf16 (round to nearest even)
// in the bf16 variant, where keys and values are operands of the q.k and p.v
// products like every other contraction operand there; arithmetic stays fp32.
//
// kv_attend: one workgroup per (sequence, head).  It appends the new token's
// key and value at position pos, then computes the single-query attention
// over positions 0..pos: scores q.k_j / sqrt(hs) (no mask: the cache holds
// only the past), a softmax, and sum_j p_j v_j.  Memory-bound: every cached
// key and value of the head is read once.
//
// sample_topk: one workgroup per sequence.  The k-th largest logit is found
// exactly by a 32-step bitwise search over order-preserving integer keys
// (count of keys >= candidate, one block reduction per step); every logit
// below it is dropped and ties with it are kept; exp((l - max)/T) is summed
// in double; the drawn id is the first (in ascending id order) whose
// cumulative weight exceeds u * sum, found by a block scan over contiguous id
// ranges and a walk inside the range that contains the crossing.
#include <algorithm>

#include "kernels.h"
#include "lanes.h"

namespace tfb {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ float block_max(float v, float* sh) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
  for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, sh[i]);
  return r;
}

__device__ __forceinline__ float block_sumf(float v, float* sh) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  float r = 0.f;
  for (int i = 0; i < NT / 64; ++i) r += sh[i];
  return r;
}

__device__ __forceinline__ int block_sumi(int v, int* sh) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  int r = 0;
  for (int i = 0; i < NT / 64; ++i) r += sh[i];
  return r;
}

// key(x) is increasing in x for every finite float
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Cross-lane sums and maxima by DPP inside each 16-lane row and by the permlane
// swaps across rows (no LDS round trip).  Every lane of the wave must be active.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// the sum over each group of G consecutive lanes, in every lane of the group: pair,
// quad, then the other quad of the half-row and the other half of the row (after
// the smaller sums those mirrors hold the partner group's sum)
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dppf<0xb1>(v);   // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v += dppf<0x4e>(v);   // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v += dppf<0x141>(v);  // row_half_mirror
  if constexpr (G >= 16) v += dppf<0x140>(v); // row_mirror
  if constexpr (G >= 32) v = lanes_xor16_add(v);
  if constexpr (G >= 64) v = lanes_xor32_add(v);
  return v;
}
// the sum (or maximum) over the lanes of this row congruent to this one mod L
// (L = 4, 8, 16 or 32), in every lane: rotations by 4 and 8 inside the row
template <int L, bool MAX>
__device__ __forceinline__ float row_stride_reduce(float v) {
  static_assert(L == 4 || L == 8 || L == 16 || L == 32, "stride");
  const auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if constexpr (L <= 4) v = op(v, dppf<0x124>(v));  // row_ror:4
  if constexpr (L <= 8) v = op(v, dppf<0x128>(v));  // row_ror:8
  return v;
}

// cache elements: fp32, or bf16 bits
__device__ __forceinline__ float kv_get(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float kv_get(const uint16_t* p, int64_t i) { return __uint_as_float((unsigned)p[i] << 16); }
__device__ __forceinline__ void kv_put(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void kv_put(uint16_t* p, int64_t i, float v) { p[i] = __builtin_bit_cast(uint16_t, (__bf16)v); }
typedef uint16_t ku4 __attribute__((ext_vector_type(4)));

template <typename KT>
__global__ __launch_bounds__(NT) void kv_store_k(const float* __restrict__ qkv, int64_t T, int C, KT* __restrict__ kv,
                                                 int layer, int B, int Tmax, int pos0) {
  // qkv [B, T, 3C] -> cache rows pos0 .. pos0 + T - 1
  const int64_t n = (int64_t)B * T * C;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) {
    const int c = (int)(i % C);
    const int64_t bt = i / C;
    const int b = (int)(bt / T), t = (int)(bt % T);
    const float* src = qkv + bt * 3 * C;
    const int64_t row = (int64_t)b * Tmax + pos0 + t;
    kv_put(kv, ((int64_t)(layer * 2 + 0) * B * Tmax + row) * C + c, src[C + c]);
    kv_put(kv, ((int64_t)(layer * 2 + 1) * B * Tmax + row) * C + c, src[2 * C + c]);
  }
}

// one workgroup per (b, head); qkv [B, 1, 3C]; y [B, 1, C]; scratch: Tmax floats of LDS
template <typename KT>
__global__ __launch_bounds__(NT) void kv_attend_k(const float* __restrict__ qkv, KT* __restrict__ kv,
                                                  float* __restrict__ y, int layer, int B, int Tmax, int C, int H,
                                                  int pos, float scale) {
  extern __shared__ float sc[];  // [pos + 1] scores, then 4 x hs partial outputs
  __shared__ float red[NT / 64];
  const int b = blockIdx.x / H, hd = blockIdx.x % H;
  const int hs = C / H;
  const float* src = qkv + (int64_t)b * 3 * C;
  KT* Kc = kv + ((int64_t)(layer * 2 + 0) * B + b) * Tmax * C + hd * hs;
  KT* Vc = kv + ((int64_t)(layer * 2 + 1) * B + b) * Tmax * C + hd * hs;
  for (int d = threadIdx.x; d < hs; d += NT) {
    kv_put(Kc, (int64_t)pos * C + d, src[C + hd * hs + d]);
    kv_put(Vc, (int64_t)pos * C + d, src[2 * C + hd * hs + d]);
  }
  __syncthreads();
  const float* q = src + hd * hs;
  for (int j = threadIdx.x; j <= pos; j += NT) {
    const KT* kr = Kc + (int64_t)j * C;
    float s = 0.f;
    for (int d = 0; d < hs; ++d) s += q[d] * kv_get(kr, d);
    sc[j] = s * scale;
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int j = threadIdx.x; j <= pos; j += NT) mx = fmaxf(mx, sc[j]);
  mx = block_max(mx, red);
  float sum = 0.f;
  for (int j = threadIdx.x; j <= pos; j += NT) {
    const float e = expf(sc[j] - mx);
    sc[j] = e;
    sum += e;
  }
  sum = block_sumf(sum, red);
  const float inv = 1.f / sum;
  __syncthreads();
  // y[d] = sum_j p_j v_j[d]: 64 d-lanes x 4 position groups
  float* part = sc + Tmax;
  const int d = threadIdx.x & 63, grp = threadIdx.x >> 6;
  for (int d0 = 0; d0 < hs; d0 += 64) {
    float acc = 0.f;
    if (d0 + d < hs)
      for (int j = grp; j <= pos; j += NT / 64) acc += sc[j] * kv_get(Vc, (int64_t)j * C + d0 + d);
    part[grp * 64 + d] = acc;
    __syncthreads();
    if (grp == 0 && d0 + d < hs) {
      float r = 0.f;
      for (int g = 0; g < NT / 64; ++g) r += part[g * 64 + d];
      y[(int64_t)b * C + hd * hs + d0 + d] = r * inv;
    }
    __syncthreads();
  }
}

// Split form of kv_attend for head sizes 32, 64 and 128.  One workgroup per
// (sequence, head, block of KVP positions): each wave takes KVP/4 positions, a
// group of lanes reads one cached key row in 16-byte pieces (8 bf16 or 4 fp32
// values per lane) and reduces its dot product across the group, then the wave
// keeps its own maximum m, weight sum l and sum_j e^(s_j - m) v_j; the four
// waves merge in LDS and the block writes (m, l, acc).  kv_attend_merge_k
// rescales the blocks to their common maximum and divides.  The block that
// holds position pos appends the new key and value and takes that row from
// registers rather than reading it back, so no block waits on the append.  The
// query, summed once per wave by a lane per float4, reaches the other lanes by
// cross-lane moves.  A block covers the same bytes of cache in either
// precision, 256 bf16 positions or 128 fp32 ones, so that a GPT-2-sized batch
// at a context near 1024 is one round of blocks.
template <typename KT>
constexpr int kv_block_positions() {
  return sizeof(KT) == 2 ? 256 : 128;
}
constexpr int KVP_MIN = 128;  // the smaller of the two: the most blocks, for workspace sizing
typedef float kf4 __attribute__((ext_vector_type(4)));
typedef unsigned kr4 __attribute__((ext_vector_type(4)));  // 16 raw bytes of a cache row

// element e of a 16-byte piece of a cache row, as fp32
template <typename KT>
struct KvPiece;
template <>
struct KvPiece<float> {
  static constexpr int W = 4;
  static __device__ __forceinline__ float at(const kr4& v, int e) { return __uint_as_float(v[e]); }
};
template <>
struct KvPiece<uint16_t> {
  static constexpr int W = 8;
  static __device__ __forceinline__ float at(const kr4& v, int e) {
    const unsigned u = v[e >> 1];
    return __uint_as_float((e & 1) ? (u & 0xffff0000u) : (u << 16));
  }
};

// qkv values of sequence b, columns i..i+3: from the stored qkv, or summed from the
// c_attn product's partials (chunks in order) plus its bias -- the values its chunk
// sum would have stored
struct QkvSrc {
  const float* qkv;
  const float* part;
  const float* bias;
  int chunks;
};
__device__ __forceinline__ kf4 qkv4(const QkvSrc& q, int B, int C, int b, int i) {
  if (!q.part) return *reinterpret_cast<const kf4*>(q.qkv + (int64_t)b * 3 * C + i);
  const int64_t stride = (int64_t)B * 3 * C;
  const float* p = q.part + (int64_t)b * 3 * C + i;
  kf4 v = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < q.chunks; c0 += 8) {  // eight loads in flight, added in chunk order
    kf4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = *reinterpret_cast<const kf4*>(p + min(c0 + j, q.chunks - 1) * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < q.chunks) v += x[j];
  }
  return v + *reinterpret_cast<const kf4*>(q.bias + i);
}

__device__ __forceinline__ void kv_put4(float* p, kf4 v) { *reinterpret_cast<kf4*>(p) = v; }
__device__ __forceinline__ void kv_put4(uint16_t* p, kf4 v) {
  *reinterpret_cast<ku4*>(p) = ku4{__builtin_bit_cast(uint16_t, (__bf16)v.x), __builtin_bit_cast(uint16_t, (__bf16)v.y),
                                   __builtin_bit_cast(uint16_t, (__bf16)v.z), __builtin_bit_cast(uint16_t, (__bf16)v.w)};
}

// raw cache bits of four values: fp32 as is, bf16 rounded to nearest-even and
// packed two to a dword (the stored form kv_put4 writes)
__device__ __forceinline__ void kv_raw4(kf4 v, unsigned* o, float*) {
  o[0] = __float_as_uint(v.x), o[1] = __float_as_uint(v.y), o[2] = __float_as_uint(v.z), o[3] = __float_as_uint(v.w);
}
__device__ __forceinline__ void kv_raw4(kf4 v, unsigned* o, uint16_t*) {
  o[0] = (unsigned)__builtin_bit_cast(uint16_t, (__bf16)v.x) | ((unsigned)__builtin_bit_cast(uint16_t, (__bf16)v.y) << 16);
  o[1] = (unsigned)__builtin_bit_cast(uint16_t, (__bf16)v.z) | ((unsigned)__builtin_bit_cast(uint16_t, (__bf16)v.w) << 16);
}

// lane (r, c) of a wave takes float4s c*N4 .. c*N4+N4-1 of a head-sized vector
// whose float4 f sits in lane f
template <int N4>
__device__ __forceinline__ void share4(kf4 v, int c, kf4* out) {
#pragma unroll
  for (int e = 0; e < N4; ++e) {
    const int src = c * N4 + e;
    out[e] = kf4{__shfl(v.x, src, 64), __shfl(v.y, src, 64), __shfl(v.z, src, 64), __shfl(v.w, src, 64)};
  }
}

template <int HS, typename KT>
__global__ __launch_bounds__(256, HS <= 64 ? 4 : 2) void kv_attend_part_k(QkvSrc qs, KT* __restrict__ kv,
                                                        float* __restrict__ pacc, float* __restrict__ pml, int layer,
                                                        int B, int Tmax, int C, int H, int pos, int S, float scale) {
  constexpr int KVP = kv_block_positions<KT>(), VW = KvPiece<KT>::W, N4 = VW / 4;
  constexpr int LPR = HS / VW, RPI = 64 / LPR, PW = KVP / 4, IT = PW / RPI;
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0 && IT >= 1 && PW % RPI == 0 && HS / 4 <= 64, "row split");
  __shared__ float wm[4], wl[4];
  __shared__ float wacc[4][HS];
  // heads fastest: the blocks that read the same cache rows (every head of one
  // block of positions) run together, so the rows' DRAM pages are opened once
  const int hd = blockIdx.x % H, s = blockIdx.x / H % S, b = blockIdx.x / H / S, bh = b * H + hd;
  KT* Kc = kv + ((int64_t)(layer * 2 + 0) * B + b) * Tmax * C + hd * HS;
  KT* Vc = kv + ((int64_t)(layer * 2 + 1) * B + b) * Tmax * C + hd * HS;
  const int j_lo = s * KVP, j_hi = min(j_lo + KVP, pos + 1);
  const bool last = pos < j_lo + KVP;  // this block holds the new token (uniform per block)
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane / LPR, c = lane % LPR;
  const int jw = j_lo + w * PW;
  // every key and value row of this wave is requested before the first is used;
  // rows past the block and the new token's row (not stored yet) read row j_lo
  // instead, an in-range address: their loaded values are replaced below
  const int j_mem = last ? pos : j_hi;
  // (non-temporal: a step streams the whole cache, more than the Infinity Cache
  // holds, so its rows are not kept there at the weights' expense)
  kr4 kr[IT], vr[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int j = jw + it * RPI + r;
    const int64_t row = (int64_t)(j < j_mem ? j : j_lo) * C + c * VW;
    kr[it] = __builtin_nontemporal_load(reinterpret_cast<const kr4*>(Kc + row));
    vr[it] = __builtin_nontemporal_load(reinterpret_cast<const kr4*>(Vc + row));
  }
  // the query: lane f < HS/4 sums float4 f once, then the wave shares it
  kf4 qf = {0.f, 0.f, 0.f, 0.f};
  if (lane < HS / 4) qf = qkv4(qs, B, C, b, hd * HS + 4 * lane);
  kf4 q4[N4];
  share4<N4>(qf, c, q4);
  if (last) {
    // the new token's key and value: wave 0 appends them to the cache; every wave
    // takes their stored (rounded) form in place of the row it did not read
    kf4 kn = {0.f, 0.f, 0.f, 0.f}, vn = {0.f, 0.f, 0.f, 0.f};
    if (lane < HS / 4) {
      kn = qkv4(qs, B, C, b, C + hd * HS + 4 * lane);
      vn = qkv4(qs, B, C, b, 2 * C + hd * HS + 4 * lane);
      if (w == 0) {
        kv_put4(Kc + (int64_t)pos * C + 4 * lane, kn);
        kv_put4(Vc + (int64_t)pos * C + 4 * lane, vn);
      }
    }
    kf4 k4[N4], v4[N4];
    share4<N4>(kn, c, k4);
    share4<N4>(vn, c, v4);
    unsigned kw[4] = {0u, 0u, 0u, 0u}, vw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < N4; ++e) {  // sizeof(KT) dwords per float4 of values
      kv_raw4(k4[e], kw + e * (int)sizeof(KT), (KT*)nullptr);
      kv_raw4(v4[e], vw + e * (int)sizeof(KT), (KT*)nullptr);
    }
    const kr4 kraw = {kw[0], kw[1], kw[2], kw[3]}, vraw = {vw[0], vw[1], vw[2], vw[3]};
#pragma unroll
    for (int it = 0; it < IT; ++it)
      if (jw + it * RPI + r == pos) kr[it] = kraw, vr[it] = vraw;
  }
  // a row past the block read a stand-in row that may not hold finite values
  // (with pos == j_lo it is the row being appended): its weight is 0, and its
  // value must be too, since 0 * inf is not 0
#pragma unroll
  for (int it = 0; it < IT; ++it)
    if (jw + it * RPI + r >= j_hi) vr[it] = kr4{0u, 0u, 0u, 0u};
  float q[VW];
#pragma unroll
  for (int e = 0; e < N4; ++e) q[4 * e] = q4[e].x, q[4 * e + 1] = q4[e].y, q[4 * e + 2] = q4[e].z, q[4 * e + 3] = q4[e].w;
  float sc[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int j = jw + it * RPI + r;
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < VW; ++e) d += q[e] * KvPiece<KT>::at(kr[it], e);
    d = group_sum<LPR>(d);
    sc[it] = j < j_hi ? d * scale : -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int it = 0; it < IT; ++it) m = fmaxf(m, sc[it]);
  m = row_stride_reduce<LPR, true>(m);
  if constexpr (LPR <= 16) m = lanes_xor16_max(m);
  m = lanes_xor32_max(m);
  // a wave past the block's end (m = -inf) gets weights exp(-inf) = 0; no branch,
  // so the value loads stay where they were issued
  const float ms = m == -INFINITY ? 0.f : m;
  float l = 0.f, acc[VW];
#pragma unroll
  for (int e = 0; e < VW; ++e) acc[e] = 0.f;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const float p = expf(sc[it] - ms);  // sc = -inf past the block: p = 0
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[e] += p * KvPiece<KT>::at(vr[it], e);
    l += p;
  }
  // across the row groups of the wave: inside each 16-lane row by DPP, then across rows
  l = row_stride_reduce<LPR, false>(l);
#pragma unroll
  for (int e = 0; e < VW; ++e) acc[e] = row_stride_reduce<LPR, false>(acc[e]);
  if constexpr (LPR <= 16) {
    l = lanes_xor16_add(l);
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[e] = lanes_xor16_add(acc[e]);
  }
  l = lanes_xor32_add(l);
#pragma unroll
  for (int e = 0; e < VW; ++e) acc[e] = lanes_xor32_add(acc[e]);
  if (lane == 0) wm[w] = m, wl[w] = l;
  if (r == 0) {
#pragma unroll
    for (int e = 0; e < VW; e += 4)
      *reinterpret_cast<kf4*>(&wacc[w][c * VW + e]) = kf4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
  }
  __syncthreads();
  if (w == 0 && lane < HS / 4) {  // one float4 of the head's output per lane
    float M = wm[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) M = fmaxf(M, wm[i]);
    float L = 0.f;
    kf4 A = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (wm[i] != -INFINITY) {
        const float f = expf(wm[i] - M);
        L += f * wl[i];
        A += f * *reinterpret_cast<const kf4*>(&wacc[i][lane * 4]);
      }
    const int64_t blk = (int64_t)bh * S + s;
    *reinterpret_cast<kf4*>(pacc + blk * HS + lane * 4) = A;
    if (lane == 0) pml[blk * 2] = M, pml[blk * 2 + 1] = L;
  }
}

// one thread per output element (b, head, d); y [B, 1, C]
__global__ __launch_bounds__(256) void kv_attend_merge_k(const float* __restrict__ pacc, const float* __restrict__ pml,
                                                         float* __restrict__ y, int BH, int HS, int S) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= BH * HS) return;
  const int bh = i / HS, d = i % HS;
  const float* ml = pml + (int64_t)bh * S * 2;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.f, A = 0.f;
  for (int s = 0; s < S; ++s) {
    const float f = expf(ml[2 * s] - M);
    L += f * ml[2 * s + 1];
    A += f * pacc[((int64_t)bh * S + s) * HS + d];
  }
  y[i] = A / L;  // y [B, C] with C = H * HS: element (b, head, d) sits at bh * HS + d
}

// one workgroup per sequence; logits rows [B, V] at stride ld; u [B] (double); out [B] ids
__global__ __launch_bounds__(NT) void sample_topk_k(const float* __restrict__ logits, int64_t ld, int V, int k,
                                                    float temperature, const double* __restrict__ u,
                                                    int32_t* __restrict__ out) {
  __shared__ int ired[NT / 64];
  __shared__ float fred[NT / 64];
  __shared__ double dsum[NT];
  const int b = blockIdx.x;
  const float* l = logits + (int64_t)b * ld;
  // k-th largest key: the largest t with #(key >= t) >= k
  uint32_t thr = 0;
  const bool filter = k > 0 && k < V;
  if (filter) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      int cnt = 0;
      for (int j = threadIdx.x; j < V; j += NT) cnt += order_key(l[j]) >= cand;
      cnt = block_sumi(cnt, ired);
      if (cnt >= k) thr = cand;
    }
  }
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < V; j += NT) mx = fmaxf(mx, l[j]);
  mx = block_max(mx, fred);
  // contiguous id range per thread, weights in double
  const int chunk = (V + NT - 1) / NT;
  const int j0 = threadIdx.x * chunk, j1 = min(V, j0 + chunk);
  double local = 0.0;
  for (int j = j0; j < j1; ++j)
    if (!filter || order_key(l[j]) >= thr) local += exp(((double)l[j] - (double)mx) / (double)temperature);
  dsum[threadIdx.x] = local;
  __syncthreads();
  // inclusive scan over the 256 per-thread sums (thread 0, in order: deterministic)
  if (threadIdx.x == 0)
    for (int i = 1; i < NT; ++i) dsum[i] += dsum[i - 1];
  __syncthreads();
  const double total = dsum[NT - 1];
  const double target = u[b] * total;
  const double before = threadIdx.x ? dsum[threadIdx.x - 1] : 0.0;
  if (before <= target && target < dsum[threadIdx.x]) {
    double c = before;
    int pick = j1 - 1;
    for (int j = j0; j < j1; ++j) {
      if (filter && order_key(l[j]) < thr) continue;
      c += exp(((double)l[j] - (double)mx) / (double)temperature);
      if (c > target) {
        pick = j;
        break;
      }
    }
    out[b] = pick;
  }
  // rounding left target at or above the total: the last id with a weight
  if (threadIdx.x == 0 && target >= total) {
    int last = V - 1;
    for (int j = V - 1; j >= 0; --j)
      if (!filter || order_key(l[j]) >= thr) {
        last = j;
        break;
      }
    out[b] = last;
  }
}

// The same draw for rows of up to SR * SPER logits, with the row held in
// registers by one 1024-thread workgroup: logit j*SR + t lives in thread t, so
// the row is read from memory once, coalesced.  The k-th largest key comes
// from the same 32-step bitwise search, counted over registers.  When at most
// SCAP logits survive the cut (the usual case: k plus its ties), their ids are
// compacted into LDS, put in ascending order by rank (ids are distinct), and
// one thread accumulates their weights in that order; otherwise the contiguous
// range scan of sample_topk_k runs with SR threads.
constexpr int SR = 1024;
constexpr int SPER = 50;
constexpr int SCAP = 512;
constexpr int SCAND = 1024;

template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
// a wave's total (or maximum) in every lane: DPP inside the 16-lane rows, then the
// four row results read as scalars
__device__ __forceinline__ int wave_sumi(int v) {
  v += dppi<0xb1>(v);
  v += dppi<0x4e>(v);
  v += dppi<0x141>(v);
  v += dppi<0x140>(v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
__device__ __forceinline__ uint32_t wave_maxu(uint32_t v) {
  v = max(v, (uint32_t)dppi<0xb1>((int)v));
  v = max(v, (uint32_t)dppi<0x4e>((int)v));
  v = max(v, (uint32_t)dppi<0x141>((int)v));
  v = max(v, (uint32_t)dppi<0x140>((int)v));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

__device__ __forceinline__ int block_sumi_sr(int v, int* sh) {
  v = wave_sumi(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int i = 0; i < SR / 64; ++i) r += sh[i];
  return r;
}

__device__ __forceinline__ uint32_t block_maxu_sr(uint32_t v, int* sh) {
  v = wave_maxu(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = (int)v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < SR / 64; ++i) r = max(r, (uint32_t)sh[i]);
  return r;
}

__global__ __launch_bounds__(SR) void sample_topk_reg_k(const float* __restrict__ logits, int64_t ld, int V, int k,
                                                        float temperature, const double* __restrict__ u,
                                                        int32_t* __restrict__ out) {
  __shared__ int ired[SR / 64];
  __shared__ int ids[SCAP];
  __shared__ int sorted[SCAP];
  __shared__ double wts[SR];  // kept weights in id order (fast path) or per-thread range sums (wide path)
  __shared__ int nkept;
  __shared__ uint32_t tmx[SR];       // per-thread maxima (the cut's lower bound)
  __shared__ uint32_t cands[SCAND];  // keys at or above the bound
  __shared__ uint32_t bound;
  __shared__ int ncand;
  const int b = blockIdx.x, t = threadIdx.x;
  const float* l = logits + (int64_t)b * ld;
  // order keys; a slot past the row holds key 0, below the key of every float but
  // a negative NaN, and the cut below is always at least 1, so it never counts.
  // Every load is issued before any is used: a slot past the row loads the row's
  // last logit and is zeroed afterwards (a load under a branch would be waited for
  // on its own, 50 round trips in a row).
  float raw[SPER];
#pragma unroll
  for (int j = 0; j < SPER; ++j) raw[j] = l[min(j * SR + t, V - 1)];
  uint32_t key[SPER];
#pragma unroll
  for (int j = 0; j < SPER; ++j) key[j] = j * SR + t < V ? order_key(raw[j]) : 0u;
  uint32_t thr = 1;  // without a cut every logit survives
  if (k > 0 && k < V) {
    // The cut is the k-th largest key: the largest x with #(key >= x) >= k.
    // A lower bound first: the k-th largest of the 1024 per-thread maxima (k of the
    // row's keys are at least that).  One wave finds it bit by bit without block
    // barriers; the keys at or above it (typically a few k) are gathered, and the
    // cut is the largest gathered key with at least k gathered keys at or above it --
    // the same value, since the counts of keys >= x agree for every x >= the bound.
    // Many gathered keys (ties across the bound) take the full search below.
    bool found = false;
    if (k <= SR) {
      uint32_t tmax = 0;
#pragma unroll
      for (int j = 0; j < SPER; ++j) tmax = max(tmax, key[j]);
      tmx[t] = tmax;
      __syncthreads();
      if (t < 64) {
        uint32_t v[SR / 64];
#pragma unroll
        for (int i = 0; i < SR / 64; ++i) v[i] = tmx[t + 64 * i];
        // Every value in [min, max] of the maxima shares their bits above the highest
        // bit where min and max differ, and so does the answer: the search starts
        // below that bit.  A step counts per lane, then sums the wave by DPP.
        uint32_t vmx = v[0], vmn = v[0];
#pragma unroll
        for (int i = 1; i < SR / 64; ++i) vmx = max(vmx, v[i]), vmn = min(vmn, v[i]);
        vmx = wave_maxu(vmx);
        vmn = ~wave_maxu(~vmn);
        const uint32_t diff = vmx ^ vmn;
        const int hb = diff ? 31 - __clz(diff) : -1;
        uint32_t lb = hb < 0 ? vmx : hb == 31 ? 0u : vmx & ~((2u << hb) - 1u);
        for (int bit = hb; bit >= 0; --bit) {
          const uint32_t cand = lb | (1u << bit);
          int c = 0;
#pragma unroll
          for (int i = 0; i < SR / 64; ++i) c += v[i] >= cand;
          if (wave_sumi(c) >= k) lb = cand;
        }
        if (t == 0) bound = lb, ncand = 0;
      }
      __syncthreads();
      const uint32_t lb = bound;
      int mine = 0;
#pragma unroll
      for (int j = 0; j < SPER; ++j) mine += key[j] >= lb;
      const int n = block_sumi_sr(mine, ired);
      if (n <= SCAND) {
#pragma unroll
        for (int j = 0; j < SPER; ++j)
          if (key[j] >= lb) cands[atomicAdd(&ncand, 1)] = key[j];
        __syncthreads();
        uint32_t best = 0;
        for (int i = t; i < n; i += SR) {
          const uint32_t c = cands[i];
          int ge = 0;
          for (int j = 0; j < n; ++j) ge += cands[j] >= c;
          if (ge >= k) best = max(best, c);
        }
        thr = block_maxu_sr(best, ired);
        found = true;
      }
    }
    if (!found) {
      thr = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < SPER; ++j) cnt += key[j] >= cand;
        if (block_sumi_sr(cnt, ired) >= k) thr = cand;
      }
    }
  }
  uint32_t kmax = 0;
  int mine = 0;
#pragma unroll
  for (int j = 0; j < SPER; ++j) {
    kmax = max(kmax, key[j]);
    mine += key[j] >= thr;
  }
  kmax = block_maxu_sr(kmax, ired);
  const float mx = __uint_as_float((kmax & 0x80000000u) ? (kmax ^ 0x80000000u) : ~kmax);
  const int n = block_sumi_sr(mine, ired);
  const double T = (double)temperature;
  if (n <= SCAP) {
    if (t == 0) nkept = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SPER; ++j)
      if (key[j] >= thr) ids[atomicAdd(&nkept, 1)] = j * SR + t;
    __syncthreads();
    if (t < n) {
      const int me = ids[t];
      int rank = 0;
      for (int i = 0; i < n; ++i) rank += ids[i] < me;
      sorted[rank] = me;
    }
    __syncthreads();
    if (t < n) wts[t] = exp(((double)l[sorted[t]] - (double)mx) / T);
    __syncthreads();
    if (t == 0) {
      double total = 0.0;
      for (int i = 0; i < n; ++i) total += wts[i];
      const double target = u[b] * total;
      double c = 0.0;
      int pick = -1, last = sorted[0];
      for (int i = 0; i < n; ++i) {
        if (wts[i] > 0.0) last = sorted[i];
        c += wts[i];
        if (c > target) {
          pick = sorted[i];
          break;
        }
      }
      out[b] = pick >= 0 ? pick : last;  // rounding left target at or above the total
    }
    return;
  }
  // many survivors (ties across the cut, or a large k): contiguous id ranges
  const int chunk = (V + SR - 1) / SR;
  const int j0 = min(V, t * chunk), j1 = min(V, j0 + chunk);
  double local = 0.0;
  for (int j = j0; j < j1; ++j)
    if (order_key(l[j]) >= thr) local += exp(((double)l[j] - (double)mx) / T);
  wts[t] = local;
  __syncthreads();
  if (t == 0)
    for (int i = 1; i < SR; ++i) wts[i] += wts[i - 1];
  __syncthreads();
  const double total = wts[SR - 1];
  const double target = u[b] * total;
  const double before = t ? wts[t - 1] : 0.0;
  if (before <= target && target < wts[t]) {
    double c = before;
    int pick = -1, last = -1;
    for (int j = j0; j < j1; ++j) {
      if (order_key(l[j]) < thr) continue;
      const double w = exp(((double)l[j] - (double)mx) / T);
      if (w > 0.0) last = j;
      c += w;
      if (c > target) {
        pick = j;
        break;
      }
    }
    out[b] = pick >= 0 ? pick : (last >= 0 ? last : j1 - 1);
  }
  if (t == 0 && target >= total) {
    int last = V - 1;
    for (int j = V - 1; j >= 0; --j)
      if (order_key(l[j]) >= thr) {
        last = j;
        break;
      }
    out[b] = last;
  }
}

}  // namespace

hipError_t kv_store(const float* qkv, int64_t T, int C, void* kv, bool kv_bf16, int layer, int B, int Tmax, int pos0,
                    hipStream_t s) {
  const int64_t n = (int64_t)B * T * C;
  if (n <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<int64_t>((n + NT - 1) / NT, 65536);
  if (kv_bf16)
    run_kernel(kv_store_k<uint16_t>, dim3(blocks), dim3(NT), 0, s, qkv, T, C, static_cast<uint16_t*>(kv), layer, B,
               Tmax, pos0);
  else
    run_kernel(kv_store_k<float>, dim3(blocks), dim3(NT), 0, s, qkv, T, C, static_cast<float*>(kv), layer, B, Tmax,
               pos0);
  return hipGetLastError();
}

static bool kv_split_ok(int C, int H) {
  const int hs = C / H;  // a head row then starts on a 16-byte boundary in either precision
  return C % H == 0 && (hs == 32 || hs == 64 || hs == 128);
}

size_t kv_attend_workspace_bytes(int B, int C, int H, int pos) {
  if (!kv_split_ok(C, H)) return 0;
  const int64_t S = (pos + KVP_MIN) / KVP_MIN;
  return (size_t)(B * S * ((int64_t)C + 2 * H)) * sizeof(float);
}

bool kv_attend_takes_parts(int C, int H) { return kv_split_ok(C, H); }

int kv_attend_blocks(bool kv_bf16, int pos) {
  const int kvp = kv_bf16 ? kv_block_positions<uint16_t>() : kv_block_positions<float>();
  return (pos + kvp) / kvp;
}

template <typename KT>
hipError_t kv_attend_t(const float* qkv, KT* kv, float* y, int layer, int B, int Tmax, int C, int H, int pos,
                       float scale, void* ws, hipStream_t s, const float* qkv_part, int qkv_chunks,
                       const float* qkv_bias) {
  if (!kv_split_ok(C, H) || ws == nullptr) {
    if (qkv_part || !y) return hipErrorInvalidValue;  // the unsplit kernel reads stored qkv, writes y
    const size_t shmem = ((size_t)Tmax + 4 * 64) * sizeof(float);
    run_kernel(kv_attend_k<KT>, dim3(B * H), dim3(NT), shmem, s, qkv, kv, y, layer, B, Tmax, C, H, pos, scale);
    return hipGetLastError();
  }
  const QkvSrc qs{qkv, qkv_part, qkv_bias, qkv_chunks};
  constexpr int KVP = kv_block_positions<KT>();
  const int hs = C / H, S = (pos + KVP) / KVP;  // blocks covering positions 0..pos
  float* pacc = static_cast<float*>(ws);
  float* pml = pacc + (int64_t)B * H * S * hs;
  const dim3 grid((unsigned)(B * H * S));
  if (hs == 32)
    run_kernel(kv_attend_part_k<32, KT>, grid, dim3(256), 0, s, qs, kv, pacc, pml, layer, B, Tmax, C, H, pos, S, scale);
  else if (hs == 64)
    run_kernel(kv_attend_part_k<64, KT>, grid, dim3(256), 0, s, qs, kv, pacc, pml, layer, B, Tmax, C, H, pos, S, scale);
  else
    run_kernel(kv_attend_part_k<128, KT>, grid, dim3(256), 0, s, qs, kv, pacc, pml, layer, B, Tmax, C, H, pos, S,
               scale);
  if (!y) return hipGetLastError();  // the per-block results are the output
  const int n = B * H * hs;
  run_kernel(kv_attend_merge_k, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, pacc, pml, y, B * H, hs, S);
  return hipGetLastError();
}

hipError_t kv_attend(const float* qkv, void* kv, bool kv_bf16, float* y, int layer, int B, int Tmax, int C, int H,
                     int pos, float scale, void* ws, hipStream_t s, const float* qkv_part, int qkv_chunks,
                     const float* qkv_bias) {
  if (kv_bf16)
    return kv_attend_t(qkv, static_cast<uint16_t*>(kv), y, layer, B, Tmax, C, H, pos, scale, ws, s, qkv_part,
                       qkv_chunks, qkv_bias);
  return kv_attend_t(qkv, static_cast<float*>(kv), y, layer, B, Tmax, C, H, pos, scale, ws, s, qkv_part, qkv_chunks,
                     qkv_bias);
}

hipError_t sample_topk(const float* logits, int64_t ld, int B, int V, int k, float temperature, const double* u,
                       int32_t* out, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (V <= SR * SPER)
    run_kernel(sample_topk_reg_k, dim3(B), dim3(SR), 0, s, logits, ld, V, k, temperature, u, out);
  else
    run_kernel(sample_topk_k, dim3(B), dim3(NT), 0, s, logits, ld, V, k, temperature, u, out);
  return hipGetLastError();
}

}  // namespace tfb
