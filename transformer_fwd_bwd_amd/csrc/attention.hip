// Fused causal multi-head attention for the bf16 variant: the forward and
// backward of  y_h = CausalSoftmax(q_h k_h^T / sqrt(hs)) v_h  without writing
// the T x T score or probability matrices to memory ([Autograd-1, table of ops:
// BatchMatMulT, Scale, CausalSoftmax, BatchMatMul; GPT2-4, "Generation with KV
// cache" for the per-head slices and the 1/sqrt(hs) scale; "The 12 unused
// tensors": row r sees keys j <= r).  The softmax is accumulated online over
// key blocks (running max m and sum l per query; the output is rescaled by
// exp(m_old - m_new) when the max grows), and the backward recomputes the
// probabilities from the saved log-sum-exp.
//
// Layout trick for the 64-lane MFMA: scores are produced transposed,
// S^T = K Q^T, with v_mfma_f32_32x32x16_bf16.  A 32x32 output block then gives
// every lane ONE query (lane % 32) and 16 keys in its registers, so the
// per-query max and sum need a single cross-lane exchange (lane ^ 32), the
// output rescale is one multiplier per lane, and the probabilities, packed to
// bf16, are directly the B operand of O^T = V^T P^T (a register block of 8
// consecutive accumulators covers keys 16s + 8(e/4) + 4(lane/32) + e%4; the
// V^T fragment is read from LDS with that same key order).  The backward uses
// the same arrangement in two kernels -- one per query block for dQ, one per
// key block for dK and dV -- so every gradient element has a single writer and
// the result is deterministic.
#include <algorithm>

#include "kernels.h"

namespace tfb {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;     // 4 wavefronts
constexpr int KVB = 64;     // keys (or queries) per staged block
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ unsigned short f2bf(float x) { return __builtin_bit_cast(unsigned short, (__bf16)x); }

__device__ __forceinline__ bf16x8 as_bf(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 consecutive accumulators (a 16-key slice of a 32x32 block) packed as a bf16 B operand
__device__ __forceinline__ bf16x8 pack8(const f32x16& acc, int base) {
  u16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = f2bf(acc[base + e]);
  return as_bf(v);
}

// row index (within a 32x32 block) held by accumulator r of lane half h
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// --- staging into LDS (all 256 threads; rows past `valid` are zero) ----------------------
// rows layout: dst[row][HS + 8], one 16-byte chunk of 8 values per transfer
template <int HS>
__device__ __forceinline__ void stage_rows(unsigned short* dst, const unsigned short* __restrict__ src, int64_t ld,
                                           int row0, int valid, int tid) {
  constexpr int CPR = HS / 8;
  for (int c = tid; c < KVB * CPR; c += NT) {
    const int row = c / CPR, col = (c % CPR) * 8;
    u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (row0 + row < valid) v = *reinterpret_cast<const u16x8*>(src + (int64_t)(row0 + row) * ld + col);
    *reinterpret_cast<u16x8*>(dst + row * (HS + 8) + col) = v;
  }
}

// transposed layout: dst[col][KVB + 8]; 4 rows x 8 columns per thread
template <int HS>
__device__ __forceinline__ void stage_cols(unsigned short* dst, const unsigned short* __restrict__ src, int64_t ld,
                                           int row0, int valid, int tid) {
  constexpr int BLOCKS = (KVB / 4) * (HS / 8);
  for (int b = tid; b < BLOCKS; b += NT) {
    const int rq = b % (KVB / 4), cq = b / (KVB / 4);
    u16x8 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + rq * 4 + i;
      v[i] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (row < valid) v[i] = *reinterpret_cast<const u16x8*>(src + (int64_t)row * ld + cq * 8);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      u16x4 w = {v[0][c], v[1][c], v[2][c], v[3][c]};
      *reinterpret_cast<u16x4*>(dst + (cq * 8 + c) * (KVB + 8) + rq * 4) = w;
    }
  }
}

// A fragment with k in the packed-register order: Xt[d][key], keys 16s + 4h + {0..3} and 16s + 8 + 4h + {0..3}
__device__ __forceinline__ bf16x8 frag_t(const unsigned short* Xt, int d, int s, int h) {
  const unsigned short* p = Xt + d * (KVB + 8) + 16 * s + 4 * h;
  u16x4 a = *reinterpret_cast<const u16x4*>(p);
  u16x4 b = *reinterpret_cast<const u16x4*>(p + 8);
  u16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return as_bf(v);
}

// A/B fragment with k contiguous: X[row][d], d = 16s + 8h + {0..7}
template <int HS>
__device__ __forceinline__ bf16x8 frag_r(const unsigned short* X, int row, int s, int h) {
  return as_bf(*reinterpret_cast<const u16x8*>(X + row * (HS + 8) + 16 * s + 8 * h));
}

// the same from global memory (zero past `valid` rows)
__device__ __forceinline__ bf16x8 frag_g(const unsigned short* __restrict__ src, int64_t ld, int row, int valid, int s,
                                         int h) {
  u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
  if (row < valid) v = *reinterpret_cast<const u16x8*>(src + (int64_t)row * ld + 16 * s + 8 * h);
  return as_bf(v);
}

struct AttnArgs {
  const unsigned short* qkv;  // bf16 [B, T, 3C]
  const unsigned short* dy;   // bf16 [B, T, C] (backward)
  const float* y;             // fp32 [B, T, C] forward output (backward: D = rowsum(dy * y))
  const float* dyf;           // fp32 [B, T, C] (backward)
  float* out;                 // forward: y; backward: dqkv fp32 [B, T, 3C]
  float* lse;                 // [B*H, T] base-2 log-sum-exp of the scaled scores
  float* D;                   // [B*H, T]
  int B, T, H, C;
  float scale;
  float beta;                 // backward: 0 overwrite dqkv, 1 add
};

// ------------------------------------------------------------------------------------ forward
template <int HS>
__global__ __launch_bounds__(NT) void attn_fwd_k(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned short Ks[KVB * (HS + 8)];
  __shared__ __attribute__((aligned(16))) unsigned short Vt[HS * (KVB + 8)];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.y, b = bh / a.H, hd = bh % a.H;
  const int q0 = blockIdx.x * 128, qw = q0 + 32 * w, q = qw + l32;
  const int64_t ld = 3LL * a.C;
  const unsigned short* base = a.qkv + (int64_t)b * a.T * ld + hd * HS;
  const unsigned short* Kg = base + a.C;
  const unsigned short* Vg = base + 2 * a.C;

  bf16x8 qf[HS / 16];
#pragma unroll
  for (int s = 0; s < HS / 16; ++s) qf[s] = frag_g(base, ld, q, a.T, s, h);

  f32x16 o[HS / 32];
#pragma unroll
  for (int i = 0; i < HS / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float sc = a.scale * LOG2E;

  const int kv_end = min(a.T, q0 + 128);
  for (int kv0 = 0; kv0 < kv_end; kv0 += KVB) {
    __syncthreads();
    stage_rows<HS>(Ks, Kg, ld, kv0, a.T, tid);
    stage_cols<HS>(Vt, Vg, ld, kv0, a.T, tid);
    __syncthreads();
    if (kv0 > qw + 31) continue;  // every key of this block is after every query of this wave
    f32x16 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[kt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < HS / 16; ++s) st[kt] = mfma(frag_r<HS>(Ks, 32 * kt + l32, s, h), qf[s], st[kt]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * kt + acc_row(r, h);
        const float v = (key <= q && key < a.T) ? st[kt][r] * sc : -INFINITY;
        st[kt][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);
    const float mref = mn == -INFINITY ? 0.f : mn;
    const float alpha = exp2f(m - mref);
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(st[kt][r] - mref);
        st[kt][r] = p;
        sum += p;
      }
    sum += __shfl_xor(sum, 32, 64);
    l = l * alpha + sum;
    m = mn;
#pragma unroll
    for (int i = 0; i < HS / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
#pragma unroll
    for (int s = 0; s < KVB / 16; ++s) {
      const bf16x8 pb = pack8(st[s >> 1], 8 * (s & 1));
#pragma unroll
      for (int i = 0; i < HS / 32; ++i) o[i] = mfma(frag_t(Vt, 32 * i + l32, s, h), pb, o[i]);
    }
  }
  if (q < a.T) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* yq = a.out + ((int64_t)b * a.T + q) * a.C + hd * HS;
#pragma unroll
    for (int i = 0; i < HS / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) yq[32 * i + acc_row(r, h)] = o[i][r] * inv;
    if (h == 0) a.lse[(int64_t)bh * a.T + q] = m + log2f(l);
  }
}

// ------------------------------------------------------------------------------------ backward
// D[bh, q] = sum_d dy[b, q, h*hs + d] * y[b, q, h*hs + d]
template <int HS>
__global__ __launch_bounds__(NT) void attn_d_k(AttnArgs a) {
  const int64_t row = (int64_t)blockIdx.x * (NT / 64) + (threadIdx.x >> 6);  // (b, q)
  const int lane = threadIdx.x & 63;
  if (row >= (int64_t)a.B * a.T) return;
  const int b = (int)(row / a.T), q = (int)(row % a.T);
  const float* g = a.dyf + row * a.C;
  const float* y = a.y + row * a.C;
  for (int hd = 0; hd < a.H; ++hd) {
    float s = 0.f;
    for (int d = lane; d < HS; d += 64) s += g[hd * HS + d] * y[hd * HS + d];
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) a.D[((int64_t)b * a.H + hd) * a.T + q] = s;
  }
}

// dQ for a block of 128 queries (4 waves x 32), looping over key blocks
template <int HS>
__global__ __launch_bounds__(NT) void attn_dq_k(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned short Ks[KVB * (HS + 8)];
  __shared__ __attribute__((aligned(16))) unsigned short Kt[HS * (KVB + 8)];
  __shared__ __attribute__((aligned(16))) unsigned short Vs[KVB * (HS + 8)];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.y, b = bh / a.H, hd = bh % a.H;
  const int q0 = blockIdx.x * 128, qw = q0 + 32 * w, q = qw + l32;
  const int64_t ld = 3LL * a.C;
  const unsigned short* base = a.qkv + (int64_t)b * a.T * ld + hd * HS;
  const unsigned short* Kg = base + a.C;
  const unsigned short* Vg = base + 2 * a.C;
  const unsigned short* dyg = a.dy + (int64_t)b * a.T * a.C + hd * HS;

  bf16x8 qf[HS / 16], df[HS / 16];
#pragma unroll
  for (int s = 0; s < HS / 16; ++s) {
    qf[s] = frag_g(base, ld, q, a.T, s, h);
    df[s] = frag_g(dyg, a.C, q, a.T, s, h);
  }
  const float lse = q < a.T ? a.lse[(int64_t)bh * a.T + q] : 0.f;
  const float Dq = q < a.T ? a.D[(int64_t)bh * a.T + q] : 0.f;
  const float sc = a.scale * LOG2E;

  f32x16 dq[HS / 32];
#pragma unroll
  for (int i = 0; i < HS / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[i][r] = 0.f;

  const int kv_end = min(a.T, q0 + 128);
  for (int kv0 = 0; kv0 < kv_end; kv0 += KVB) {
    __syncthreads();
    stage_rows<HS>(Ks, Kg, ld, kv0, a.T, tid);
    stage_cols<HS>(Kt, Kg, ld, kv0, a.T, tid);
    stage_rows<HS>(Vs, Vg, ld, kv0, a.T, tid);
    __syncthreads();
    if (kv0 > qw + 31) continue;
    f32x16 st[2], dp[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[kt][r] = dp[kt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < HS / 16; ++s) {
        st[kt] = mfma(frag_r<HS>(Ks, 32 * kt + l32, s, h), qf[s], st[kt]);
        dp[kt] = mfma(frag_r<HS>(Vs, 32 * kt + l32, s, h), df[s], dp[kt]);
      }
    }
    // dS^T = P^T (dP^T - D)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * kt + acc_row(r, h);
        const float p = (key <= q && key < a.T) ? exp2f(st[kt][r] * sc - lse) : 0.f;
        st[kt][r] = p * (dp[kt][r] - Dq);
      }
#pragma unroll
    for (int s = 0; s < KVB / 16; ++s) {
      const bf16x8 sb = pack8(st[s >> 1], 8 * (s & 1));
#pragma unroll
      for (int i = 0; i < HS / 32; ++i) dq[i] = mfma(frag_t(Kt, 32 * i + l32, s, h), sb, dq[i]);
    }
  }
  if (q < a.T) {
    float* dst = a.out + ((int64_t)b * a.T + q) * ld + hd * HS;
#pragma unroll
    for (int i = 0; i < HS / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = a.scale * dq[i][r];
        float* p = dst + 32 * i + acc_row(r, h);
        if (a.beta != 0.f) v += *p;
        *p = v;
      }
  }
}

// dK and dV for a block of 128 keys (4 waves x 32), looping over query blocks
template <int HS>
__global__ __launch_bounds__(NT) void attn_dkv_k(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned short Qs[KVB * (HS + 8)];
  __shared__ __attribute__((aligned(16))) unsigned short Qt[HS * (KVB + 8)];
  __shared__ __attribute__((aligned(16))) unsigned short Ds[KVB * (HS + 8)];
  __shared__ __attribute__((aligned(16))) unsigned short Dt[HS * (KVB + 8)];
  __shared__ float Ls[KVB], Dd[KVB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.y, b = bh / a.H, hd = bh % a.H;
  const int k0 = blockIdx.x * 128, kw = k0 + 32 * w, key = kw + l32;
  const int64_t ld = 3LL * a.C;
  const unsigned short* base = a.qkv + (int64_t)b * a.T * ld + hd * HS;
  const unsigned short* dyg = a.dy + (int64_t)b * a.T * a.C + hd * HS;

  bf16x8 kf[HS / 16], vf[HS / 16];
#pragma unroll
  for (int s = 0; s < HS / 16; ++s) {
    kf[s] = frag_g(base + a.C, ld, key, a.T, s, h);
    vf[s] = frag_g(base + 2 * a.C, ld, key, a.T, s, h);
  }
  const float sc = a.scale * LOG2E;
  f32x16 dk[HS / 32], dv[HS / 32];
#pragma unroll
  for (int i = 0; i < HS / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[i][r] = dv[i][r] = 0.f;

  for (int qb = (k0 / KVB) * KVB; qb < a.T; qb += KVB) {
    __syncthreads();
    stage_rows<HS>(Qs, base, ld, qb, a.T, tid);
    stage_cols<HS>(Qt, base, ld, qb, a.T, tid);
    stage_rows<HS>(Ds, dyg, a.C, qb, a.T, tid);
    stage_cols<HS>(Dt, dyg, a.C, qb, a.T, tid);
    if (tid < KVB) {
      const int qq = qb + tid;
      Ls[tid] = qq < a.T ? a.lse[(int64_t)bh * a.T + qq] : 0.f;
      Dd[tid] = qq < a.T ? a.D[(int64_t)bh * a.T + qq] : 0.f;
    }
    __syncthreads();
    if (qb + KVB - 1 < kw) continue;  // every query of this block precedes every key of this wave
    f32x16 st[2], dp[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[qt][r] = dp[qt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < HS / 16; ++s) {
        st[qt] = mfma(frag_r<HS>(Qs, 32 * qt + l32, s, h), kf[s], st[qt]);
        dp[qt] = mfma(frag_r<HS>(Ds, 32 * qt + l32, s, h), vf[s], dp[qt]);
      }
    }
    // P and dS with queries in registers, this lane's key in the column
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = 32 * qt + acc_row(r, h), qq = qb + qi;
        const float p = (key <= qq && qq < a.T && key < a.T) ? exp2f(st[qt][r] * sc - Ls[qi]) : 0.f;
        st[qt][r] = p;
        dp[qt][r] = p * (dp[qt][r] - Dd[qi]);
      }
#pragma unroll
    for (int s = 0; s < KVB / 16; ++s) {
      const bf16x8 pb = pack8(st[s >> 1], 8 * (s & 1));
      const bf16x8 db = pack8(dp[s >> 1], 8 * (s & 1));
#pragma unroll
      for (int i = 0; i < HS / 32; ++i) {
        dv[i] = mfma(frag_t(Dt, 32 * i + l32, s, h), pb, dv[i]);
        dk[i] = mfma(frag_t(Qt, 32 * i + l32, s, h), db, dk[i]);
      }
    }
  }
  if (key < a.T) {
    float* dst = a.out + ((int64_t)b * a.T + key) * ld + hd * HS;
#pragma unroll
    for (int i = 0; i < HS / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * i + acc_row(r, h);
        float vk = a.scale * dk[i][r], vv = dv[i][r];
        if (a.beta != 0.f) {
          vk += dst[a.C + d];
          vv += dst[2 * a.C + d];
        }
        dst[a.C + d] = vk;
        dst[2 * a.C + d] = vv;
      }
  }
}

}  // namespace

bool flash_attention_supported(int hs, int64_t C) { return (hs == 64 || hs == 32) && C % 8 == 0; }

hipError_t flash_attention_fwd(const uint16_t* qkv, float* y, float* lse, int B, int T, int H, int C, float scale,
                               hipStream_t s) {
  if (B <= 0 || T <= 0) return hipSuccess;
  AttnArgs a{};
  a.qkv = qkv, a.out = y, a.lse = lse, a.B = B, a.T = T, a.H = H, a.C = C, a.scale = scale;
  dim3 grid((T + 127) / 128, B * H);
  const int hs = C / H;
  if (hs == 64)
    hipLaunchKernelGGL(attn_fwd_k<64>, grid, dim3(NT), 0, s, a);
  else if (hs == 32)
    hipLaunchKernelGGL(attn_fwd_k<32>, grid, dim3(NT), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t flash_attention_bwd(const uint16_t* qkv, const float* y, const float* dyf, const uint16_t* dy,
                               const float* lse, float* D, float* dqkv, float beta, int B, int T, int H, int C,
                               float scale, hipStream_t s) {
  if (B <= 0 || T <= 0) return hipSuccess;
  AttnArgs a{};
  a.qkv = qkv, a.y = y, a.dyf = dyf, a.dy = dy, a.lse = const_cast<float*>(lse), a.D = D, a.out = dqkv;
  a.B = B, a.T = T, a.H = H, a.C = C, a.scale = scale, a.beta = beta;
  const int hs = C / H;
  dim3 gd((unsigned)(((int64_t)B * T + 3) / 4));
  dim3 grid((T + 127) / 128, B * H);
  if (hs == 64) {
    hipLaunchKernelGGL(attn_d_k<64>, gd, dim3(NT), 0, s, a);
    hipLaunchKernelGGL(attn_dq_k<64>, grid, dim3(NT), 0, s, a);
    hipLaunchKernelGGL(attn_dkv_k<64>, grid, dim3(NT), 0, s, a);
  } else if (hs == 32) {
    hipLaunchKernelGGL(attn_d_k<32>, gd, dim3(NT), 0, s, a);
    hipLaunchKernelGGL(attn_dq_k<32>, grid, dim3(NT), 0, s, a);
    hipLaunchKernelGGL(attn_dkv_k<32>, grid, dim3(NT), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tfb
