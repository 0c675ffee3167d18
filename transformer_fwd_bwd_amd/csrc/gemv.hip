// Products with at most 16 rows: C = alpha A B + bias + beta C + resid with A
// [M, K] row-major and B [K, N] row-major (the Linear of one token per sequence
// in cached decoding; [Autograd-1, "Why fast MatMul"] defines the product).
//
// Such a product reads its weight once and does 16 multiply-adds per weight,
// so it is bound by how many bytes are in flight, not by arithmetic.  The
// columns go in strips of 64 and k in chunks of kc <= 128 rows, one 256-thread
// workgroup per (strip, chunk), which puts a few hundred workgroups on the
// 256 CUs.  In the bf16 variant (both operands bf16 values, stored so or
// rounded as they load) a workgroup multiplies on MFMA (gemv_k's MF path); in
// fp32, lane 4c + r of wave w multiplies columns 4c..4c+3 of k rows
// 4w + r + 16i by the 16 rows of A (staged in LDS, k-major, as fp32) and the
// four lanes of a quad sum through DPP.  Either way the four waves' partial
// tiles meet in LDS.  A product with B stored [N, K] (the LM head) takes the
// NT form below, one launch with no partials.
//
// With one chunk the workgroup applies the epilogue; otherwise it writes its
// partial to ws[chunk][M][N] and gemv_reduce_k sums the chunks in order and
// applies the epilogue.  Summing them in the workgroup of a strip that
// finishes last would need device-scope fences, which write back and
// invalidate the L2 of the workgroup's XCD: far slower here.
#include <algorithm>
#include <type_traits>

#include "gelu_dev.h"
#include "kernels.h"

namespace tfb {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr int SM = 16;    // rows of A held
constexpr int SNS = 64;   // columns per strip
constexpr int SKC = 128;  // largest k chunk
constexpr int ST = 256;

__device__ __forceinline__ float bf16_val(unsigned short b) { return __uint_as_float((unsigned)b << 16); }
__device__ __forceinline__ unsigned short bf16_of(float x) { return __builtin_bit_cast(unsigned short, (__bf16)x); }
__device__ __forceinline__ float round_bf16(float x) { return bf16_val(bf16_of(x)); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// sum over the four lanes of a quad (quad_perm [1,0,3,2], then [2,3,0,1])
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp<0xb1>(v);
  return v + dpp<0x4e>(v);
}

struct SkArgs {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  float* C;
  int64_t ldc;
  uint16_t* Cbf;
  const float* bias;
  const float* resid;
  float alpha, beta;
  int M, N, K, kc, chunks, skipc;
  float* ws;  // [chunks][M][N] partials
  int post;   // GemmPost
  const float* ln_gamma;
  const float* ln_beta;
  float ln_eps;
  float* ln_y;
  uint16_t* ln_ybf;
  const float* a_part;  // A_PARTS: A from the previous product's partials (GemmArgs)
  const float* a_bias;
  int a_chunks;
  const float* att_acc;  // A_ATTN: A merged from the cached attention's blocks (GemmArgs)
  const float* att_ml;
  int att_blocks, att_hs, att_heads;
};

// where the kernel takes A from
enum ASrc { A_MEM = 0, A_PARTS = 1, A_ATTN = 2 };

// A from the cached attention's per-block results: their merge, in the order and
// arithmetic of the attention's own merge pass, rounded to bf16 in the bf16
// variant.  A thread stages four consecutive columns of one head (head sizes are
// multiples of 4), so one (M_s, l_s) load and one float4 of acc_s serve four
// elements.  With at most AT_BATCH blocks (a context of 2048 bf16 or 1024 fp32
// positions) all of a thread's loads are issued before the first is used: one
// round of loads for the whole staging.  Longer contexts walk the blocks.
constexpr int AT_BATCH = 8;
template <bool RND>
__device__ __forceinline__ f4 att_finish(f4 A, float L) {
  f4 v = {A.x / L, A.y / L, A.z / L, A.w / L};
  if constexpr (RND) v = f4{round_bf16(v.x), round_bf16(v.y), round_bf16(v.z), round_bf16(v.w)};
  return v;
}

// MF: both operands are bf16 values (stored so, or rounded as they load), so
// the 16-row product runs on MFMA: A staged as bf16 rows [m][k], B as bf16
// k-rows of the strip (64-byte column blocks swapped on every other pair of
// k-rows, so the four k-rows of a transposing read fall in distinct banks), each
// wave taking two of the chunk's 16-deep k-steps on 32x32x16 tiles (rows 16..31
// zero); the waves' partial tiles meet in `red` as the VALU path's do.
template <bool A_BF, bool B_BF, bool RND, int ASRC>
__global__ __launch_bounds__(ST) void gemv_k(SkArgs a) {
  constexpr bool MF = B_BF && (A_BF || RND);
  constexpr int AP = SKC + 8;  // sA16 row pitch (elements)
  __shared__ f4 sA[MF ? 1 : SKC][SM / 4];  // sA[k][q] = A rows 4q..4q+3 at k (VALU path)
  __shared__ __attribute__((aligned(16))) unsigned short sA16[MF ? SM : 1][AP];    // MFMA path: A[m][k]
  __shared__ __attribute__((aligned(16))) unsigned short sB[MF ? SKC * SNS : 1];   // MFMA path: B k-rows
  __shared__ f4 red[4][SM * SNS / 4];
  const int strips = (a.N + SNS - 1) / SNS;
  const int strip = blockIdx.x % strips, chunk = blockIdx.x / strips;
  const int n0 = strip * SNS, k0 = chunk * a.kc;
  const int kn = min(a.kc, a.K - k0);
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, r = lane & 3, c = lane >> 2;

  // every load is issued before any value is used: indexes out of range are
  // clamped to a valid element and the value is zeroed afterwards (a load under a
  // branch would be waited for on its own)
  using braw_t = typename std::conditional<B_BF, u16x4, f4>::type;
  using araw_t = typename std::conditional<A_BF, unsigned short, float>::type;
  using belem_t = typename std::conditional<B_BF, unsigned short, float>::type;
  const belem_t* Bp = static_cast<const belem_t*>(a.B);
  const int n = n0 + 4 * c;
  const bool ncol = n < a.N;
  braw_t braw[SKC / 16];
#pragma unroll
  for (int i = 0; i < SKC / 16; ++i) {
    const int kk = 4 * w + r + 16 * i;
    const int64_t off = (int64_t)(k0 + (kk < kn ? kk : 0)) * a.ldb + (ncol ? n : 0);
    braw[i] = *reinterpret_cast<const braw_t*>(Bp + off);
  }
  // A[0..M) x [k0, k0 + kn): element i of this thread's share is (i / SKC, i % SKC)
  araw_t araw[SM * SKC / ST];
  if constexpr (ASRC == A_MEM) {
#pragma unroll
    for (int j = 0; j < SM * SKC / ST; ++j) {
      const int i = t + j * ST, m = i / SKC, kk = i % SKC;
      araw[j] = static_cast<const araw_t*>(a.A)[(int64_t)(m < a.M ? m : 0) * a.lda + k0 + (kk < kn ? kk : 0)];
    }
  }
  f4 b[SKC / 16];
  if constexpr (MF) {
    // k-row kk of the strip: 128 bytes, column block (32 columns, 64 bytes) cb at
    // block cb ^ ((kk >> 1) & 1); out-of-range weights are stored as zeros
#pragma unroll
    for (int i = 0; i < SKC / 16; ++i) {
      const int kk = 4 * w + r + 16 * i, cl = 4 * c;
      const int blk = (cl >> 5) ^ ((kk >> 1) & 1);
      *reinterpret_cast<u16x4*>(reinterpret_cast<char*>(sB) + kk * 128 + blk * 64 + (cl & 31) * 2) =
          ncol && kk < kn ? braw[i] : u16x4{0, 0, 0, 0};
    }
  } else {
#pragma unroll
  for (int i = 0; i < SKC / 16; ++i) {
    const int kk = 4 * w + r + 16 * i;
    f4 v;
    if constexpr (B_BF) {
      v = f4{bf16_val(braw[i].x), bf16_val(braw[i].y), bf16_val(braw[i].z), bf16_val(braw[i].w)};
    } else {
      v = braw[i];
      if constexpr (RND) v = f4{round_bf16(v.x), round_bf16(v.y), round_bf16(v.z), round_bf16(v.w)};
    }
    b[i] = ncol && kk < kn ? v : f4{0.f, 0.f, 0.f, 0.f};
  }
  }
  // staged as fp32, k-major (bf16 [m][k] on the MFMA path); rows past M and k past
  // the chunk are zero
  auto put = [&](int m, int kk, float v) __attribute__((always_inline)) {
    if constexpr (MF)
      sA16[m][kk] = bf16_of(v);  // a bf16 value already: exact
    else
      reinterpret_cast<float*>(sA)[kk * SM + m] = v;
  };
  constexpr int E = SM * SKC / ST;
  if constexpr (ASRC == A_ATTN) {
    // thread t stages columns kq..kq+3 of rows m = t / (SKC/4) + g * (ST / (SKC/4))
    constexpr int Q = SKC / 4, G = E / 4;
    const int S = a.att_blocks;
    const int kq = 4 * (t % Q);
    const bool kin = kq < kn;
    const int k = k0 + (kin ? kq : 0), hd = k / a.att_hs, d = k - hd * a.att_hs;
    const float* mlp[G];
    const float* accp[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int m = t / Q + g * (ST / Q);
      const int64_t blk0 = ((int64_t)(m < a.M ? m : 0) * a.att_heads + hd) * S;
      mlp[g] = a.att_ml + blk0 * 2;
      accp[g] = a.att_acc + blk0 * a.att_hs + d;
    }
    float M[G], L[G];
    f4 A[G];
#pragma unroll
    for (int g = 0; g < G; ++g) M[g] = -INFINITY, L[g] = 0.f, A[g] = f4{0.f, 0.f, 0.f, 0.f};
    if (S <= AT_BATCH) {  // uniform over the grid
      typedef float ff2 __attribute__((ext_vector_type(2)));
      ff2 ml[G][AT_BATCH];
      f4 ac[G][AT_BATCH];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int q = 0; q < AT_BATCH; ++q) {  // blocks past S repeat block S - 1 and are skipped
          const int sq = min(q, S - 1);
          ml[g][q] = *reinterpret_cast<const ff2*>(mlp[g] + 2 * sq);
          ac[g][q] = *reinterpret_cast<const f4*>(accp[g] + (int64_t)sq * a.att_hs);
        }
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int q = 0; q < AT_BATCH; ++q) M[g] = fmaxf(M[g], ml[g][q].x);
#pragma unroll
        for (int q = 0; q < AT_BATCH; ++q)
          if (q < S) {
            const float f = expf(ml[g][q].x - M[g]);
            L[g] += f * ml[g][q].y;
            A[g] += f * ac[g][q];
          }
      }
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        for (int s = 0; s < S; ++s) M[g] = fmaxf(M[g], mlp[g][2 * s]);
        for (int s = 0; s < S; ++s) {
          const float f = expf(mlp[g][2 * s] - M[g]);
          L[g] += f * mlp[g][2 * s + 1];
          A[g] += f * *reinterpret_cast<const f4*>(accp[g] + (int64_t)s * a.att_hs);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int m = t / Q + g * (ST / Q);
      const bool ok = m < a.M && kin;
      const f4 v = ok ? att_finish<RND>(A[g], L[g]) : f4{0.f, 0.f, 0.f, 0.f};
      if constexpr (MF) {
        *reinterpret_cast<u16x4*>(&sA16[m][kq]) = u16x4{bf16_of(v.x), bf16_of(v.y), bf16_of(v.z), bf16_of(v.w)};
      } else {
        float* col = reinterpret_cast<float*>(sA) + kq * SM + m;
        col[0] = v.x, col[SM] = v.y, col[2 * SM] = v.z, col[3 * SM] = v.w;
      }
    }
  } else if constexpr (ASRC == A_PARTS) {
    // A from the previous few-row product's partials: gelu(the sum of its chunks in
    // chunk order + bias), rounded to bf16 in the bf16 variant -- the values that
    // product's reduction would have stored.  As above, a thread stages four
    // consecutive columns of one row (K is a multiple of 4 here), and the chunks of
    // both its rows are requested before any is used.
    constexpr int Q = SKC / 4, G = E / 4;
    const int kq = 4 * (t % Q);
    const bool kin = kq < kn;
    const int k = k0 + (kin ? kq : 0);
    const int64_t stride = (int64_t)a.M * a.K;
    const int CH = a.a_chunks;
    f4 v[G];
#pragma unroll
    for (int g = 0; g < G; ++g) v[g] = f4{0.f, 0.f, 0.f, 0.f};
    if (CH <= 8) {  // uniform over the grid
      f4 x[G][8];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int m = t / Q + g * (ST / Q);
        const float* p = a.a_part + (int64_t)(m < a.M ? m : 0) * a.K + k;
#pragma unroll
        for (int j = 0; j < 8; ++j) x[g][j] = *reinterpret_cast<const f4*>(p + min(j, CH - 1) * stride);
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < CH) v[g] += x[g][j];
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int m = t / Q + g * (ST / Q);
        const float* p = a.a_part + (int64_t)(m < a.M ? m : 0) * a.K + k;
        for (int c0 = 0; c0 < CH; c0 += 8) {
          f4 x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = *reinterpret_cast<const f4*>(p + min(c0 + j, CH - 1) * stride);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (c0 + j < CH) v[g] += x[j];
        }
      }
    }
    const f4 bias = *reinterpret_cast<const f4*>(a.a_bias + k);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int m = t / Q + g * (ST / Q);
      f4 y = v[g] + bias;
      y = f4{gelu_f(y.x), gelu_f(y.y), gelu_f(y.z), gelu_f(y.w)};
      if constexpr (RND) y = f4{round_bf16(y.x), round_bf16(y.y), round_bf16(y.z), round_bf16(y.w)};
      if (!(m < a.M && kin)) y = f4{0.f, 0.f, 0.f, 0.f};
      if constexpr (MF) {
        *reinterpret_cast<u16x4*>(&sA16[m][kq]) = u16x4{bf16_of(y.x), bf16_of(y.y), bf16_of(y.z), bf16_of(y.w)};
      } else {
        float* col = reinterpret_cast<float*>(sA) + kq * SM + m;
        col[0] = y.x, col[SM] = y.y, col[2 * SM] = y.z, col[3 * SM] = y.w;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int i = t + j * ST, m = i / SKC, kk = i % SKC;
      float v;
      if constexpr (A_BF) {
        v = bf16_val(araw[j]);
      } else {
        v = araw[j];
        if constexpr (RND) v = round_bf16(v);
      }
      put(m, kk, m < a.M && kk < kn ? v : 0.f);
    }
  }
  __syncthreads();

  if constexpr (MF) {
    // wave w takes k-steps w and w + 4 (16 k each) of the chunk, both 32-column
    // blocks of the strip; the tile's rows 16..31 are zero
    const int l32 = lane & 31, h = lane >> 5;
    const int tr_row = 8 * h + ((lane & 15) >> 2), tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    f32x16 acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int q = w + 4 * qq;
      if (q * 16 >= kn) break;  // uniform per wave: the rest of the chunk is past its end
      bf16x8 af = *reinterpret_cast<const bf16x8*>(&sA16[l32 & 15][q * 16 + 8 * h]);
      if (l32 >= SM) af = bf16x8{};
      const int k = q * 16 + tr_row;
      const char* rowk = reinterpret_cast<const char*>(sB) + k * 128 + tr_col * 2;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const char* p = rowk + ((j ^ ((k >> 1) & 1)) << 6);  // k + 4 has the same swap
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p + 4 * 128));
        const bf16x8 bfr = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr, af, acc[j], 0, 0, 0);
      }
    }
    // register e of lane l holds row l % 32, column 32 j + 8 (e / 4) + 4 h + e % 4
    if (l32 < SM) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 16; e4 += 4)
          red[w][l32 * (SNS / 4) + (32 * j + 8 * (e4 >> 2) + 4 * h) / 4] =
              f4{acc[j][e4], acc[j][e4 + 1], acc[j][e4 + 2], acc[j][e4 + 3]};
    }
  } else {
  f4 acc[SM];
#pragma unroll
  for (int m = 0; m < SM; ++m) acc[m] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < SKC / 16; ++i) {
    const int kk = 4 * w + r + 16 * i;
    if (kk < kn) {
#pragma unroll
      for (int q = 0; q < SM / 4; ++q) {
        const f4 av = sA[kk][q];
        acc[4 * q + 0] += av.x * b[i];
        acc[4 * q + 1] += av.y * b[i];
        acc[4 * q + 2] += av.z * b[i];
        acc[4 * q + 3] += av.w * b[i];
      }
    }
  }
  // quad sum over r; lane r of the quad keeps rows 4r..4r+3
#pragma unroll
  for (int m = 0; m < SM; ++m) {
    acc[m].x = quad_sum(acc[m].x);
    acc[m].y = quad_sum(acc[m].y);
    acc[m].z = quad_sum(acc[m].z);
    acc[m].w = quad_sum(acc[m].w);
  }
  // red[w][m * 16 + c] = rows m, columns 4c..4c+3
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // selects, not an indexed register array (that would live in scratch)
    const f4 x = r == 0 ? acc[j] : r == 1 ? acc[4 + j] : r == 2 ? acc[8 + j] : acc[12 + j];
    red[w][(4 * r + j) * (SNS / 4) + c] = x;
  }
  }
  __syncthreads();
  // thread t owns output f4 t: row t / 16, columns n0 + 4 (t % 16)
  f4 v = red[0][t] + red[1][t] + red[2][t] + red[3][t];
  const int m = t / (SNS / 4), nn = n0 + 4 * (t % (SNS / 4));
  if (m >= a.M || nn >= a.N) return;
  v *= a.alpha;
  if (a.chunks > 1 || a.post == POST_LN || a.post == POST_PARTIALS) {  // the reduction adds bias, beta C, resid
    *reinterpret_cast<f4*>(a.ws + ((int64_t)chunk * a.M + m) * a.N + nn) = v;
    return;
  }
  if (a.bias) v += *reinterpret_cast<const f4*>(a.bias + nn);
  if (a.post == POST_GELU) v = f4{gelu_f(v.x), gelu_f(v.y), gelu_f(v.z), gelu_f(v.w)};
  float* dst = a.C + (int64_t)m * a.ldc + nn;
  if (a.beta != 0.f) v += a.beta * *reinterpret_cast<const f4*>(dst);
  if (a.resid) v += *reinterpret_cast<const f4*>(a.resid + (int64_t)m * a.ldc + nn);
  if (!a.skipc) *reinterpret_cast<f4*>(dst) = v;
  if (a.Cbf)
    *reinterpret_cast<u16x4*>(a.Cbf + (int64_t)m * a.ldc + nn) = u16x4{bf16_of(v.x), bf16_of(v.y), bf16_of(v.z), bf16_of(v.w)};
}

// C = sum over chunks (in chunk order) of ws[chunk][M][N] + bias + beta C + resid, one
// thread per 4 outputs; the partials are loaded eight chunks at a time before they
// are added, so a thread has eight loads in flight
__global__ __launch_bounds__(ST) void gemv_reduce_k(SkArgs a) {
  const int N4 = a.N / 4;
  const int e = blockIdx.x * ST + threadIdx.x;
  if (e >= a.M * N4) return;
  const int m = e / N4, nn = 4 * (e % N4);
  const f4* p = reinterpret_cast<const f4*>(a.ws) + e;
  const int64_t stride = (int64_t)a.M * N4;
  f4 v = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < a.chunks; c0 += 8) {
    f4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = p[(int64_t)min(c0 + j, a.chunks - 1) * stride];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < a.chunks) v += x[j];
  }
  if (a.bias) v += *reinterpret_cast<const f4*>(a.bias + nn);
  if (a.post == POST_GELU) v = f4{gelu_f(v.x), gelu_f(v.y), gelu_f(v.z), gelu_f(v.w)};
  float* dst = a.C + (int64_t)m * a.ldc + nn;
  if (a.beta != 0.f) v += a.beta * *reinterpret_cast<const f4*>(dst);
  if (a.resid) v += *reinterpret_cast<const f4*>(a.resid + (int64_t)m * a.ldc + nn);
  if (!a.skipc) *reinterpret_cast<f4*>(dst) = v;
  if (a.Cbf)
    *reinterpret_cast<u16x4*>(a.Cbf + (int64_t)m * a.ldc + nn) = u16x4{bf16_of(v.x), bf16_of(v.y), bf16_of(v.z), bf16_of(v.w)};
}

// POST_LN: one workgroup per row m.  C = the sum of the chunks (in chunk order) + bias +
// beta C + resid, stored as usual; the row is then layer-normalised from registers (its
// mean, then the mean square of the centred values) and written to ln_y and/or ln_ybf.
constexpr int LN_MAXN = 2048;
constexpr int LN_PER = LN_MAXN / 4 / ST;  // float4s per thread

// the workgroup's sum: each wave's by DPP inside its 16-lane rows (the quad_sum
// steps, then the half-row and row mirrors) and the four row sums read as scalars,
// then the four waves through LDS
__device__ __forceinline__ float block_sum_ln(float v, float* sh) {
  v = quad_sum(v);
  v += dpp<0x141>(v);  // row_half_mirror: the other quad of the half-row
  v += dpp<0x140>(v);  // row_mirror: the other half of the row
  v = (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))) +
      (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48)));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < ST / 64; ++i) r += sh[i];
  return r;
}

__global__ __launch_bounds__(ST) void gemv_reduce_ln_k(SkArgs a) {
  __shared__ float red[ST / 64];
  const int m = blockIdx.x, t = threadIdx.x, N4 = a.N / 4;
  const int64_t stride = (int64_t)a.M * N4;
  const f4* p = reinterpret_cast<const f4*>(a.ws) + (int64_t)m * N4;
  f4 v[LN_PER];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < LN_PER; ++j) {
    const int e = t + j * ST;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    if (e < N4) {
      for (int c0 = 0; c0 < a.chunks; c0 += 8) {
        f4 x[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) x[q] = p[(int64_t)min(c0 + q, a.chunks - 1) * stride + e];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (c0 + q < a.chunks) acc += x[q];
      }
      const int nn = 4 * e;
      if (a.bias) acc += *reinterpret_cast<const f4*>(a.bias + nn);
      float* dst = a.C + (int64_t)m * a.ldc + nn;
      if (a.beta != 0.f) acc += a.beta * *reinterpret_cast<const f4*>(dst);
      if (a.resid) acc += *reinterpret_cast<const f4*>(a.resid + (int64_t)m * a.ldc + nn);
      if (!a.skipc) *reinterpret_cast<f4*>(dst) = acc;
      if (a.Cbf)
        *reinterpret_cast<u16x4*>(a.Cbf + (int64_t)m * a.ldc + nn) =
            u16x4{bf16_of(acc.x), bf16_of(acc.y), bf16_of(acc.z), bf16_of(acc.w)};
      s += (acc.x + acc.y) + (acc.z + acc.w);
    }
    v[j] = acc;
  }
  const float invN = 1.f / (float)a.N;
  const float mu = block_sum_ln(s, red) * invN;
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < LN_PER; ++j)
    if (t + j * ST < N4) {
      const f4 d = v[j] - mu;
      q += (d.x * d.x + d.y * d.y) + (d.z * d.z + d.w * d.w);
    }
  const float rs = rsqrtf(block_sum_ln(q, red) * invN + a.ln_eps);
#pragma unroll
  for (int j = 0; j < LN_PER; ++j) {
    const int e = t + j * ST;
    if (e >= N4) continue;
    const int nn = 4 * e;
    const f4 o = (v[j] - mu) * rs * *reinterpret_cast<const f4*>(a.ln_gamma + nn) +
                 *reinterpret_cast<const f4*>(a.ln_beta + nn);
    if (a.ln_y) *reinterpret_cast<f4*>(a.ln_y + (int64_t)m * a.N + nn) = o;
    if (a.ln_ybf)
      *reinterpret_cast<u16x4*>(a.ln_ybf + (int64_t)m * a.N + nn) = u16x4{bf16_of(o.x), bf16_of(o.y), bf16_of(o.z), bf16_of(o.w)};
  }
}

// ------------------------------------------------------------------ NT form
// C = alpha A B^T + bias + beta C with A [M <= 16, K] and B [N, K], both
// k-contiguous and B stored as bf16: the LM head of one token per sequence,
// logits = h wte^T ([GPT2-4, "Generation with KV Cache"]; the product is
// MatMulT of [Autograd-1, "Ops"]).  Each lane's MFMA fragment of B, 8
// consecutive k of one row, is then 16 contiguous bytes of memory, so B goes
// from HBM straight into registers and only A is staged, once per pass, in
// LDS.  Wave w of workgroup b owns rows 128b + 16w .. +15 of B over all of k
// and multiplies them by the 16 rows of A with v_mfma_f32_16x16x32_bf16: lane
// l brings row l % 16 of B and of A for the k slots of its lane group l / 16,
// and within a 128-deep k block a lane's share is 64 contiguous bytes (k = 32
// (l / 16) + 8q + 0..7 for its four products q); both operands list the same k
// in every slot, so the sum runs over each k once.  No partial leaves the
// wave: one launch, no reduction.
constexpr int NTB = 6;           // 128-deep k blocks held in registers per pass
constexpr int NTK = NTB * 128;   // k per pass
constexpr int NTW = 8;           // waves per workgroup (A staging then takes 12 VGPRs a lane: four waves a SIMD fit)
constexpr int NT_ROWS = 16 * NTW;  // rows of B per workgroup

struct NtArgs {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  float* C;
  int64_t ldc;
  uint16_t* Cbf;
  const float* bias;
  float alpha, beta;
  int M, N, K, skipc, vec;
};

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

// FULL: K is a multiple of the pass depth, so no k is out of range
template <bool FULL>
__global__ __launch_bounds__(64 * NTW, 2) void gemv_nt_k(NtArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[SM][NTK + 8];  // 16-byte row pad: conflict-free fragment reads
  constexpr int AU = NTK / 8 / 32;  // 16-byte units of A per thread and pass
  static_assert(64 * NTW == 32 * SM && NTK % 256 == 0, "A staging: 32 threads per row of A");
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int r = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * NT_ROWS + w * 16;
  // rows past N read the last row again; their results are never stored
  const uint16_t* brow = a.B + (int64_t)min(n0 + r, a.N - 1) * a.ldb + 32 * lg;
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int kb = 0; kb < a.K; kb += NTK) {
    // Every k block of B this pass needs, then A.  Out-of-range elements load a
    // valid one (clamped index) and are zeroed afterwards: a load under a branch
    // would be waited for on its own.  A is stored to LDS once B has arrived
    // (loads retire in order), which costs nothing: the products wait for B anyway.
    u16x8 bv[NTB][4];
#pragma unroll
    for (int p = 0; p < NTB; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = kb + 128 * p + 32 * lg + 8 * q;
        bv[p][q] = *reinterpret_cast<const u16x8*>(brow + (FULL || k < a.K ? kb + 128 * p + 8 * q : -32 * lg));
      }
    // thread t stages row t / 32 of A, 16-byte units t % 32 + 32 i of the pass
    const int am = t >> 5, ac = t & 31;
    const bool arow = am < a.M;
    u16x8 av[AU];
    bool aok[AU];
#pragma unroll
    for (int i = 0; i < AU; ++i) {
      const int k = kb + 8 * (ac + 32 * i);
      aok[i] = arow && (FULL || k < a.K);
      av[i] = *reinterpret_cast<const u16x8*>(a.A + (int64_t)(arow ? am : 0) * a.lda + (FULL || k < a.K ? k : 0));
    }
    if (kb > 0) __syncthreads();  // the previous pass's fragment reads are done
#pragma unroll
    for (int i = 0; i < AU; ++i)
      *reinterpret_cast<u16x8*>(&sA[am][8 * (ac + 32 * i)]) = aok[i] ? av[i] : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    __syncthreads();
#pragma unroll
    for (int p = 0; p < NTB; ++p) {
      if (!FULL && kb + 128 * p >= a.K) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool in = FULL || kb + 128 * p + 32 * lg + 8 * q < a.K;
        const u16x8 bz = in ? bv[p][q] : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(&sA[r][128 * p + 32 * lg + 8 * q]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bz), af, acc, 0, 0, 0);
      }
    }
  }
  // lane l holds rows 4 (l / 16) + e of this wave's 16 rows of B, for row l % 16 of A
  const int m = r, n = n0 + 4 * lg;
  if (m >= a.M || n >= a.N) return;
  f4 v = acc * a.alpha;
  float* row = a.C + (int64_t)m * a.ldc;
  if (a.vec && n + 3 < a.N) {
    if (a.bias) v += *reinterpret_cast<const f4*>(a.bias + n);
    if (a.beta != 0.f) v += a.beta * *reinterpret_cast<const f4*>(row + n);
    if (!a.skipc) *reinterpret_cast<f4*>(row + n) = v;
    if (a.Cbf)
      *reinterpret_cast<u16x4*>(a.Cbf + (int64_t)m * a.ldc + n) = u16x4{bf16_of(v.x), bf16_of(v.y), bf16_of(v.z), bf16_of(v.w)};
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (n + e >= a.N) break;
    float x = v[e];
    if (a.bias) x += a.bias[n + e];
    if (a.beta != 0.f) x += a.beta * row[n + e];
    if (!a.skipc) row[n + e] = x;
    if (a.Cbf) a.Cbf[(int64_t)m * a.ldc + n + e] = bf16_of(x);
  }
}

// the NT form's conditions: few rows, both operands stored as bf16 with rows of
// whole 16-byte units, and none of the fused epilogues
bool nt_ok(const GemmArgs& g) {
  const auto al = [](const void* q, int bytes) { return (reinterpret_cast<uintptr_t>(q) & (bytes - 1)) == 0; };
  if (!g.b_kcontig || !g.b_bf16 || !g.a_bf16) return false;
  if (g.M < 1 || g.M > SM || g.batch != 1 || g.K < 1 || g.N < 1 || g.K % 8) return false;
  if (g.post != POST_NONE || g.resid || g.a_part || g.att_acc || g.a_mcontig || g.causal_a != CAUSAL_NONE ||
      g.causal_out)
    return false;
  if (g.ldb % 8 || !al(g.B, 16) || g.lda % 8 || !al(g.A, 16)) return false;
  if (!g.C && !g.c_bf16_only) return false;
  return (int64_t)g.M * g.ldc < (1ll << 40) && (int64_t)(g.N + NT_ROWS - 1) / NT_ROWS < (1 << 24);
}

hipError_t launch_nt(const GemmArgs& g, hipStream_t s) {
  const auto al = [](const void* q, int bytes) { return (reinterpret_cast<uintptr_t>(q) & (bytes - 1)) == 0; };
  NtArgs a;
  a.A = reinterpret_cast<const uint16_t*>(g.A), a.lda = g.lda, a.B = reinterpret_cast<const uint16_t*>(g.B), a.ldb = g.ldb;
  a.C = g.C, a.ldc = g.ldc, a.Cbf = g.Cbf, a.bias = g.bias, a.alpha = g.alpha, a.beta = g.beta;
  a.M = g.M, a.N = g.N, a.K = g.K, a.skipc = g.c_bf16_only ? 1 : 0;
  a.vec = g.ldc % 4 == 0 && al(g.C, 16) && al(g.bias, 16) && al(g.Cbf, 8);
  const dim3 grid((unsigned)((g.N + NT_ROWS - 1) / NT_ROWS));
  const dim3 block(64 * NTW);
  if (g.K % NTK == 0)
    run_kernel(gemv_nt_k<true>, grid, block, 0, s, a);
  else
    run_kernel(gemv_nt_k<false>, grid, block, 0, s, a);
  return hipGetLastError();
}

struct SkPlan {
  bool ok = false;
  int kc = SKC, chunks = 1, strips = 0;
};

SkPlan plan(const GemmArgs& g) {
  SkPlan p;
  const auto al = [](const void* q, int bytes) { return (reinterpret_cast<uintptr_t>(q) & (bytes - 1)) == 0; };
  if (g.M < 1 || g.M > SM || g.batch != 1 || g.K < 1 || g.N < 1) return p;
  if (g.post == POST_GELU && (g.resid || g.beta != 0.f)) return p;
  if (g.a_part && (!g.a_bias || g.a_chunks < 1 || g.a_bf16 || g.post == POST_PARTIALS || g.K % 4 || !al(g.a_part, 16) ||
                   !al(g.a_bias, 16)))
    return p;
  if (g.att_acc && (g.a_part || !g.att_ml || g.att_blocks < 1 || g.att_hs < 1 || g.att_heads < 1 ||
                    (int64_t)g.att_hs * g.att_heads != g.K || g.a_bf16))
    return p;
  if (g.post == POST_PARTIALS && (g.bias || g.resid || g.beta != 0.f || g.Cbf)) return p;
  if (g.post == POST_LN && (g.N > LN_MAXN || !g.ln_gamma || !g.ln_beta || !al(g.ln_gamma, 16) || !al(g.ln_beta, 16) ||
                            !al(g.ln_y, 16) || !al(g.ln_ybf, 8) || (!g.ln_y && !g.ln_ybf)))
    return p;
  if ((int64_t)g.M * g.N > (1 << 28)) return p;  // keeps the launches' int indexes in range
  if (g.causal_a != CAUSAL_NONE || g.causal_out || g.a_mcontig || g.b_kcontig) return p;
  if (g.N % 4 || g.ldb % 4 || g.ldc % 4 || !al(g.B, g.b_bf16 ? 8 : 16) || !al(g.C, 16) || !al(g.bias, 16) ||
      !al(g.resid, 16) || !al(g.Cbf, 8))
    return p;
  p.strips = (g.N + SNS - 1) / SNS;
  // a few hundred workgroups: 64-row chunks when 128-row ones leave under ~200
  p.kc = (int64_t)p.strips * ((g.K + SKC - 1) / SKC) < 192 ? SKC / 2 : SKC;
  p.chunks = (g.K + p.kc - 1) / p.kc;
  if ((int64_t)p.strips * p.chunks > (1 << 24)) return p;
  p.ok = true;
  return p;
}

template <bool A_BF, bool B_BF, bool RND, int ASRC = A_MEM>
void launch(const SkArgs& a, int grid, hipStream_t s) {
  run_kernel((gemv_k<A_BF, B_BF, RND, ASRC>), dim3(grid), dim3(ST), 0, s, a);
}

}  // namespace

size_t gemv_workspace_bytes(const GemmArgs& g) {
  const SkPlan p = plan(g);
  if (!p.ok || (p.chunks == 1 && g.post != POST_LN && g.post != POST_PARTIALS)) return 0;
  return (size_t)p.chunks * g.M * g.N * sizeof(float);
}

bool gemv_accepts(const GemmArgs& g) { return plan(g).ok; }

int gemv_chunks(const GemmArgs& g) {
  const SkPlan p = plan(g);
  return p.ok ? p.chunks : 0;
}

bool gemv(const GemmArgs& g, void* ws, size_t ws_bytes, hipStream_t s, hipError_t* err) {
  if (nt_ok(g)) {
    *err = launch_nt(g, s);
    return true;
  }
  const SkPlan p = plan(g);
  if (!p.ok) return false;
  if ((p.chunks > 1 || g.post == POST_LN || g.post == POST_PARTIALS) && (!ws || ws_bytes < gemv_workspace_bytes(g)))
    return false;
  SkArgs a;
  a.A = g.A, a.lda = g.lda, a.B = g.B, a.ldb = g.ldb, a.C = g.C, a.ldc = g.ldc, a.Cbf = g.Cbf;
  a.bias = g.bias, a.resid = g.resid, a.alpha = g.alpha, a.beta = g.beta;
  a.M = g.M, a.N = g.N, a.K = g.K, a.kc = p.kc, a.chunks = p.chunks, a.skipc = g.c_bf16_only ? 1 : 0;
  a.ws = static_cast<float*>(ws);
  a.post = g.post, a.ln_gamma = g.ln_gamma, a.ln_beta = g.ln_beta, a.ln_eps = g.ln_eps, a.ln_y = g.ln_y;
  a.ln_ybf = g.ln_ybf;
  a.a_part = g.a_part, a.a_bias = g.a_bias, a.a_chunks = g.a_chunks;
  a.att_acc = g.att_acc, a.att_ml = g.att_ml, a.att_blocks = g.att_blocks, a.att_hs = g.att_hs;
  a.att_heads = g.att_heads;
  const int grid = p.strips * p.chunks;
  const bool rnd = g.prec == PREC_BF16;
  if (g.a_part) {
    if (g.b_bf16)
      rnd ? launch<false, true, true, A_PARTS>(a, grid, s) : launch<false, true, false, A_PARTS>(a, grid, s);
    else
      rnd ? launch<false, false, true, A_PARTS>(a, grid, s) : launch<false, false, false, A_PARTS>(a, grid, s);
  } else if (g.att_acc) {
    if (g.b_bf16)
      rnd ? launch<false, true, true, A_ATTN>(a, grid, s) : launch<false, true, false, A_ATTN>(a, grid, s);
    else
      rnd ? launch<false, false, true, A_ATTN>(a, grid, s) : launch<false, false, false, A_ATTN>(a, grid, s);
  } else if (g.a_bf16 && g.b_bf16)
    launch<true, true, false>(a, grid, s);
  else if (g.a_bf16)
    rnd ? launch<true, false, true>(a, grid, s) : launch<true, false, false>(a, grid, s);
  else if (g.b_bf16)
    rnd ? launch<false, true, true>(a, grid, s) : launch<false, true, false>(a, grid, s);
  else
    rnd ? launch<false, false, true>(a, grid, s) : launch<false, false, false>(a, grid, s);
  if (g.post == POST_LN) {
    run_kernel(gemv_reduce_ln_k, dim3(g.M), dim3(ST), 0, s, a);
  } else if (p.chunks > 1 && g.post != POST_PARTIALS) {
    const int n4 = g.M * (g.N / 4);
    run_kernel(gemv_reduce_k, dim3((n4 + ST - 1) / ST), dim3(ST), 0, s, a);
  }
  *err = hipGetLastError();
  return true;
}

}  // namespace tfb
