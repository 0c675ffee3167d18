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
#include "lanes.h"

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
constexpr float RESCALE_MARGIN = 8.f;  // the forward's running reference may trail the max by this (log2 units)

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x by the hardware instruction; arguments here are <= 0 (or -inf), so the
// only difference from exp2f is that results below 2^-126 flush to zero
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ unsigned short f2bf(float x) { return __builtin_bit_cast(unsigned short, (__bf16)x); }

__device__ __forceinline__ bf16x8 as_bf(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 consecutive accumulators (a 16-key slice of a 32x32 block) packed as a bf16 B operand
__device__ __forceinline__ bf16x8 pack8(const f32x16& acc, int base) {
  u16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = f2bf(acc[base + e]);
  return as_bf(v);
}

__device__ __forceinline__ u16x4 pack4(f4 v) { return u16x4{f2bf(v[0]), f2bf(v[1]), f2bf(v[2]), f2bf(v[3])}; }
__device__ __forceinline__ f4 bf4(u16x4 v) {  // exact float values of 4 bf16 numbers
  return f4{__uint_as_float((unsigned)v[0] << 16), __uint_as_float((unsigned)v[1] << 16),
            __uint_as_float((unsigned)v[2] << 16), __uint_as_float((unsigned)v[3] << 16)};
}

// row index (within a 32x32 block) held by accumulator r of lane half h
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }
// the part of it that depends on r alone (a constant after unrolling)
__device__ __forceinline__ constexpr int acc_row0(int r) { return 8 * (r >> 2) + (r & 3); }

// --- staging ------------------------------------------------------------------------------
// A KVB x HS block of rows (keys or queries) goes global -> registers -> LDS as
// X[row][HS + 8], one 16-byte chunk of 8 values per transfer; rows past
// `valid` are zero.  The register step lets the next block be fetched while
// the current one is multiplied.
template <int HS, int NTH = NT>
struct RowStage {
  static constexpr int CPR = HS / 8, CHUNKS = KVB * CPR, PER = (CHUNKS + NTH - 1) / NTH;
  u16x8 v[PER];
  // Buffer loads over the first `valid` rows of src (valid * ld * 2 < 2^31 bytes):
  // the hardware's range check returns zeros for rows past them, and the
  // per-thread offsets are loop-invariant, so a load costs one add.
  __device__ __forceinline__ void load(const unsigned short* __restrict__ src, int64_t ld, int row0, int valid,
                                       int tid) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, valid * (int)ld * 2, 0x00020000);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NTH;
      if (CHUNKS % NTH != 0 && c >= CHUNKS) break;
      const int row = c / CPR, col = (c % CPR) * 8;
      v[i] = __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, ((row0 + row) * (int)ld + col) * 2, 0, 0));
    }
  }
  __device__ __forceinline__ void store(unsigned short* dst, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NTH;
      if (CHUNKS % NTH != 0 && c >= CHUNKS) break;
      *reinterpret_cast<u16x8*>(dst + (c / CPR) * (HS + 8) + (c % CPR) * 8) = v[i];
    }
  }
};

// A fragment of X^T (rows d = d0 + lane%32, k = rows of X in the packed-register
// order 16s + 4h + {0..3}, 16s + 8 + 4h + {0..3}) from the row-major tile X[row][HS + 8],
// by two transposing LDS reads.  ds_read_b64_tr_b16 hands lane j of a 16-lane
// group element e of the 8 bytes addressed by lane 4e + j/4, at position j%4:
// lane i of group g therefore points at row 16s + 4(g/2) + i/4 (+8 for the
// second read), columns d0 + 16(g%2) + 4(i%4), and receives column d0 + 16(g%2) + i.
template <int HS>
__device__ __forceinline__ bf16x8 frag_tr(const unsigned short* X, int d0, int s, int lane) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const int g = lane >> 4, i = lane & 15;
  const unsigned short* p = X + (16 * s + 4 * (g >> 1) + (i >> 2)) * (HS + 8) + d0 + 16 * (g & 1) + 4 * (i & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p + 8 * (HS + 8)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Work assignment.  The grid is 1-D over nx blocks x (B*H rounded up to 8).
// Workgroup w runs on XCD w % 8, and causal work grows (forward, dQ) or shrinks
// (dK/dV) with the block index, so each XCD takes a fixed eighth of the heads
// and walks them block-index-major, largest blocks first: every XCD gets the
// same mix, and the short blocks fill in behind the long ones.
struct BlockId {
  int x, bh;
};
__device__ __forceinline__ BlockId block_id(int nx, bool large_x_first) {
  const int L = blockIdx.x, local = L >> 3;
  const int heads_per_xcd = (int)(gridDim.x >> 3) / nx;
  const int rank = local / heads_per_xcd;
  BlockId r;
  r.bh = (L & 7) + 8 * (local % heads_per_xcd);
  r.x = large_x_first ? nx - 1 - rank : rank;
  return r;
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
  const unsigned short* ybf;  // bf16 copy of y (backward: D from dy and ybf when y or dyf is null)
  float* out;                 // forward: y; backward: dqkv fp32 [B, T, 3C]
  unsigned short* outbf;      // optional bf16 copy of `out` (same layout)
  float* lse;                 // [B*H, T] base-2 log-sum-exp of the scaled scores
  float* D;                   // [B*H, T]
  int B, T, H, C;
  float scale;
  float beta;                 // backward: 0 overwrite dqkv, 1 add
};

// ------------------------------------------------------------------------------------ forward
// A workgroup of 4 waves owns 64 queries.  Waves w and w + 2 hold the same 32
// queries and take alternate 64-key blocks (even blocks: waves 0-1, odd: 2-3), so
// each wave's chain of dependent blocks is half as long as the query block's; the
// two partial results (output, running sum, reference) are merged through LDS.
constexpr int FQ = 64;  // queries per forward workgroup
template <int HS>
__global__ __launch_bounds__(NT, 3) void attn_fwd_k(AttnArgs a) {
  constexpr int XS = KVB * (HS + 8), HT = NT / 2;
  // [K half 0 | K half 1 | V half 0 | V half 1]; after the loop: the merge area
  __shared__ __attribute__((aligned(16))) unsigned short S[4 * XS];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform by construction
  const int w = wv & 1, half = wv >> 1, htid = tid & (HT - 1);
  unsigned short* Kh = S + half * XS;
  unsigned short* Vh = S + (2 + half) * XS;
  const BlockId id = block_id((a.T + FQ - 1) / FQ, true);
  if (id.bh >= a.B * a.H) return;
  const int bh = id.bh, b = bh / a.H, hd = bh % a.H;
  const int q0 = id.x * FQ, qw = q0 + 32 * w, q = qw + l32;
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

  const int kv_end = min(a.T, q0 + FQ);
  // each half stages its own block: one LDS buffer, the next block waits in registers
  const int nit = (kv_end + 2 * KVB - 1) / (2 * KVB);
  RowStage<HS, HT> kst, vst;
  kst.load(Kg, ld, half * KVB, a.T, htid);
  vst.load(Vg, ld, half * KVB, a.T, htid);
  for (int j = 0; j < nit; ++j) {
    const int kv0 = (2 * j + half) * KVB;
    kst.store(Kh, htid);
    vst.store(Vh, htid);
    __syncthreads();
    if (j + 1 < nit) {
      kst.load(Kg, ld, kv0 + 2 * KVB, a.T, htid);
      vst.load(Vg, ld, kv0 + 2 * KVB, a.T, htid);
    }
    // else every key of this block is after every query of this wave (or past the end)
    if (kv0 < kv_end && kv0 <= qw + 31) {
      f32x16 st[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kt][r] = 0.f;
#pragma unroll
        for (int s = 0; s < HS / 16; ++s) st[kt] = mfma(frag_r<HS>(Kh, 32 * kt + l32, s, h), qf[s], st[kt]);
      }
      // every key of the block visible to every query of the wave: no mask.  Other
      // blocks set the scores of hidden keys to -inf; the empty asm keeps that a
      // real (wave-uniform) branch instead of selects that every block would run.
      const bool full = kv0 + KVB - 1 <= qw && kv0 + KVB <= a.T;
      if (!full) {
        asm volatile("");
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int lim = min(q, a.T - 1) - kv0 - 32 * kt - 4 * h;  // key visible: acc_row0(r) <= lim
#pragma unroll
          for (int r = 0; r < 16; ++r) st[kt][r] = acc_row0(r) <= lim ? st[kt][r] : -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kt][r]);
      mx *= sc;
      mx = lanes_xor32_max(mx);
      // m is the reference the running sum l and the output o are scaled to.  It
      // only moves when a score exceeds it by more than RESCALE_MARGIN (log2
      // units), so p <= 2^RESCALE_MARGIN; o / l and m + log2(l) are unchanged by
      // the choice of reference.  After the first visible block a wave almost
      // never has to rescale, and the test is one wave-uniform branch.
      const bool need = mx > m + RESCALE_MARGIN;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float mn = need ? mx : m;
        const float alpha = need ? fexp2(m - mn) : 1.f;  // m = -inf: alpha = 0, o and l are 0
        l *= alpha;
#pragma unroll
        for (int i = 0; i < HS / 32; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[i][r] *= alpha;
        m = mn;
      }
      const float mref = m == -INFINITY ? 0.f : m;
      float sum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fexp2(fmaf(st[kt][r], sc, -mref));  // -inf (masked) -> 0
          st[kt][r] = p;
          sum += p;
        }
      sum = lanes_xor32_add(sum);
      l += sum;
#pragma unroll
      for (int s = 0; s < KVB / 16; ++s) {
        const bf16x8 pb = pack8(st[s >> 1], 8 * (s & 1));
#pragma unroll
        for (int i = 0; i < HS / 32; ++i) o[i] = mfma(frag_tr<HS>(Vh, 32 * i, s, lane), pb, o[i]);
      }
    }
    __syncthreads();
  }
  // merge: waves 2-3 leave output, reference and sum in LDS (lane-major, so the
  // accesses are conflict-free); waves 0-1 rescale both parts to the larger reference
  constexpr int NR = HS / 32 * 16;
  float* Pm = reinterpret_cast<float*>(S);
  const int slot = w * 64 + lane;
  if (half == 1) {
#pragma unroll
    for (int i = 0; i < HS / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) Pm[(i * 16 + r) * HT + slot] = o[i][r];
    Pm[NR * HT + slot] = m;
    Pm[(NR + 1) * HT + slot] = l;
  }
  __syncthreads();
  if (half == 1) return;
  {
    const float m1 = Pm[NR * HT + slot], l1 = Pm[(NR + 1) * HT + slot];
    const float mn = fmaxf(m, m1);
    const float mref = mn == -INFINITY ? 0.f : mn;
    const float a0 = fexp2(m - mref), a1 = fexp2(m1 - mref);  // a part that saw no key: 0
    l = l * a0 + l1 * a1;
#pragma unroll
    for (int i = 0; i < HS / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] = o[i][r] * a0 + Pm[(i * 16 + r) * HT + slot] * a1;
    m = mn;
  }
  if (q < a.T) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t off = ((int64_t)b * a.T + q) * a.C + hd * HS;
#pragma unroll
    for (int i = 0; i < HS / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {  // registers r .. r+3 hold 4 consecutive columns of this query's row
        const f4 v = f4{o[i][r], o[i][r + 1], o[i][r + 2], o[i][r + 3]} * inv;
        const int d = 32 * i + acc_row(r, h);
        if (a.out) *reinterpret_cast<f4*>(a.out + off + d) = v;  // null: the bf16 copy alone
        if (a.outbf) *reinterpret_cast<u16x4*>(a.outbf + off + d) = pack4(v);
      }
    if (h == 0) a.lse[(int64_t)bh * a.T + q] = m + log2f(l);
  }
}

// ------------------------------------------------------------------------------------ backward
// dQ for a block of 128 queries (4 waves x 32), looping over key blocks
template <int HS>
__global__ __launch_bounds__(NT, 2) void attn_dq_k(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned short Ks[2][KVB * (HS + 8)];
  __shared__ __attribute__((aligned(16))) unsigned short Vs[2][KVB * (HS + 8)];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform by construction
  const BlockId id = block_id((a.T + 127) / 128, true);
  if (id.bh >= a.B * a.H) return;
  const int bh = id.bh, b = bh / a.H, hd = bh % a.H;
  const int q0 = id.x * 128, qw = q0 + 32 * w, q = qw + l32;
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
  // D = rowsum(dO * O) of this query: each lane half sums half the head's columns,
  // one exchange adds the halves; it is stored for the dK/dV kernel that follows.
  // From the fp32 values where both exist, else from the bf16 copies of both.
  float Dq = 0.f;
  if (q < a.T) {
    const int64_t off = ((int64_t)b * a.T + q) * a.C + hd * HS + h * (HS / 2);
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    if (a.y && a.dyf) {
      const f4* g4 = reinterpret_cast<const f4*>(a.dyf + off);
      const f4* y4 = reinterpret_cast<const f4*>(a.y + off);
#pragma unroll
      for (int j = 0; j < HS / 8; ++j) acc += g4[j] * y4[j];
    } else {
      const u16x4* g4 = reinterpret_cast<const u16x4*>(a.dy + off);
      const u16x4* y4 = reinterpret_cast<const u16x4*>(a.ybf + off);
#pragma unroll
      for (int j = 0; j < HS / 8; ++j) acc += bf4(g4[j]) * bf4(y4[j]);
    }
    Dq = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
  Dq = lanes_xor32_add(Dq);
  if (h == 0 && q < a.T) a.D[(int64_t)bh * a.T + q] = Dq;
  const float sc = a.scale * LOG2E;

  f32x16 dq[HS / 32];
#pragma unroll
  for (int i = 0; i < HS / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[i][r] = 0.f;

  const int kv_end = min(a.T, q0 + 128);
  RowStage<HS> kst, vst;
  kst.load(Kg, ld, 0, a.T, tid);
  vst.load(Vg, ld, 0, a.T, tid);
  kst.store(Ks[0], tid);
  vst.store(Vs[0], tid);
  __syncthreads();
  int buf = 0;
  for (int kv0 = 0; kv0 < kv_end; kv0 += KVB) {
    const bool more = kv0 + KVB < kv_end;
    if (more) {
      kst.load(Kg, ld, kv0 + KVB, a.T, tid);
      vst.load(Vg, ld, kv0 + KVB, a.T, tid);
    }
    if (kv0 <= qw + 31) {
      f32x16 st[2], dp[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kt][r] = dp[kt][r] = 0.f;
#pragma unroll
        for (int s = 0; s < HS / 16; ++s) {
          st[kt] = mfma(frag_r<HS>(Ks[buf], 32 * kt + l32, s, h), qf[s], st[kt]);
          dp[kt] = mfma(frag_r<HS>(Vs[buf], 32 * kt + l32, s, h), df[s], dp[kt]);
        }
      }
      // dS^T = P^T (dP^T - D); a block every query of the wave sees whole needs no
      // mask.  The test is wave-uniform: one scalar branch per block, then a
      // straight loop either way.
      // Hidden keys get score -inf (so p = 0) in a real branch, as in the forward
      const bool full = kv0 + KVB - 1 <= qw && kv0 + KVB <= a.T;
      if (!full) {
        asm volatile("");
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int lim = min(q, a.T - 1) - kv0 - 32 * kt - 4 * h;
#pragma unroll
          for (int r = 0; r < 16; ++r) st[kt][r] = acc_row0(r) <= lim ? st[kt][r] : -INFINITY;
        }
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kt][r] = fexp2(fmaf(st[kt][r], sc, -lse)) * (dp[kt][r] - Dq);
#pragma unroll
      for (int s = 0; s < KVB / 16; ++s) {
        const bf16x8 sb = pack8(st[s >> 1], 8 * (s & 1));
#pragma unroll
        for (int i = 0; i < HS / 32; ++i) dq[i] = mfma(frag_tr<HS>(Ks[buf], 32 * i, s, lane), sb, dq[i]);
      }
    }
    if (more) {
      kst.store(Ks[buf ^ 1], tid);
      vst.store(Vs[buf ^ 1], tid);
    }
    __syncthreads();
    buf ^= 1;
  }
  if (q < a.T) {
    const int64_t off = ((int64_t)b * a.T + q) * ld + hd * HS;
#pragma unroll
    for (int i = 0; i < HS / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const int d = 32 * i + acc_row(r, h);
        f4 v = f4{dq[i][r], dq[i][r + 1], dq[i][r + 2], dq[i][r + 3]} * a.scale;
        if (a.out) {  // null: the bf16 copy alone
          f4* p = reinterpret_cast<f4*>(a.out + off + d);
          if (a.beta != 0.f) v += *p;
          *p = v;
        }
        if (a.outbf) *reinterpret_cast<u16x4*>(a.outbf + off + d) = pack4(v);
      }
  }
}

// dK and dV for a block of 128 keys (4 waves x 32), looping over query blocks
template <int HS>
__global__ __launch_bounds__(NT, 2) void attn_dkv_k(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned short Qs[2][KVB * (HS + 8)];
  __shared__ __attribute__((aligned(16))) unsigned short Ds[2][KVB * (HS + 8)];
  __shared__ __attribute__((aligned(16))) float Ls[2][KVB];
  __shared__ __attribute__((aligned(16))) float Dd[2][KVB];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform by construction
  const BlockId id = block_id((a.T + 127) / 128, false);
  if (id.bh >= a.B * a.H) return;
  const int bh = id.bh, b = bh / a.H, hd = bh % a.H;
  const int k0 = id.x * 128, kw = k0 + 32 * w, key = kw + l32;
  const int64_t ld = 3LL * a.C;
  const unsigned short* base = a.qkv + (int64_t)b * a.T * ld + hd * HS;
  const unsigned short* dyg = a.dy + (int64_t)b * a.T * a.C + hd * HS;
  const float* lse_g = a.lse + (int64_t)bh * a.T;
  const float* D_g = a.D + (int64_t)bh * a.T;

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

  const int qstart = (k0 / KVB) * KVB;
  RowStage<HS> qst, dst_;
  float lnext = 0.f, dnext = 0.f;
  auto fetch = [&](int qb) {
    qst.load(base, ld, qb, a.T, tid);
    dst_.load(dyg, a.C, qb, a.T, tid);
    if (tid < KVB) {
      const int qq = qb + tid;
      lnext = qq < a.T ? lse_g[qq] : 0.f;
      dnext = qq < a.T ? D_g[qq] : 0.f;
    }
  };
  auto put = [&](int bf) {
    qst.store(Qs[bf], tid);
    dst_.store(Ds[bf], tid);
    if (tid < KVB) {
      Ls[bf][tid] = lnext;
      Dd[bf][tid] = dnext;
    }
  };
  if (qstart < a.T) {
    fetch(qstart);
    put(0);
  }
  __syncthreads();
  int buf = 0;
  for (int qb = qstart; qb < a.T; qb += KVB) {
    const bool more = qb + KVB < a.T;
    if (more) fetch(qb + KVB);
    if (qb + KVB - 1 >= kw) {  // else every query of this block precedes every key of this wave
      f32x16 st[2], dp[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) st[qt][r] = dp[qt][r] = 0.f;
#pragma unroll
        for (int s = 0; s < HS / 16; ++s) {
          st[qt] = mfma(frag_r<HS>(Qs[buf], 32 * qt + l32, s, h), kf[s], st[qt]);
          dp[qt] = mfma(frag_r<HS>(Ds[buf], 32 * qt + l32, s, h), vf[s], dp[qt]);
        }
      }
      // P and dS with queries in registers, this lane's key in the column; the
      // saved statistics of 4 consecutive query rows come in one 16-byte read.
      // A block whose every query sees every key of the wave needs no mask.
      // The test is wave-uniform: one scalar branch per block, then a straight
      // loop.  Each 32-query half is finished (P, dS, and its dV / dK products)
      // before the next, so only one half's fp32 P and dS are live at a time.
      const bool full = qb >= kw + 31 && qb + KVB <= a.T && kw + 32 <= a.T;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        if (full) {
#pragma unroll
          for (int r4 = 0; r4 < 16; r4 += 4) {
            const int qi0 = 32 * qt + acc_row(r4, h);
            const f4 L4 = *reinterpret_cast<const f4*>(&Ls[buf][qi0]);
            const f4 D4 = *reinterpret_cast<const f4*>(&Dd[buf][qi0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = r4 + e;
              const float p = fexp2(fmaf(st[qt][r], sc, -L4[e]));
              st[qt][r] = p;
              dp[qt][r] = p * (dp[qt][r] - D4[e]);
            }
          }
        } else {
#pragma unroll
          for (int r4 = 0; r4 < 16; r4 += 4) {
            const int qi0 = 32 * qt + acc_row(r4, h);
            const f4 L4 = *reinterpret_cast<const f4*>(&Ls[buf][qi0]);
            const f4 D4 = *reinterpret_cast<const f4*>(&Dd[buf][qi0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = r4 + e, qq = qb + qi0 + e;
              const bool vis = key <= qq && qq < a.T && key < a.T;
              const float p = vis ? fexp2(fmaf(st[qt][r], sc, -L4[e])) : 0.f;
              st[qt][r] = p;
              dp[qt][r] = p * (dp[qt][r] - D4[e]);
            }
          }
        }
#pragma unroll
        for (int s = 2 * qt; s < 2 * qt + 2; ++s) {
          const bf16x8 pb = pack8(st[qt], 8 * (s & 1));
          const bf16x8 db = pack8(dp[qt], 8 * (s & 1));
#pragma unroll
          for (int i = 0; i < HS / 32; ++i) {
            dv[i] = mfma(frag_tr<HS>(Ds[buf], 32 * i, s, lane), pb, dv[i]);
            dk[i] = mfma(frag_tr<HS>(Qs[buf], 32 * i, s, lane), db, dk[i]);
          }
        }
      }
    }
    if (more) put(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  if (key < a.T) {
    const int64_t off = ((int64_t)b * a.T + key) * ld + hd * HS;
#pragma unroll
    for (int i = 0; i < HS / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        const int d = 32 * i + acc_row(r, h);
        f4 vk = f4{dk[i][r], dk[i][r + 1], dk[i][r + 2], dk[i][r + 3]} * a.scale;
        f4 vv = f4{dv[i][r], dv[i][r + 1], dv[i][r + 2], dv[i][r + 3]};
        if (a.out) {  // null: the bf16 copy alone
          f4* pk = reinterpret_cast<f4*>(a.out + off + a.C + d);
          f4* pv = reinterpret_cast<f4*>(a.out + off + 2 * a.C + d);
          if (a.beta != 0.f) {
            vk += *pk;
            vv += *pv;
          }
          *pk = vk;
          *pv = vv;
        }
        if (a.outbf) {
          *reinterpret_cast<u16x4*>(a.outbf + off + a.C + d) = pack4(vk);
          *reinterpret_cast<u16x4*>(a.outbf + off + 2 * a.C + d) = pack4(vv);
        }
      }
  }
}

// 1-D grid for block_id: (T/128 blocks) x (B*H rounded up to a multiple of 8)
unsigned attn_grid(int T, int BH) { return (unsigned)(((T + 127) / 128) * ((BH + 7) / 8 * 8)); }

}  // namespace

// the staging's buffer offsets are 32-bit: one batch entry's rows must span < 2 GB
static bool offsets_fit(int64_t T, int64_t C) { return (T + 2 * KVB) * 3 * C * 2 < (1LL << 31); }

bool flash_attention_supported(int hs, int64_t C, int64_t T) {
  return (hs == 64 || hs == 32) && C % 8 == 0 && offsets_fit(T, C);
}

hipError_t flash_attention_fwd(const uint16_t* qkv, float* y, uint16_t* ybf, float* lse, int B, int T, int H, int C,
                               float scale, hipStream_t s) {
  if (B <= 0 || T <= 0) return hipSuccess;
  if (!offsets_fit(T, C)) return hipErrorInvalidValue;
  if (!y && !ybf) return hipErrorInvalidValue;
  AttnArgs a{};
  a.qkv = qkv, a.out = y, a.outbf = ybf, a.lse = lse, a.B = B, a.T = T, a.H = H, a.C = C, a.scale = scale;
  const dim3 fgrid((unsigned)(((T + FQ - 1) / FQ) * ((B * H + 7) / 8 * 8)));
  const int hs = C / H;
  if (hs == 64)
    run_kernel(attn_fwd_k<64>, fgrid, dim3(NT), 0, s, a);
  else if (hs == 32)
    run_kernel(attn_fwd_k<32>, fgrid, dim3(NT), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t flash_attention_bwd(const uint16_t* qkv, const float* y, const float* dyf, const uint16_t* dy,
                               const float* lse, float* D, float* dqkv, uint16_t* dqkv_bf, float beta, int B, int T,
                               int H, int C, float scale, hipStream_t s, const uint16_t* ybf) {
  if (B <= 0 || T <= 0) return hipSuccess;
  if (!offsets_fit(T, C)) return hipErrorInvalidValue;
  if (!dqkv && (!dqkv_bf || beta != 0.f)) return hipErrorInvalidValue;
  if ((!y || !dyf) && !ybf) return hipErrorInvalidValue;
  AttnArgs a{};
  a.qkv = qkv, a.y = y, a.dyf = dyf, a.dy = dy, a.ybf = ybf, a.lse = const_cast<float*>(lse), a.D = D, a.out = dqkv;
  a.outbf = dqkv_bf;
  a.B = B, a.T = T, a.H = H, a.C = C, a.scale = scale, a.beta = beta;
  const int hs = C / H;
  dim3 grid(attn_grid(T, B * H));
  if (hs == 64) {
    run_kernel(attn_dq_k<64>, grid, dim3(NT), 0, s, a);
    run_kernel(attn_dkv_k<64>, grid, dim3(NT), 0, s, a);
  } else if (hs == 32) {
    run_kernel(attn_dq_k<32>, grid, dim3(NT), 0, s, a);
    run_kernel(attn_dkv_k<32>, grid, dim3(NT), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tfb
