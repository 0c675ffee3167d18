// MFMA contraction kernels for gfx950: the MatMul family and the attention
// products ([Autograd-1, "Ops": MatMul with dx = g w^T and dw = x^T g; the
// table of ops: MatMulT, BatchMatMul, BatchMatMulT]).
//
// One kernel template covers every layout the autograd rules need:
//   NN  A(m,k) k-contiguous, B(k,n) n-contiguous   (forward x @ w, dx of MatMulT)
//   NT  A k-contiguous,      B(k,n) k-contiguous   (x @ w^T, dx = g @ w^T, q k^T)
//   TN  A(m,k) m-contiguous, B n-contiguous        (dw = x^T @ g, P^T @ dO)
// A workgroup of WM x WN wavefronts computes a BM x BN tile of C; each wave owns
// TM x TN blocks of 32x32 accumulated by v_mfma_f32_32x32x16_bf16 (bf16
// operands) or v_mfma_f32_32x32x2_f32 (fp32 operands), fp32 accumulation.
// A k-contiguous operand is staged through LDS as [row][k] (16-byte padded rows
// for 64-deep k-tiles, XOR-swizzled 16-byte chunks for 32-deep ones), so a lane
// reads its MFMA fragment with one 16-byte LDS load.  An m- or n-contiguous
// operand stored as bf16 keeps its own [k][row] layout in LDS and its fragments
// are gathered by the transposing LDS read (ds_read_b64_tr_b16); in fp32
// storage it is transposed in small register blocks on the way in.  Every
// layout is free of bank conflicts on gfx950's 64 four-byte LDS banks.
// Operands may be stored as fp32 (rounded to bf16, nearest even, while staging
// in the bf16 variant) or already as bf16.  The next k-tile is fetched into
// registers while the current one is multiplied (two LDS buffers, one barrier
// per k-tile).
//
// Work items (output tiles of every batch entry and K split) are renumbered so
// that each of the 8 XCDs (dispatched round-robin) gets one contiguous range,
// walked in groups of GEMM_GROUP_M tile rows: the workgroups an XCD holds at
// once share A row panels and B column panels through its L2.
#include <algorithm>
#include <type_traits>

#include "kernels.h"

namespace tfb {
namespace {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

constexpr int KALIGN = 64;  // split-K chunks are multiples of this (and of every k-tile depth)
#ifndef GEMM_BIG_TILES
#define GEMM_BIG_TILES 4096  // products with at least this many 256x128 tiles use them (vocabulary-sized)
#endif
#ifndef GEMM_PIPE
#define GEMM_PIPE 1
#endif
#ifndef GEMM_DMA_TILES
#define GEMM_DMA_TILES 512   // products with at least this many 256x256 tiles take gemm_dma_kernel
#endif
#ifndef GEMM_DMA_SPLIT_K
#define GEMM_DMA_SPLIT_K 4096        // fewer tiles, but K at least this: the same kernel split over K, for ...
#endif
#ifndef GEMM_DMA_SPLIT_K_ANY
#define GEMM_DMA_SPLIT_K_ANY 16384   // ... weight gradients (A m-contiguous), or any layout with K at least this
#endif
#ifndef GEMM_DMA128_DW
#define GEMM_DMA128_DW 1  // weight gradients split over K on 128x128 tiles (two workgroups per CU)
#endif
#ifndef GEMM_GROUP_M
#define GEMM_GROUP_M 8       // tile rows per raster group
#endif
#ifndef GEMM_GROUP_WIDE
#define GEMM_GROUP_WIDE 2    // the same for products a few dozen tiles wide
#endif
#ifndef GEMM_GROUP_TALL
#define GEMM_GROUP_TALL 16   // the same for tall, narrow products
#endif

template <bool BF16, int BK>
struct Lds;
template <int BK>
struct Lds<true, BK> {
  using T = bf16_t;
  // 64-deep rows are padded by 16 bytes (a 16-lane fragment read then walks
  // all 64 banks); 32-deep rows are unpadded with chunk c of row r stored at
  // chunk c ^ ((r >> 2) & 3), which keeps both the 16-row fragment reads and
  // the 4-rows-at-a-time staging stores on distinct banks
  static constexpr bool SWZ = BK == 32;
  static constexpr int LDK = SWZ ? BK : BK + 8;
  // element offset of (row r, k) for k a multiple of 4
  __device__ __forceinline__ static int off(int r, int k) {
    return SWZ ? r * LDK + ((((k >> 3) ^ ((r >> 2) & 3)) << 3) | (k & 7)) : r * LDK + k;
  }
};
template <int BK>
struct Lds<false, BK> {
  using T = float;
  static constexpr int LDK = BK + 4;
  __device__ __forceinline__ static int off(int r, int k) { return r * LDK + k; }
};

__device__ __forceinline__ float mask_causal(float v, int causal, int m, int k) {
  if (causal == CAUSAL_UPTO && k > m) return 0.f;
  if (causal == CAUSAL_FROM && k < m) return 0.f;
  return v;
}

__device__ __forceinline__ float bf16_bits_to_f32(unsigned short b) { return __uint_as_float((unsigned)b << 16); }
__device__ __forceinline__ unsigned short bf16_bits(float x) { return __builtin_bit_cast(unsigned short, (bf16_t)x); }
__device__ __forceinline__ u16x4 bf16x4_bits(f4 v) {
  return u16x4{bf16_bits(v[0]), bf16_bits(v[1]), bf16_bits(v[2]), bf16_bits(v[3])};
}

// One thread's share of an R_TILE x BK operand tile held in registers.
//   SRC_BF16 = false: fp32 source; k-contiguous units are 4 k of one row,
//                     r-contiguous units are 4 rows x 4 k (four 16-byte loads)
//   SRC_BF16 = true:  bf16 source; k-contiguous units are 8 k of one row (16 B),
//                     r-contiguous units are 4 rows x 8 k (eight 8-byte loads)
template <int R_TILE, int NT, bool RCONTIG, bool SRC_BF16, int BK>
struct Stage {
  static constexpr int UK = SRC_BF16 ? 8 : 4;   // k per unit
  static constexpr int UR = RCONTIG ? 4 : 1;    // rows per unit
  static constexpr int UNITS = R_TILE * BK / (UK * UR);
  static constexpr int PER = (UNITS + NT - 1) / NT;
  // fp32: f4 per (unit, k-row of the block); bf16: raw 16-bit lanes
  static constexpr int REGS = SRC_BF16 ? (RCONTIG ? PER * 8 : PER) : (RCONTIG ? PER * 4 : PER);
  using R = typename std::conditional<SRC_BF16, typename std::conditional<RCONTIG, u16x4, u16x8>::type, f4>::type;
  R r[REGS];

  __device__ __forceinline__ void load(const void* __restrict__ Pv, int64_t ld, int r0, int k0, int R_, int K,
                                       bool vec, int causal, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = tid + i * NT;
      if (UNITS % NT != 0 && u >= UNITS) break;
      if constexpr (!RCONTIG) {
        const int rr = u / (BK / UK), kq = u % (BK / UK);
        const int gr = r0 + rr, gk = k0 + kq * UK;
        if constexpr (!SRC_BF16) {
          const float* P = static_cast<const float*>(Pv);
          f4 v = {0.f, 0.f, 0.f, 0.f};
          if (gr < R_) {
            const float* src = P + (int64_t)gr * ld + gk;
            if (vec && gk + 3 < K) {
              v = *reinterpret_cast<const f4*>(src);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = (gk + e < K) ? src[e] : 0.f;
            }
            if (causal != CAUSAL_NONE) {
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = mask_causal(v[e], causal, gr, gk + e);
            }
          }
          r[i] = v;
        } else {
          const unsigned short* P = static_cast<const unsigned short*>(Pv);
          u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
          if (gr < R_) {
            const unsigned short* src = P + (int64_t)gr * ld + gk;
            if (vec && gk + 7 < K) {
              v = *reinterpret_cast<const u16x8*>(src);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] = (gk + e < K) ? src[e] : (unsigned short)0;
            }
            if (causal != CAUSAL_NONE) {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if ((causal == CAUSAL_UPTO && gk + e > gr) || (causal == CAUSAL_FROM && gk + e < gr)) v[e] = 0;
            }
          }
          r[i] = v;
        }
      } else {
        const int rq = u % (R_TILE / 4), kq = u / (R_TILE / 4);
        const int gr = r0 + rq * 4;
#pragma unroll
        for (int kk = 0; kk < UK; ++kk) {
          const int gk = k0 + kq * UK + kk;
          if constexpr (!SRC_BF16) {
            const float* P = static_cast<const float*>(Pv);
            f4 v = {0.f, 0.f, 0.f, 0.f};
            if (gk < K) {
              const float* src = P + (int64_t)gk * ld + gr;
              if (vec && gr + 3 < R_) {
                v = *reinterpret_cast<const f4*>(src);
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (gr + e < R_) ? src[e] : 0.f;
              }
              if (causal != CAUSAL_NONE) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = mask_causal(v[e], causal, gr + e, gk);
              }
            }
            r[i * 4 + kk] = v;
          } else {
            const unsigned short* P = static_cast<const unsigned short*>(Pv);
            u16x4 v = {0, 0, 0, 0};
            if (gk < K) {
              const unsigned short* src = P + (int64_t)gk * ld + gr;
              if (vec && gr + 3 < R_) {
                v = *reinterpret_cast<const u16x4*>(src);
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (gr + e < R_) ? src[e] : (unsigned short)0;
              }
              if (causal != CAUSAL_NONE) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if ((causal == CAUSAL_UPTO && gk > gr + e) || (causal == CAUSAL_FROM && gk < gr + e)) v[e] = 0;
              }
            }
            r[i * 8 + kk] = v;
          }
        }
      }
    }
  }

  // Interior tile: every element of the R_TILE x BK block is in range, the
  // rows are 16-byte aligned and no causal mask applies -- straight-line loads.
  __device__ __forceinline__ void load_fast(const void* __restrict__ Pv, int64_t ld, int r0, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = tid + i * NT;
      if (UNITS % NT != 0 && u >= UNITS) break;
      if constexpr (!RCONTIG) {
        const int rr = u / (BK / UK), kq = u % (BK / UK);
        const int64_t off = (int64_t)(r0 + rr) * ld + k0 + kq * UK;
        if constexpr (!SRC_BF16)
          r[i] = *reinterpret_cast<const f4*>(static_cast<const float*>(Pv) + off);
        else
          r[i] = *reinterpret_cast<const u16x8*>(static_cast<const unsigned short*>(Pv) + off);
      } else {
        const int rq = u % (R_TILE / 4), kq = u / (R_TILE / 4);
#pragma unroll
        for (int kk = 0; kk < UK; ++kk) {
          const int64_t off = (int64_t)(k0 + kq * UK + kk) * ld + r0 + rq * 4;
          if constexpr (!SRC_BF16)
            r[i * 4 + kk] = *reinterpret_cast<const f4*>(static_cast<const float*>(Pv) + off);
          else
            r[i * 8 + kk] = *reinterpret_cast<const u16x4*>(static_cast<const unsigned short*>(Pv) + off);
        }
      }
    }
  }

  // LDK: LDS row pitch in elements (Lds<BF16, BK>::LDK)
  template <bool BF16, int LDK>
  __device__ __forceinline__ void store(typename Lds<BF16, BK>::T* L, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = tid + i * NT;
      if (UNITS % NT != 0 && u >= UNITS) break;
      if constexpr (!RCONTIG) {
        const int rr = u / (BK / UK), kq = u % (BK / UK);
        if constexpr (!SRC_BF16)
          put4<BF16>(L + Lds<BF16, BK>::off(rr, kq * 4), r[i]);
        else
          *reinterpret_cast<u16x8*>(L + Lds<BF16, BK>::off(rr, kq * 8)) = r[i];
      } else {
        const int rq = u % (R_TILE / 4), kq = u / (R_TILE / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (!SRC_BF16) {
            f4 v = {r[i * 4 + 0][e], r[i * 4 + 1][e], r[i * 4 + 2][e], r[i * 4 + 3][e]};
            put4<BF16>(L + Lds<BF16, BK>::off(rq * 4 + e, kq * 4), v);
          } else {
            u16x8 v;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) v[kk] = r[i * 8 + kk][e];
            *reinterpret_cast<u16x8*>(L + Lds<BF16, BK>::off(rq * 4 + e, kq * 8)) = v;
          }
        }
      }
    }
  }

  template <bool BF16>
  __device__ __forceinline__ static void put4(typename Lds<BF16, BK>::T* dst, f4 v) {
    if constexpr (BF16) {
      bf16x4 b = {(bf16_t)v[0], (bf16_t)v[1], (bf16_t)v[2], (bf16_t)v[3]};
      *reinterpret_cast<bf16x4*>(dst) = b;
    } else {
      *reinterpret_cast<f4*>(dst) = v;
    }
  }
};

// A bf16 r-contiguous (m- or n-contiguous) operand staged in its own layout:
// LDS holds the tile as [k][r] with rows of R_TILE + 32 elements, filled by
// straight 16-byte copies; the MFMA fragments (8 consecutive k of one r per
// lane) are read with the transposing LDS read ds_read_b64_tr_b16.  Within a
// group of 16 lanes that instruction hands lane j element e of the 8 bytes
// addressed by lane 4e + j/4, at position j%4; so lane i of the group points at
// row kb + i/4, columns rb + 4(i%4) .. +3, and lane j receives r = rb + j,
// k = kb .. kb + 3.  A 32-lane phase of the read covers four k-rows x 64
// bytes; the 64-byte row pad staggers consecutive rows by 16 banks, so the
// phase touches each of the 64 banks once.
template <int R_TILE, int NT, int BK>
struct StageTr {
  static constexpr int LDR = R_TILE + 32;
  static constexpr int CPR = R_TILE / 8;  // 16-byte chunks per k-row
  static constexpr int UNITS = BK * CPR;
  static constexpr int PER = (UNITS + NT - 1) / NT;
  u16x8 r[PER];

  __device__ __forceinline__ void load(const void* __restrict__ Pv, int64_t ld, int r0, int k0, int R_, int K,
                                       bool vec, int causal, int tid) {
    const unsigned short* P = static_cast<const unsigned short*>(Pv);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = tid + i * NT;
      if (UNITS % NT != 0 && u >= UNITS) break;
      const int kk = u / CPR, rc = u % CPR;
      const int gk = k0 + kk, gr = r0 + rc * 8;
      u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (gk < K) {
        const unsigned short* src = P + (int64_t)gk * ld + gr;
        if (vec && gr + 7 < R_) {
          v = *reinterpret_cast<const u16x8*>(src);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (gr + e < R_) ? src[e] : (unsigned short)0;
        }
        if (causal != CAUSAL_NONE) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if ((causal == CAUSAL_UPTO && gk > gr + e) || (causal == CAUSAL_FROM && gk < gr + e)) v[e] = 0;
        }
      }
      r[i] = v;
    }
  }

  __device__ __forceinline__ void load_fast(const void* __restrict__ Pv, int64_t ld, int r0, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = tid + i * NT;
      if (UNITS % NT != 0 && u >= UNITS) break;
      const int kk = u / CPR, rc = u % CPR;
      r[i] = *reinterpret_cast<const u16x8*>(static_cast<const unsigned short*>(Pv) + (int64_t)(k0 + kk) * ld + r0 +
                                              rc * 8);
    }
  }

  template <bool BF16, int LDK>
  __device__ __forceinline__ void store(bf16_t* L, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int u = tid + i * NT;
      if (UNITS % NT != 0 && u >= UNITS) break;
      const int kk = u / CPR, rc = u % CPR;
      *reinterpret_cast<u16x8*>(L + kk * LDR + rc * 8) = r[i];
    }
  }
};

// the 8 bf16 of one MFMA fragment from two transposing reads, 4 k-rows apart
__device__ __forceinline__ bf16x8 frag_tr(const bf16_t* p, int ld) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p + 4 * ld));
  const v8i16 c = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

struct KArgs {
  GemmArgs g;
  int tiles_m, tiles_n;
  int splits;
  int k_per_split;  // multiple of KALIGN
  int group_m;      // tile rows per raster group
  float* ws;        // split-K partials [batch*splits][M][N]
};

template <int WM, int WN, int TM, int TN, int BK, bool BF16, bool A_RC, bool B_KC, bool A_BF, bool B_BF>
__global__ __launch_bounds__(WM* WN * 64, 2) void gemm_kernel(KArgs ka) {
  constexpr int NT = WM * WN * 64;
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int LDK = Lds<BF16, BK>::LDK;
  using LT = typename Lds<BF16, BK>::T;
  // a bf16 r-contiguous operand keeps its own [k][r] layout in LDS (StageTr)
  constexpr bool TRA = BF16 && A_BF && A_RC && BK % 16 == 0;
  constexpr bool TRB = BF16 && B_BF && !B_KC && BK % 16 == 0;
  constexpr int LDA = TRA ? BM + 32 : LDK, LDB = TRB ? BN + 32 : LDK;
  constexpr int ASZ = TRA ? BK * LDA : BM * LDA, BSZ = TRB ? BK * LDB : BN * LDB;
  // after the k loop the epilogue restages each wave's 32-row slabs of C here
  constexpr int EP = TN * 32 + 4;
  constexpr int SMEM = std::max<int>((2 * ASZ + 2 * BSZ) * (int)sizeof(LT), WM * WN * 32 * EP * 4);
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  LT(*As)[ASZ] = reinterpret_cast<LT(*)[ASZ]>(smem);
  LT(*Bs)[BSZ] = reinterpret_cast<LT(*)[BSZ]>(smem + 2 * ASZ * sizeof(LT));

  const GemmArgs& g = ka.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform by construction
  const int wm = wave / WN, wn = wave % WN;

  // Work item order.  The grid is 1-D over (batch x split) slabs of tiles_m x
  // tiles_n tiles.  Workgroup w runs on XCD w % 8, so the ids are renumbered to
  // give each XCD one contiguous range of work items; inside a slab, items run
  // in groups of GEMM_GROUP_M tile rows, column by column, so the workgroups an
  // XCD holds at once share a few A row panels and B column panels in its L2.
  const int ntiles = ka.tiles_m * ka.tiles_n;
  const int total = (int)gridDim.x;
  int id;
  {
    const int w = blockIdx.x, xcd = w & 7, per = total >> 3, rem = total & 7;
    id = xcd * per + min(xcd, rem) + (w >> 3);
  }
  const int zz = id / ntiles;
  int t = id - zz * ntiles;
  int tm, tn;
  {
    const int gm = ka.group_m;
    const int band = gm * ka.tiles_n;
    const int first = (t / band) * gm;
    const int rows = min(ka.tiles_m - first, gm);
    t -= (first / gm) * band;
    tm = first + t % rows;
    tn = t / rows;
  }
  const int z = zz / ka.splits, split = zz % ka.splits;
  const int m0 = tm * BM, n0 = tn * BN;
  if (g.causal_out && n0 > m0 + BM - 1) return;

  const int z1 = z / g.batch_div, z2 = z % g.batch_div;
  const int eA = A_BF ? 2 : 4, eB = B_BF ? 2 : 4;
  const char* A = reinterpret_cast<const char*>(g.A) + (z1 * g.sa1 + z2 * g.sa2) * eA;
  const char* B = reinterpret_cast<const char*>(g.B) + (z1 * g.sb1 + z2 * g.sb2) * eB;

  int kb = split * ka.k_per_split;
  int ke = min(g.K, kb + ka.k_per_split);
  if (g.causal_a == CAUSAL_UPTO) ke = min(ke, m0 + BM);
  if (g.causal_a == CAUSAL_FROM) kb = max(kb, (m0 / BK) * BK);

  // 16-byte vector loads need 16-byte aligned rows and batch offsets
  const bool vecA = ((reinterpret_cast<uintptr_t>(A) & 15) == 0) && (g.lda % (16 / eA) == 0);
  const bool vecB = ((reinterpret_cast<uintptr_t>(B) & 15) == 0) && (g.ldb % (16 / eB) == 0);
  // the m/n extent of this tile is entirely in range for both operands
  const bool interior = vecA && vecB && m0 + BM <= g.M && n0 + BN <= g.N;

  // a k-tile is loaded without checks when it is interior, complete and away from the causal diagonal
  auto load_tile = [&](auto& xa, auto& xb, int k0) {
    bool fast = interior && k0 + BK <= ke;
    if (g.causal_a == CAUSAL_UPTO) fast = fast && k0 + BK - 1 <= m0;
    if (g.causal_a == CAUSAL_FROM) fast = fast && k0 >= m0 + BM - 1;
    if (fast) {
      xa.load_fast(A, g.lda, m0, k0, tid);
      xb.load_fast(B, g.ldb, n0, k0, tid);
    } else {
      xa.load(A, g.lda, m0, k0, g.M, ke, vecA, g.causal_a, tid);
      xb.load(B, g.ldb, n0, k0, g.N, ke, vecB, CAUSAL_NONE, tid);
    }
  };
  auto store_tile = [&](const auto& xa, const auto& xb, int b) {
    xa.template store<BF16, LDA>(As[b], tid);
    xb.template store<BF16, LDB>(Bs[b], tid);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lrow = lane & 31, lhalf = lane >> 5;
  // transposing-read lane offsets: lane 16g + i reads row 8(g/2) + i/4 (+4 for the
  // second half), columns 16(g%2) + 4(i%4)
  const int tr_row = 8 * (lane >> 5) + ((lane & 15) >> 2), tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto compute = [&](int b) {
    const LT* Ab = TRA ? As[b] + tr_row * LDA + wm * TM * 32 + tr_col : As[b] + (wm * TM * 32 + lrow) * LDA;
    const LT* Bb = TRB ? Bs[b] + tr_row * LDB + wn * TN * 32 + tr_col : Bs[b] + (wn * TN * 32 + lrow) * LDB;
    if constexpr (BF16) {
#pragma unroll
      for (int ks = 0; ks < BK; ks += 16) {
        bf16x8 af[TM], bf[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if constexpr (TRA)
            af[i] = frag_tr(Ab + ks * LDA + i * 32, LDA);
          else
            af[i] = *reinterpret_cast<const bf16x8*>(Ab + i * 32 * LDA + Lds<true, BK>::off(lrow, ks + lhalf * 8) -
                                                     lrow * LDA);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (TRB)
            bf[j] = frag_tr(Bb + ks * LDB + j * 32, LDB);
          else
            bf[j] = *reinterpret_cast<const bf16x8*>(Bb + j * 32 * LDB + Lds<true, BK>::off(lrow, ks + lhalf * 8) -
                                                     lrow * LDB);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kg = 0; kg < BK; kg += 8) {
        f4 af[TM], bf[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const f4*>(Ab + i * 32 * LDA + kg + lhalf * 4);
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[j] = *reinterpret_cast<const f4*>(Bb + j * 32 * LDB + kg + lhalf * 4);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(bf[j][c], af[i][c], acc[i][j], 0, 0, 0);
      }
    }
  };

  // Pipeline: k-tile t is multiplied out of LDS buffer t % 2 while tile t + 1
  // is fetched into registers; one barrier per k-tile.
  using SA = typename std::conditional<TRA, StageTr<BM, NT, BK>, Stage<BM, NT, A_RC, A_BF, BK>>::type;
  using SB = typename std::conditional<TRB, StageTr<BN, NT, BK>, Stage<BN, NT, !B_KC, B_BF, BK>>::type;
  bool done = false;
  if constexpr (GEMM_PIPE && BF16 && A_BF && B_BF && TM * TN <= 6 && BK == 64) {
    // Interior tile free of the causal mask: a branch-free two-deep pipeline over
    // its whole k-tiles.  Tile j waits in register set j % 2; at step t the loads
    // of tile t + 2, the LDS stores of tile t + 1 and the MFMAs of tile t are
    // interleaved in one basic block, one barrier per step.  A ragged last k-tile
    // follows through the checked loader.
    const int nt = (ke - kb) / BK;
    if (interior && g.causal_a == CAUSAL_NONE && nt >= 1) {
      done = true;
      SA a0, a1;
      SB b0, b1;
      a0.load_fast(A, g.lda, m0, kb, tid);
      b0.load_fast(B, g.ldb, n0, kb, tid);
      if (nt > 1) {
        a1.load_fast(A, g.lda, m0, kb + BK, tid);
        b1.load_fast(B, g.ldb, n0, kb + BK, tid);
      }
      store_tile(a0, b0, 0);
      __syncthreads();
      auto hint = [&]() {
        constexpr int NMF = TM * TN * (BK / 16);
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
        }
      };
      int t = 0;
      for (; t + 3 < nt; t += 2) {
        a0.load_fast(A, g.lda, m0, kb + (t + 2) * BK, tid);
        b0.load_fast(B, g.ldb, n0, kb + (t + 2) * BK, tid);
        compute(0);
        store_tile(a1, b1, 1);
        hint();
        __syncthreads();
        a1.load_fast(A, g.lda, m0, kb + (t + 3) * BK, tid);
        b1.load_fast(B, g.ldb, n0, kb + (t + 3) * BK, tid);
        compute(1);
        store_tile(a0, b0, 0);
        hint();
        __syncthreads();
      }
      for (; t < nt; ++t) {  // the last one to three tiles; t is even on entry
        if ((t & 1) == 0) {
          if (t + 2 < nt) {
            a0.load_fast(A, g.lda, m0, kb + (t + 2) * BK, tid);
            b0.load_fast(B, g.ldb, n0, kb + (t + 2) * BK, tid);
          }
          compute(0);
          if (t + 1 < nt) store_tile(a1, b1, 1);
        } else {
          compute(1);
          if (t + 1 < nt) store_tile(a0, b0, 0);
        }
        __syncthreads();
      }
      const int kt = kb + nt * BK;
      if (kt < ke) {  // ragged last k-tile; every LDS buffer is free after the barrier above
        load_tile(a0, b0, kt);
        store_tile(a0, b0, 0);
        __syncthreads();
        compute(0);
      }
    }
  }
  if (!done) {
    SA sa;
    SB sb;
    if (kb < ke) {
      load_tile(sa, sb, kb);
      store_tile(sa, sb, 0);
    }
    __syncthreads();
    int buf = 0;
    for (int k0 = kb; k0 < ke; k0 += BK) {
      const bool more = k0 + BK < ke;
      if (more) load_tile(sa, sb, k0 + BK);
      compute(buf);
      if (more) store_tile(sa, sb, buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  // Epilogue.  The MFMAs take B's fragment as their first operand, so each
  // 32x32 block accumulates C^T: register r holds C[lane%32][8*(r/4) + 4*(lane/32) + r%4],
  // and registers 4q .. 4q+3 are four consecutive columns of one row.
  const bool to_ws = ka.splits > 1;
  float* C;
  int64_t ldc;
  if (to_ws) {
    C = ka.ws + (int64_t)zz * g.M * g.N;
    ldc = g.N;
  } else {
    C = g.C + z1 * g.sc1 + z2 * g.sc2;
    ldc = g.ldc;
  }
  const float* bias = to_ws ? nullptr : g.bias;
  const float* resid = to_ws ? nullptr : g.resid;
  uint16_t* Cbf = to_ws ? nullptr : g.Cbf;
  const bool skipc = !to_ws && g.c_bf16_only;  // the bf16 copy alone
  const bool vec = (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(C) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(bias) & 15) == 0) && ((reinterpret_cast<uintptr_t>(Cbf) & 7) == 0) &&
                   ((reinterpret_cast<uintptr_t>(resid) & 15) == 0);
  if (vec) {
    // 16-byte rows: each wave writes one 32-row slab of its blocks to its own
    // LDS region and reads it back so that 16 lanes hold 64 consecutive
    // columns of one row; a store instruction then writes 4 rows x 256
    // contiguous bytes (whole cache lines) instead of 32 rows x 32 bytes.  The
    // regions are wave-private: one workgroup barrier frees the operand tiles.
    __syncthreads();
    float* E = reinterpret_cast<float*>(smem) + wave * 32 * EP;
    constexpr int C4 = TN * 8;  // float4 per slab row
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f4*>(E + lrow * EP + j * 32 + 8 * q + 4 * lhalf) =
              f4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int it = 0; it < 32 * C4 / 64; ++it) {
        const int f = it * 64 + lane, r = f / C4, c4 = f % C4;
        f4 v = *reinterpret_cast<const f4*>(E + r * EP + c4 * 4) * g.alpha;
        const int m = m0 + wm * TM * 32 + i * 32 + r, n = n0 + wn * TN * 32 + c4 * 4;
        if (m >= g.M) continue;
        float* row = C + (int64_t)m * ldc;
        if (n + 3 < g.N) {
          if (bias) v += *reinterpret_cast<const f4*>(bias + n);
          f4* dst = reinterpret_cast<f4*>(row + n);
          if (!to_ws && g.beta != 0.f) v += g.beta * *dst;
          if (resid) v += *reinterpret_cast<const f4*>(resid + (int64_t)m * ldc + n);
          if (!skipc) *dst = v;
          if (Cbf) *reinterpret_cast<u16x4*>(Cbf + (int64_t)m * ldc + n) = bf16x4_bits(v);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (n + e >= g.N) break;
            float x = v[e];
            if (bias) x += bias[n + e];
            if (!to_ws && g.beta != 0.f) x += g.beta * row[n + e];
            if (resid) x += resid[(int64_t)m * ldc + n + e];
            if (!skipc) row[n + e] = x;
            if (Cbf) Cbf[(int64_t)m * ldc + n + e] = bf16_bits(x);
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    return;
  }
  // otherwise element stores straight from the accumulators
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm * TM * 32 + i * 32 + lrow;
    if (m >= g.M) continue;
    float* row = C + (int64_t)m * ldc;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * TN * 32 + j * 32 + 8 * q + 4 * lhalf;
        const f4 v = f4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]} * g.alpha;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (n + e >= g.N) break;
          float x = v[e];
          if (bias) x += bias[n + e];
          if (!to_ws && g.beta != 0.f) x += g.beta * row[n + e];
          if (resid) x += resid[(int64_t)m * ldc + n + e];
          if (!skipc) row[n + e] = x;
          if (Cbf) Cbf[(int64_t)m * ldc + n + e] = bf16_bits(x);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large products with both operands stored as bf16 (the LM head and its weight
// gradient): 256x256 tiles, eight waves of 128x64, operands loaded from global
// memory straight into LDS (buffer_load ... lds), two LDS stages of 64-deep
// k-tiles.  A tile this size does twice the MFMA work per byte fetched of a
// 128x128 one, and the loads need neither staging registers nor LDS stores.
//
// LDS layout.  One load instruction moves 64 lanes x 16 bytes into 1 KB of LDS
// at consecutive addresses, so the layout is chosen through which global chunk
// each lane fetches:
//   k-contiguous operand: rows of 64 k (128 bytes); 16-byte chunk p of row r
//     holds k-chunk p ^ ((r >> 1) & 7), so the 16 rows a fragment read touches
//     at once cover all 64 banks;
//   m- or n-contiguous operand: k-rows of 256 elements (512 bytes); 64-byte
//     block b of k-row k holds column block b ^ (k & 3), so the four k-rows a
//     transposing read (ds_read_b64_tr_b16) touches at once cover all banks.
// Buffer loads return zeros past the operand's end (rounded up to its last
// 16-byte chunk): rows and columns beyond M, N or K read nothing outside the
// operand.  In a k-tile that runs past K, the columns beyond K of a k-contiguous
// operand (the next row's elements) are cleared in LDS before use.
namespace dma {

constexpr int BK = 64;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

struct Args {
  const void* A;
  const void* B;
  float* C;
  uint16_t* Cbf;
  const float* bias;
  const float* resid;
  int M, N, K;
  int64_t lda, ldb, ldc;
  float alpha, beta;
  int skipc;
  int tiles_m, tiles_n, group_m;
  int a_bytes, b_bytes;  // readable bytes of A and B
  int splits, kps;       // K split: items of kps k (a multiple of BK) ...
  float* ws;             // ... write raw partials ws[split][M][N] (splits > 1)
};

// One operand's k-tile: R rows (m or n) x 64 k, R * 128 bytes in 1 KB segments,
// PER of them per wave (wave w issues segments w, w + NW, w + 2 NW, ...).
template <int R, int NW>
struct Seg {
  static constexpr int BYTES = R * BK * 2;
  static constexpr int PER = BYTES / 1024 / NW;
  static_assert(PER * NW * 1024 == BYTES, "whole segments per wave");
};

// Per-lane global byte offsets of one operand's share of k-tile 0
template <bool RC, int R, int NW>
__device__ __forceinline__ void seg_offsets(int* voff, int r0, int64_t ld, int wave, int lane) {
  constexpr int PER = Seg<R, NW>::PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int s = i * NW + wave;
    if constexpr (!RC) {  // 8 rows of 128 bytes per segment
      const int r = s * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      voff[i] = (int)(((int64_t)(r0 + r) * ld + c * 8) * 2);
    } else {              // 512 / R k-rows of 2R bytes per segment
      constexpr int CPR = R / 8;  // 16-byte chunks per k-row
      const int k = s * (64 / CPR) + lane / CPR, p = lane % CPR;
      const int c = (((p >> 2) ^ (k & 3)) << 2) | (p & 3);
      voff[i] = (int)(((int64_t)k * ld + r0 + 8 * c) * 2);
    }
  }
}

template <int R, int NW>
__device__ __forceinline__ void load_segs(__amdgpu_buffer_rsrc_t rs, char* stage, const int* voff, int adv, int wave) {
#pragma unroll
  for (int i = 0; i < Seg<R, NW>::PER; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(stage + (i * NW + wave) * 1024), 16, voff[i] + adv, 0,
                                             0, 0);
}

// k-contiguous layout: the 8 k of the MFMA fragment of row `row`, k-step q
__device__ __forceinline__ bf16x8 frag_rows(const char* st, int row, int q, int lane) {
  const int c = 2 * q + (lane >> 5);
  return *reinterpret_cast<const bf16x8*>(st + row * 128 + ((c ^ ((row >> 1) & 7)) << 4));
}
// m/n-contiguous layout (k-rows of R elements): the fragment of column block blk (32 columns), k-step q
template <int R>
__device__ __forceinline__ bf16x8 frag_cols(const char* st, int blk, int q, int lane) {
  const int tr_row = 8 * (lane >> 5) + ((lane & 15) >> 2), tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int k = q * 16 + tr_row;
  const char* p = st + k * (2 * R) + ((blk ^ (k & 3)) << 6) + tr_col * 2;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p + 8 * R));
  const v8i16 c = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// clear k-columns kr..63 of a k-contiguous operand's k-tile (R rows) in LDS
template <int R, int NT>
__device__ __forceinline__ void clear_tail(char* st, int kr, int tid) {
  for (int u = tid; u < R * 8; u += NT) {
    const int r = u >> 3, p = u & 7, c = p ^ ((r >> 1) & 7);
    unsigned short* e = reinterpret_cast<unsigned short*>(st + r * 128 + p * 16);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c * 8 + j >= kr) e[j] = 0;
  }
}

}  // namespace dma

// WM x WN waves of TM x TN blocks: 2x4 of 4x2 (256x256 tiles, one workgroup per
// CU) or 2x2 of 2x2 (128x128 tiles, two per CU)
template <int WM, int WN, int TM, int TN, bool A_RC, bool B_KC>
__global__ __launch_bounds__(WM* WN * 64, WM* WN == 4 ? 2 : 1) void gemm_dma_kernel(dma::Args g) {
  using namespace dma;
  constexpr bool B_RC = !B_KC;
  constexpr int NT = WM * WN * 64, NW = WM * WN;
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int OPA = Seg<BM, NW>::BYTES, OPB = Seg<BN, NW>::BYTES;
  constexpr int STAGE = OPA + OPB;
  constexpr int EP = TN * 32 + 4;  // epilogue row pitch (floats)
  constexpr int SMEM = 2 * STAGE;
  static_assert(WM * WN * 32 * EP * 4 <= SMEM, "epilogue staging fits in the operand stages");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // the XCD-contiguous, row-grouped tile order of gemm_kernel, K splits outermost
  const int total = (int)gridDim.x;
  int t;
  {
    const int w = blockIdx.x, xcd = w & 7, per = total >> 3, rem = total & 7;
    t = xcd * per + min(xcd, rem) + (w >> 3);
  }
  const int split = t / (g.tiles_m * g.tiles_n);
  t -= split * (g.tiles_m * g.tiles_n);
  int tm, tn;
  {
    const int gm = g.group_m, band = gm * g.tiles_n, first = (t / band) * gm;
    const int rows = min(g.tiles_m - first, gm);
    t -= (first / gm) * band;
    tm = first + t % rows;
    tn = t / rows;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb = split * g.kps, ke = min(g.K, kb + g.kps);

  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)g.A, (short)0, g.a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void*)g.B, (short)0, g.b_bytes, 0x00020000);
  int va[Seg<BM, NW>::PER], vb[Seg<BN, NW>::PER];
  seg_offsets<A_RC, BM, NW>(va, m0, g.lda, wave, lane);
  seg_offsets<B_RC, BN, NW>(vb, n0, g.ldb, wave, lane);
  const int adv_a = A_RC ? (int)(BK * g.lda * 2) : BK * 2;
  const int adv_b = B_RC ? (int)(BK * g.ldb * 2) : BK * 2;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lrow = lane & 31;
  const int nt = (ke - kb + BK - 1) / BK, kr = ke - kb - (nt - 1) * BK;  // kr: k in the last k-tile
  const int t0 = kb / BK;
  load_segs<BM, NW>(ra, smem, va, t0 * adv_a, wave);
  load_segs<BN, NW>(rb, smem + OPA, vb, t0 * adv_b, wave);
  // k-tile kt is multiplied out of stage kt % 2 while k-tile kt + 1 loads into
  // the other: its fragments are read first, then the next loads are issued
  // (the compiler waits for every outstanding LDS load before an LDS read, so
  // the reads must precede them), then the MFMAs run.
  for (int kt = 0; kt < nt; ++kt) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's share of k-tile kt is in LDS
    __syncthreads();                     // everyone's is; everyone is done reading k-tile kt - 1
    char* As = smem + (kt & 1) * STAGE;
    char* Bs = As + OPA;
    if (kt == nt - 1 && kr < BK && (!A_RC || B_KC)) {
      if constexpr (!A_RC) clear_tail<BM, NT>(As, kr, tid);
      if constexpr (B_KC) clear_tail<BN, NT>(Bs, kr, tid);
      __syncthreads();
    }
    bf16x8 af[BK / 16][TM], bf[BK / 16][TN];
#pragma unroll
    for (int q = 0; q < BK / 16; ++q) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[q][i] = A_RC ? frag_cols<BM>(As, wm * TM + i, q, lane) : frag_rows(As, wm * TM * 32 + i * 32 + lrow, q, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[q][j] = B_RC ? frag_cols<BN>(Bs, wn * TN + j, q, lane) : frag_rows(Bs, wn * TN * 32 + j * 32 + lrow, q, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nt) {
      char* nx = smem + ((kt + 1) & 1) * STAGE;  // last read in iteration kt - 1, before the barrier above
      load_segs<BM, NW>(ra, nx, va, (t0 + kt + 1) * adv_a, wave);
      load_segs<BN, NW>(rb, nx + OPA, vb, (t0 + kt + 1) * adv_b, wave);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < BK / 16; ++q)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[q][j], af[q][i], acc[i][j], 0, 0, 0);
  }

  // Epilogue as in gemm_kernel: each wave restages a 32-row slab of its blocks
  // (C^T per block: register r holds row lane%32, column 8(r/4) + 4(lane/32) + r%4)
  // through its own LDS region into whole rows.
  __syncthreads();
  const int lhalf = lane >> 5;
  float* E = reinterpret_cast<float*>(smem) + wave * 32 * EP;
  constexpr int C4 = TN * 8;
  // a K split writes its raw partial; the reduction applies the rest
  const bool part = g.splits > 1;
  float* const Cd = part ? g.ws + (int64_t)split * g.M * g.N : g.C;
  const int64_t ldc = part ? g.N : g.ldc;
  const float* const bias = part ? nullptr : g.bias;
  const float* const resid = part ? nullptr : g.resid;
  uint16_t* const Cbf = part ? nullptr : g.Cbf;
  const float beta = part ? 0.f : g.beta;
  const bool skipc = !part && g.skipc;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f4*>(E + lrow * EP + j * 32 + 8 * q + 4 * lhalf) =
            f4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < 32 * C4 / 64; ++it) {
      const int f = it * 64 + lane, r = f / C4, c4 = f % C4;
      f4 v = *reinterpret_cast<const f4*>(E + r * EP + c4 * 4) * g.alpha;
      const int m = m0 + wm * TM * 32 + i * 32 + r, n = n0 + wn * TN * 32 + c4 * 4;
      if (m >= g.M || n >= g.N) continue;
      float* row = Cd + (int64_t)m * ldc;
      if (n + 3 < g.N) {
        if (bias) v += *reinterpret_cast<const f4*>(bias + n);
        f4* dst = reinterpret_cast<f4*>(row + n);
        if (beta != 0.f) v += beta * *dst;
        if (resid) v += *reinterpret_cast<const f4*>(resid + (int64_t)m * ldc + n);
        if (!skipc) *dst = v;
        if (Cbf) *reinterpret_cast<u16x4*>(Cbf + (int64_t)m * ldc + n) = bf16x4_bits(v);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (n + e >= g.N) break;
          float x = v[e];
          if (bias) x += bias[n + e];
          if (beta != 0.f) x += beta * row[n + e];
          if (resid) x += resid[(int64_t)m * ldc + n + e];
          if (!skipc) row[n + e] = x;
          if (Cbf) Cbf[(int64_t)m * ldc + n + e] = bf16_bits(x);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// The same over float4 (N, ldc multiples of 4, 16-byte aligned C and bias)
__global__ void splitk_reduce4(const f4* __restrict__ ws, int splits, int M, int N4, float* C, int64_t ldc,
                               int batch_div, int64_t sc1, int64_t sc2, float beta, const f4* bias, uint16_t* Cbf,
                               const float* resid, int skipc) {
  const int z = blockIdx.y;
  const int64_t MN4 = (int64_t)M * N4;
  const int z1 = z / batch_div, z2 = z % batch_div;
  float* Cz = C + z1 * sc1 + z2 * sc2;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < MN4; e += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(e / N4), n4 = (int)(e % N4);
    f4 s = {0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < splits; ++p) s += ws[((int64_t)z * splits + p) * MN4 + e];
    if (bias) s += bias[n4];
    f4* dst = reinterpret_cast<f4*>(Cz + (int64_t)m * ldc) + n4;
    if (beta != 0.f) s += beta * *dst;
    if (resid) s += *reinterpret_cast<const f4*>(resid + (int64_t)m * ldc + 4 * n4);
    if (!skipc) *dst = s;
    if (Cbf) *reinterpret_cast<u16x4*>(Cbf + (Cz - C) + (int64_t)m * ldc + 4 * n4) = bf16x4_bits(s);
  }
}

// C = sum over splits of the partials + beta*C + bias
__global__ void splitk_reduce(const float* __restrict__ ws, int splits, int M, int N, float* C, int64_t ldc,
                              int batch_div, int64_t sc1, int64_t sc2, float beta, const float* bias, uint16_t* Cbf,
                              const float* resid, int skipc) {
  const int z = blockIdx.y;
  const int64_t MN = (int64_t)M * N;
  const int z1 = z / batch_div, z2 = z % batch_div;
  float* Cz = C + z1 * sc1 + z2 * sc2;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < MN; e += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(e / N), n = (int)(e % N);
    float s = 0.f;
    for (int p = 0; p < splits; ++p) s += ws[((int64_t)z * splits + p) * MN + e];
    if (bias) s += bias[n];
    float* dst = Cz + (int64_t)m * ldc + n;
    if (beta != 0.f) s += beta * *dst;
    if (resid) s += resid[(int64_t)m * ldc + n];
    if (!skipc) *dst = s;
    if (Cbf) Cbf[(Cz - C) + (int64_t)m * ldc + n] = bf16_bits(s);
  }
}

enum Cfg { CFG_128x128 = 1, CFG_128x64 = 2, CFG_256x128 = 3, CFG_128x192 = 4 };

struct Plan {
  int cfg;
  int BM, BN;
  int bk;  // k-tile depth when both operands are stored as bf16
  int splits;
  int k_per_split;
};

Plan make_plan(const GemmArgs& g) {
  Plan p;
  if (g.N <= 64) {
    p.cfg = CFG_128x64, p.BM = 128, p.BN = 64;
  } else if (g.prec == PREC_BF16 && g.a_bf16 && g.b_bf16 && g.causal_a == CAUSAL_NONE && !g.causal_out &&
             (int64_t)((g.M + 255) / 256) * ((g.N + 127) / 128) * g.batch >= GEMM_BIG_TILES) {
    // 4 waves of 128x64 read a quarter less LDS per MFMA; two workgroups fit per CU
    // only with 32-deep k-tiles, which pays off on vocabulary-sized products
    p.cfg = CFG_256x128, p.BM = 256, p.BN = 128;
  } else if (g.prec == PREC_BF16 && g.a_bf16 && g.b_bf16 && g.causal_a == CAUSAL_NONE && !g.causal_out &&
             g.N % 192 == 0 && g.K >= 2048 && (int64_t)((g.M + 127) / 128) * (g.N / 192) * g.batch <= 256 &&
             (int64_t)((g.M + 127) / 128) * (g.N / 192) * g.batch > 192) {
    // About one 128x192 tile per CU (N = 768 against 8192 rows): the 128x128
    // tiling would leave half the CUs with two tiles and half with one.  These
    // tiles take 92 KB of LDS and ~410 registers, one workgroup per CU; with
    // long reductions that beats the 128x128 tiles (and their K split)
    p.cfg = CFG_128x192, p.BM = 128, p.BN = 192;
  } else {
    p.cfg = CFG_128x128, p.BM = 128, p.BN = 128;
  }
  const int64_t tiles = (int64_t)((g.M + p.BM - 1) / p.BM) * ((g.N + p.BN - 1) / p.BN) * g.batch;
  // Both operands bf16: 64-deep k-tiles (72 KB of LDS, two workgroups per CU,
  // the pipelined path); the 256x128 tiles fit two per CU only 32 deep.
  p.bk = p.cfg == CFG_256x128 ? 32 : 64;
  // K split: the workgroups resident at once (slots) run in rounds, so a tile
  // count just past a multiple of the slots wastes most of a round.  Pick the
  // split that minimizes rounds x (k-tiles per item) plus the partials'
  // traffic (written and read once more by the reduction, priced at 2.5 TB/s:
  // it competes with the product's own traffic; 5 TB/s chose splits 7% slower
  // on the GPT-2 dW products), with at least 512 k per item.
  // Products of at most 64 rows (cached decoding: one token per sequence) have
  // a few tiles whose k loop is pure latency: there the split goes down to two
  // k-tiles per item.
  p.splits = 1;
  const bool skinny = g.M <= 64 && g.batch == 1;
  if (g.causal_a == CAUSAL_NONE && !g.causal_out && (g.K >= 1024 || (skinny && g.K >= 256))) {
    const int64_t slots = 256 * (p.cfg == CFG_128x192 ? 1 : p.bk == 32 ? 3 : 2);
    const double tile_s_per_k = 2.0 * p.BM * p.BN / 1.0e12;  // ~1 TFLOP/s per resident workgroup
    const double out_bytes = 4.0 * g.M * g.N * g.batch;
    const int min_k = skinny ? 128 : 512;
    double best = 0.0;
    for (int sp = 1; sp <= (skinny ? 32 : 16); ++sp) {
      if (sp > 1 && g.K / sp < min_k) break;
      const int64_t items = tiles * sp;
      const double rounds = (double)((items + slots - 1) / slots);
      const double t = rounds * ((double)g.K / sp) * tile_s_per_k + (sp > 1 ? (sp + 1) * out_bytes / 2.5e12 : 0.0);
      if (sp == 1 || t < best * 0.97) best = t, p.splits = sp;
    }
  }
  const int kps = (g.K + p.splits - 1) / p.splits;
  p.k_per_split = ((kps + KALIGN - 1) / KALIGN) * KALIGN;
  p.splits = std::max(1, (g.K + p.k_per_split - 1) / p.k_per_split);
  return p;
}

template <int WM, int WN, int TM, int TN, int BK, bool BF16, bool A_BF, bool B_BF>
hipError_t launch_layout(const KArgs& ka, dim3 grid, hipStream_t s) {
  const GemmArgs& g = ka.g;
  dim3 block(WM * WN * 64);
  if (!g.a_mcontig && !g.b_kcontig)
    run_kernel((gemm_kernel<WM, WN, TM, TN, BK, BF16, false, false, A_BF, B_BF>), grid, block, 0, s, ka);
  else if (!g.a_mcontig && g.b_kcontig)
    run_kernel((gemm_kernel<WM, WN, TM, TN, BK, BF16, false, true, A_BF, B_BF>), grid, block, 0, s, ka);
  else if (g.a_mcontig && !g.b_kcontig)
    run_kernel((gemm_kernel<WM, WN, TM, TN, BK, BF16, true, false, A_BF, B_BF>), grid, block, 0, s, ka);
  else
    return hipErrorInvalidValue;  // A^T B^T is never needed
  return hipGetLastError();
}

// k-tile depth: the plan's choice (32 or 64) when both operands are stored as
// bf16, 32 otherwise (fp32 staging registers would double)
template <int WM, int WN, int TM, int TN>
hipError_t launch_prec(const KArgs& ka, int bk, dim3 grid, hipStream_t s) {
  const GemmArgs& g = ka.g;
  if (g.prec != PREC_BF16) {
    if (g.a_bf16 || g.b_bf16) return hipErrorInvalidValue;
    return launch_layout<WM, WN, TM, TN, 32, false, false, false>(ka, grid, s);
  }
  if (g.a_bf16 && g.b_bf16)
    return bk == 32 ? launch_layout<WM, WN, TM, TN, 32, true, true, true>(ka, grid, s)
                    : launch_layout<WM, WN, TM, TN, 64, true, true, true>(ka, grid, s);
  if (g.a_bf16) return launch_layout<WM, WN, TM, TN, 32, true, true, false>(ka, grid, s);
  if (g.b_bf16) return launch_layout<WM, WN, TM, TN, 32, true, false, true>(ka, grid, s);
  return launch_layout<WM, WN, TM, TN, 32, true, false, false>(ka, grid, s);
}

// gemm_dma_kernel's plan: 0 when it does not take the product, else its K
// splits (*small: 128x128 tiles instead of 256x256).  Conditions: both operands
// bf16 with 16-byte rows, one product, no mask, a vector epilogue, every byte
// offset the loads form within 31 bits, and either enough 256x256 tiles to fill
// the GPU twice or a K long enough to split into items that fill it (N a
// multiple of 4 then, for the partials' rows):
//  - weight gradients (A m-contiguous, K >= 4096) split over K on 128x128 tiles
//    (four waves of 64x64, 64 KB of LDS, two workgroups per CU), with as many
//    splits as fill the CUs once: on the GPT-2 ones (K = 8192) 3-14 splits, 8-17%
//    faster with the reduction than 7-8 splits of 256x256 tiles (half the
//    partials), which ran 14-16% faster than gemm_kernel;
//  - any other layout only with K >= 16,384 (the LM head's dX, K = 50,257: 7%
//    faster), on 256x256 tiles: the 768-wide products with K = 2304-3072 ran
//    20-30% slower split this way (gemm_kernel's one-tile-per-CU 128x192 plan suits
//    them), and the K = 768 products gained nothing from 128x128 tiles of this
//    kernel in the training step.
// 256x256 splits are priced as rounds of 256 items (one per CU) of 1.7 us per
// 64-deep k-tile plus 3 us per item, plus the partials' round trip at 2.5 TB/s.
int dma_plan(const GemmArgs& g, int* kps_out, bool* small) {
  *small = false;
  auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; };
  if (g.prec != PREC_BF16 || !g.a_bf16 || !g.b_bf16 || g.batch != 1 || g.causal_a != CAUSAL_NONE || g.causal_out)
    return 0;
  if (g.K < 1 || g.lda % 8 || g.ldb % 8 || !al(g.A, 16) || !al(g.B, 16)) return 0;
  if (g.ldc % 4 || !al(g.C, 16) || !al(g.bias, 16) || !al(g.resid, 16) || !al(g.Cbf, 8)) return 0;
  const int64_t tm = (g.M + 255) / 256, tn = (g.N + 255) / 256;
  const int64_t kp = (g.K + 63) / 64 * 64;
  const int64_t reach_a = g.a_mcontig ? (kp - 1) * g.lda + tm * 256 : (tm * 256 - 1) * g.lda + kp;
  const int64_t reach_b = g.b_kcontig ? (tn * 256 - 1) * g.ldb + kp : (kp - 1) * g.ldb + tn * 256;
  if (2 * std::max(reach_a, reach_b) >= ((int64_t)1 << 31) - 64) return 0;
  const int nt = (int)(kp / 64);
  *kps_out = (int)kp;
  if (tm * tn >= GEMM_DMA_TILES) return 1;
  if (g.K < GEMM_DMA_SPLIT_K || g.N % 4 || (!g.a_mcontig && g.K < GEMM_DMA_SPLIT_K_ANY)) return 0;
  if (GEMM_DMA128_DW && g.a_mcontig) {  // as many K splits of 128x128 tiles as fill two per CU once
    const int64_t t128 = (int64_t)((g.M + 127) / 128) * ((g.N + 127) / 128);
    const int sp = (int)std::max<int64_t>(1, std::min<int64_t>(512 / t128, nt / 8));
    const int per = (nt + sp - 1) / sp;
    *small = true;
    *kps_out = per * 64;
    return (nt + per - 1) / per;
  }
  int best_sp = 0;
  double best = 0.0;
  for (int sp = 2; sp <= 32; ++sp) {
    const int per = (nt + sp - 1) / sp;
    if (per < 8) break;
    const int64_t items = tm * tn * sp;
    const double t = (double)((items + 255) / 256) * (per * 1.7e-6 + 3e-6) + (sp + 1) * 4.0 * g.M * g.N / 2.5e12;
    if (best_sp == 0 || t < best) best = t, best_sp = sp;
  }
  if (best_sp == 0 || tm * tn * best_sp < 192) return 0;
  const int per = (nt + best_sp - 1) / best_sp;
  *kps_out = per * 64;
  return (nt + per - 1) / per;  // no empty split
}

hipError_t launch_dma(const GemmArgs& g, int splits, int kps, float* ws, bool small, hipStream_t s) {
  dma::Args a;
  a.splits = splits, a.kps = kps, a.ws = ws;
  a.A = g.A, a.B = g.B, a.C = g.C, a.Cbf = g.Cbf, a.bias = g.bias, a.resid = g.resid;
  a.M = g.M, a.N = g.N, a.K = g.K, a.lda = g.lda, a.ldb = g.ldb, a.ldc = g.ldc;
  a.alpha = g.alpha, a.beta = g.beta, a.skipc = g.c_bf16_only ? 1 : 0;
  const int bt = small ? 128 : 256;
  a.tiles_m = (g.M + bt - 1) / bt, a.tiles_n = (g.N + bt - 1) / bt;
  // row groups as gemm_kernel's; tall and narrow (the LM-head weight gradient, 197 x 3 tiles): long ones
  a.group_m = a.tiles_n <= 8 && a.tiles_m >= (small ? 256 : 128)                   ? GEMM_GROUP_TALL
              : small && a.tiles_m >= 32 && a.tiles_n >= 16 && a.tiles_n <= 32 ? GEMM_GROUP_WIDE
                                                                               : GEMM_GROUP_M;
  // Readable bytes: through the 16-byte chunk that holds the last element of the
  // last row.  A 16-byte load that crosses the bound returns zeros for all of it,
  // so the bound must not cut that chunk; the chunk starts 16-byte aligned (rows
  // are), so it lies in the operand's own allocation granule.  Its elements past
  // the end only meet rows or columns of C that are not stored, or k past K,
  // which is cleared in LDS.
  auto chunk_end = [](int64_t elems) { return (int)((2 * elems + 15) / 16 * 16); };
  a.a_bytes = chunk_end(g.a_mcontig ? (int64_t)(g.K - 1) * g.lda + g.M : (int64_t)(g.M - 1) * g.lda + g.K);
  a.b_bytes = chunk_end(g.b_kcontig ? (int64_t)(g.N - 1) * g.ldb + g.K : (int64_t)(g.K - 1) * g.ldb + g.N);
  const dim3 grid(a.tiles_m * a.tiles_n * splits);
  if (small) {
    const dim3 block(256);
    if (!g.a_mcontig && !g.b_kcontig)
      run_kernel(gemm_dma_kernel<2, 2, 2, 2, false, false>, grid, block, 0, s, a);
    else if (!g.a_mcontig && g.b_kcontig)
      run_kernel(gemm_dma_kernel<2, 2, 2, 2, false, true>, grid, block, 0, s, a);
    else if (g.a_mcontig && !g.b_kcontig)
      run_kernel(gemm_dma_kernel<2, 2, 2, 2, true, false>, grid, block, 0, s, a);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  const dim3 block(512);
  if (!g.a_mcontig && !g.b_kcontig)
    run_kernel(gemm_dma_kernel<2, 4, 4, 2, false, false>, grid, block, 0, s, a);
  else if (!g.a_mcontig && g.b_kcontig)
    run_kernel(gemm_dma_kernel<2, 4, 4, 2, false, true>, grid, block, 0, s, a);
  else if (g.a_mcontig && !g.b_kcontig)
    run_kernel(gemm_dma_kernel<2, 4, 4, 2, true, false>, grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

// C = sum of the partials ws[split][M][N] (per batch) + beta C + bias (+ resid), the bf16 copy
static hipError_t reduce_splits(const GemmArgs& g, const float* ws, int splits, hipStream_t s) {
  const int64_t MN = (int64_t)g.M * g.N;
  const bool vec = g.N % 4 == 0 && g.ldc % 4 == 0 && g.sc1 % 4 == 0 && g.sc2 % 4 == 0 &&
                   (reinterpret_cast<uintptr_t>(g.C) & 15) == 0 && (reinterpret_cast<uintptr_t>(g.bias) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(g.Cbf) & 7) == 0 && (reinterpret_cast<uintptr_t>(g.resid) & 15) == 0;
  if (vec) {
    dim3 rgrid((unsigned)std::min<int64_t>((MN / 4 + 255) / 256, 4096), g.batch);
    run_kernel(splitk_reduce4, rgrid, dim3(256), 0, s, reinterpret_cast<const f4*>(ws), splits, g.M,
                       g.N / 4, g.C, g.ldc, g.batch_div, g.sc1, g.sc2, g.beta, reinterpret_cast<const f4*>(g.bias),
                       g.Cbf, g.resid, (int)g.c_bf16_only);
  } else {
    dim3 rgrid((unsigned)std::min<int64_t>((MN + 255) / 256, 4096), g.batch);
    run_kernel(splitk_reduce, rgrid, dim3(256), 0, s, ws, splits, g.M, g.N, g.C, g.ldc, g.batch_div,
                       g.sc1, g.sc2, g.beta, g.bias, g.Cbf, g.resid, (int)g.c_bf16_only);
  }
  return hipGetLastError();
}

size_t gemm_workspace_bytes(const GemmArgs& g) {
  int kps;
  bool small;
  const int dsp = dma_plan(g, &kps, &small);
  if (dsp == 1) return gemv_workspace_bytes(g);
  if (dsp > 1) return std::max((size_t)dsp * g.M * g.N * sizeof(float), gemv_workspace_bytes(g));
  Plan p = make_plan(g);
  const size_t tiled = p.splits <= 1 ? 0 : (size_t)p.splits * g.batch * g.M * g.N * sizeof(float);
  return std::max(tiled, gemv_workspace_bytes(g));
}

hipError_t gemm(const GemmArgs& g, void* workspace, size_t ws_bytes, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  if (g.resid && g.batch != 1) return hipErrorInvalidValue;
  if (g.c_bf16_only && (!g.Cbf || g.beta != 0.f)) return hipErrorInvalidValue;
  hipError_t ge;
  if (gemv(g, workspace, ws_bytes, s, &ge)) return ge;
  if (g.post != POST_NONE || g.a_part || g.att_acc) return hipErrorInvalidValue;  // the inference fusions are few-row only
  int kps;
  bool small;
  const int dsp = dma_plan(g, &kps, &small);
  if (dsp > 0 && (dsp == 1 || (size_t)dsp * g.M * g.N * sizeof(float) <= ws_bytes)) {
    const hipError_t e = launch_dma(g, dsp, kps, static_cast<float*>(workspace), small, s);
    if (e != hipSuccess || dsp == 1) return e;
    return reduce_splits(g, static_cast<const float*>(workspace), dsp, s);
  }
  // K == 0 needs no special case: the k loop is empty and the epilogue writes beta*C + bias
  Plan p = make_plan(g);
  if (p.splits > 1 && (size_t)p.splits * g.batch * g.M * g.N * sizeof(float) > ws_bytes) p.splits = 1;
  if (p.splits == 1) p.k_per_split = ((std::max(g.K, 1) + KALIGN - 1) / KALIGN) * KALIGN;
  KArgs ka;
  ka.g = g;
  ka.splits = p.splits;
  ka.k_per_split = p.k_per_split;
  ka.ws = static_cast<float*>(workspace);
  ka.tiles_m = (g.M + p.BM - 1) / p.BM;
  ka.tiles_n = (g.N + p.BN - 1) / p.BN;
  // a tall, narrow product (the LM-head dW: 393 x 6 tiles, K = 8192) re-reads its
  // narrow operand once per group: longer groups (measured 1105 -> 1054 us at 16);
  // the 8192-row products 18-24 tiles wide (qkv and fc forward, the MLP's second dX)
  // run 6-10% faster with groups of 2 (the LM-head forward, 393 wide, is slower so)
  ka.group_m = ka.tiles_n <= 8 && ka.tiles_m >= 256                     ? GEMM_GROUP_TALL
               : ka.tiles_m >= 32 && ka.tiles_n >= 16 && ka.tiles_n <= 32 ? GEMM_GROUP_WIDE
                                                                          : GEMM_GROUP_M;
  dim3 grid(ka.tiles_m * ka.tiles_n * g.batch * p.splits);
  hipError_t e;
  if (p.cfg == CFG_128x128)
    e = launch_prec<2, 2, 2, 2>(ka, p.bk, grid, s);
  else if (p.cfg == CFG_256x128)
    e = launch_prec<2, 2, 4, 2>(ka, 32, grid, s);
  else if (p.cfg == CFG_128x192)
    e = launch_layout<2, 2, 2, 3, 64, true, true, true>(ka, grid, s);
  else
    e = launch_prec<4, 1, 1, 2>(ka, p.bk, grid, s);
  if (e != hipSuccess || p.splits == 1) return e;
  return reduce_splits(g, ka.ws, p.splits, s);
}

}  // namespace tfb
