// Internal interface between the host runtime (tfb_runtime.cpp) and the HIP
// kernels.  Every launcher enqueues on the given stream and returns the launch
// status; shape checks are the runtime's job.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace tfb {

// Kernel timing for the runtime's profiler.  While `stop` is set (per host
// thread, by the runtime around one family's launches), tfb::run_kernel attaches
// the events to the dispatches themselves: `start` to the first launch, `stop`
// to every launch (the last one's end counts), so the elapsed time is that of
// the kernels alone, without the gaps an event recorded on the stream adds.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  int launches = 0;
};
LaunchEvents& launch_events();

template <typename F, typename... Args>
inline void run_kernel(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args) {
  LaunchEvents& ev = launch_events();
  if (ev.stop) {
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, ev.launches == 0 ? ev.start : nullptr, ev.stop, 0u,
                          args...);
    ev.launches++;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
  }
}

enum Prec { PREC_F32 = 0, PREC_BF16 = 1 };

// Causal masks applied to the A operand while it is staged:
//   CAUSAL_UPTO: A(m, k) = 0 for k > m  (P @ V, dS @ K: a query row sees keys <= itself)
//   CAUSAL_FROM: A(m, k) = 0 for k < m  (P^T @ dO, dS^T @ Q: a key column gets queries >= itself)
enum CausalA { CAUSAL_NONE = 0, CAUSAL_UPTO = 1, CAUSAL_FROM = 2 };

// C = alpha * op(A) op(B) + beta * C (+ bias[n]), batched.
//   A(m, k) = a_mcontig ? A[k*lda + m] : A[m*lda + k]
//   B(k, n) = b_kcontig ? B[n*ldb + k] : B[k*ldb + n]
//   C(m, n) = C[m*ldc + n]
// Batch entry z (0 <= z < batch) uses z1 = z / batch_div, z2 = z % batch_div and
// offsets A + z1*sa1 + z2*sa2 (likewise B, C): a [B, H] head split folds into
// the addressing.  causal_out skips output tiles entirely above the diagonal.
struct GemmArgs {
  int M = 0, N = 0, K = 0;
  const float* A = nullptr;
  int64_t lda = 0;
  bool a_mcontig = false;
  const float* B = nullptr;
  int64_t ldb = 0;
  bool b_kcontig = false;
  float* C = nullptr;
  int64_t ldc = 0;
  float alpha = 1.f, beta = 0.f;
  const float* bias = nullptr;
  int batch = 1, batch_div = 1;
  int64_t sa1 = 0, sa2 = 0, sb1 = 0, sb2 = 0, sc1 = 0, sc2 = 0;
  int causal_a = CAUSAL_NONE;
  bool causal_out = false;
  int prec = PREC_F32;
  // bf16 storage of an operand (bf16 variant only): A/B then point at uint16 data
  bool a_bf16 = false, b_bf16 = false;
  // optional bf16 copy (round to nearest even) of the final C, same layout and ldc
  uint16_t* Cbf = nullptr;
  // optional residual added to the result, same layout and ldc as C (batch 1):
  // C = alpha A B + bias + beta C + resid
  const float* resid = nullptr;
  // with Cbf and beta == 0: the bf16 copy alone is written, C (fp32) is left untouched
  bool c_bf16_only = false;
  // Inference epilogues of the few-row path only (gemv.hip; gemm() refuses them
  // elsewhere with hipErrorInvalidValue):
  //   POST_GELU: C = gelu(alpha A B + bias) (no beta term, no residual)
  //   POST_LN:   C = alpha A B + bias + resid as usual, then each row of C is
  //              layer-normalised: ln_y = (C - mean) / sqrt(var + ln_eps) * ln_gamma
  //              + ln_beta (biased variance), written as fp32 (ln_y, may be null)
  //              and/or bf16 (ln_ybf, may be null); N <= 2048
  int post = 0;
  const float* ln_gamma = nullptr;
  const float* ln_beta = nullptr;
  float ln_eps = 0.f;
  float* ln_y = nullptr;
  uint16_t* ln_ybf = nullptr;
  //   POST_PARTIALS: only the per-chunk partial products are written, to the
  //              workspace as [chunks][M][N] (no bias, no C): the next few-row
  //              kernel sums them itself (gemv_chunks() gives their number)
  // A taken from such partials (few-row path only; A, lda, a_bf16 unused):
  //   A(m, k) = gelu(sum over the a_chunks chunks, in order, of a_part[c][m][k] +
  //   a_bias[k]), the previous product's GELU epilogue, rounded to bf16 in the bf16
  //   variant -- the values that product would have stored with TFB_OUT_BF16_ONLY
  const float* a_part = nullptr;
  const float* a_bias = nullptr;
  int a_chunks = 0;
  // A taken from the cached attention's per-block results (few-row path only; A,
  // lda, a_bf16 unused; K = att_heads * att_hs): for column k of row m, head
  // hd = k / att_hs, d = k % att_hs, bh = m * att_heads + hd and blocks s < att_blocks,
  //   A(m, k) = sum_s e^(M_s - M) acc_s[d] / sum_s e^(M_s - M) l_s,  M = max_s M_s,
  // with (M_s, l_s) = att_ml[(bh * att_blocks + s) * 2 + {0, 1}] and acc_s[d] =
  // att_acc[(bh * att_blocks + s) * att_hs + d] -- the merge kv_attend would have
  // stored, in the same order, rounded to bf16 in the bf16 variant
  const float* att_acc = nullptr;
  const float* att_ml = nullptr;
  int att_blocks = 0, att_hs = 0, att_heads = 0;
};
enum GemmPost { POST_NONE = 0, POST_GELU = 1, POST_LN = 2, POST_PARTIALS = 3 };

size_t gemm_workspace_bytes(const GemmArgs& g);
hipError_t gemm(const GemmArgs& g, void* workspace, size_t ws_bytes, hipStream_t s);

// Products of at most 16 rows, A [M, K] and B [K, N] row-major (gemv.hip), taken
// by gemm() when the layout fits; returns false (launching nothing) otherwise
size_t gemv_workspace_bytes(const GemmArgs& g);
bool gemv(const GemmArgs& g, void* ws, size_t ws_bytes, hipStream_t s, hipError_t* err);
// whether gemv() takes this product (alignment, sizes); a product with an inference
// epilogue (g.post) must be taken by it
bool gemv_accepts(const GemmArgs& g);
int gemv_chunks(const GemmArgs& g);

// ---- elementwise (elementwise.hip); beta in {0, 1}: overwrite or accumulate
hipError_t fill(float* p, float v, int64_t n, hipStream_t s);
// dst[i] = bf16(src[i]), round to nearest even
hipError_t to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s);
// dst[i] = the float value of the bf16 bits src[i] (exact)
hipError_t to_f32(const uint16_t* src, float* dst, int64_t n, hipStream_t s);
hipError_t add_bcast(const float* a, const float* b, float* y, int64_t n, int64_t nb, hipStream_t s);
hipError_t axpby(float* dst, const float* src, float alpha, float beta, int64_t n, hipStream_t s);
// Several independent dst = src + beta * dst (beta 0: dst = src) in one launch; the
// destinations must be pairwise distinct (the jobs run concurrently)
constexpr int AXPBY_BATCH = 64;
struct AxpbyJob {
  float* dst;
  const float* src;
  int64_t n;
  float beta;
};
struct AxpbyJobs {
  AxpbyJob j[AXPBY_BATCH];
  int count = 0;
};
hipError_t axpby_batch(const AxpbyJobs& jobs, hipStream_t s);
// The second stage of a column reduction (LayerNorm parameter gradients, column sums
// of a gradient), described instead of launched where a caller passes a ReduceJob*:
// the caller then runs it later, batched with others (reduce_batch), each job with the
// same arithmetic as the one-at-a-time launch.  Outputs of one batch must be distinct.
enum { REDUCE_LN = 1, REDUCE_COLSUM = 2 };
struct ReduceJob {
  int kind = 0;
  const float* part = nullptr;  // slab partials (kept alive by the caller until the batch runs)
  int nparts = 0, np = 1;       // slabs; planes per slab (REDUCE_LN)
  int64_t cols = 0;
  float* out[3] = {nullptr, nullptr, nullptr};  // LN: dgamma, dbeta, dx column sums (optional)
  float beta[3] = {0.f, 0.f, 0.f};
};
constexpr int REDUCE_BATCH = 32;
struct ReduceJobs {
  ReduceJob j[REDUCE_BATCH];
  int count = 0;
};
hipError_t reduce_batch(const ReduceJobs& jobs, hipStream_t s);
// dst[r*ldd + c] = src[r*lds + c] (+ dst when beta == 1), c < cols
hipError_t copy_pitched(const float* src, int64_t lds, float* dst, int64_t ldd, int64_t rows, int64_t cols,
                        float beta, hipStream_t s);
hipError_t mul_fwd(const float* a, const float* b, float* y, int64_t n, hipStream_t s);
hipError_t mul_bwd(const float* g, const float* other, float* d, float beta, int64_t n, hipStream_t s);
hipError_t scale_fwd(const float* a, float sc, float* y, int64_t n, hipStream_t s);
hipError_t tanh_fwd(const float* a, float* y, int64_t n, hipStream_t s);
hipError_t tanh_bwd(const float* g, const float* y, float* d, float beta, int64_t n, hipStream_t s);
// Producers of contraction operands take an optional `*bf` pointer: when it is
// non-null they also write the bf16 (round-to-nearest-even) copy of what they
// store, in the same layout, sparing a separate conversion pass.
hipError_t gelu_fwd(const float* a, float* y, uint16_t* ybf, int64_t n, hipStream_t s);
hipError_t gelu_bwd(const float* g, const float* x, float* d, uint16_t* dbf, float beta, int64_t n, hipStream_t s);
// the same over [rows, cols], also writing dcol[c] = sum over rows of the result
// where the row-slab path runs (*dcol_written); ws: colsum_workspace_bytes(rows, cols)
// xbf (optional): x given as its bf16 copy instead; gbf (optional): g given as bf16
// instead; d may be null with dbf given and beta == 0 (the bf16 copy alone).  These
// need the row-slab path: hipErrorInvalidValue where it does not fit (gelu_bwd_cols_fits)
hipError_t gelu_bwd_cols(const float* g, const float* x, float* d, uint16_t* dbf, float beta, int64_t rows,
                         int64_t cols, float* dcol, void* ws, hipStream_t s, bool* dcol_written,
                         const uint16_t* xbf = nullptr, const uint16_t* gbf = nullptr, ReduceJob* defer = nullptr);
bool gelu_bwd_cols_fits(const float* g, const void* x, const float* d, const uint16_t* dbf, int64_t rows,
                        int64_t cols, const void* ws);
// gelu_fwd reading the input's bf16 copy
hipError_t gelu_fwd_bf(const uint16_t* a, float* y, uint16_t* ybf, int64_t n, hipStream_t s);
// out[c] = beta*out[c] + sum_r g[r*cols + c]; deterministic two-stage reduction.
// gbf (optional, g then unused): the gradient held as bf16 (cols % 4 == 0, else
// hipErrorInvalidValue)
size_t colsum_workspace_bytes(int64_t rows, int64_t cols);
hipError_t colsum(const float* g, int64_t rows, int64_t cols, float* out, float beta, void* ws, hipStream_t s,
                  const uint16_t* gbf = nullptr, ReduceJob* defer = nullptr);
// out[0] = sum of a (deterministic); sum_bwd: d = beta*d + g[0]
size_t sum_workspace_bytes(int64_t n);
hipError_t sum_all(const float* a, int64_t n, float* out, void* ws, hipStream_t s);
hipError_t bcast_scalar_bwd(const float* g_scalar, float* d, float beta, int64_t n, hipStream_t s);
// last-dim slice copy and its inverse (the inverse writes zeros outside the slice when beta == 0)
hipError_t narrow_fwd(const float* x, float* y, int64_t rows, int64_t cols, int64_t start, int64_t len,
                      hipStream_t s);
hipError_t narrow_bwd(const float* g, float* d, int64_t rows, int64_t cols, int64_t start, int64_t len,
                      float beta, hipStream_t s);
// [B, T, H, hs] <-> [B, H, T, hs]; to_heads selects the direction
hipError_t permute_heads(const float* x, float* y, int64_t B, int64_t T, int64_t H, int64_t hs, bool to_heads,
                         float beta, hipStream_t s);

// ---- row reductions (rowops.hip)
hipError_t layernorm_fwd(const float* x, const float* gamma, const float* beta, float* y, uint16_t* ybf, float* mean,
                         float* rstd, int64_t rows, int64_t C, float eps, hipStream_t s);
size_t layernorm_bwd_workspace_bytes(int64_t rows, int64_t C);
// dxbf (optional) receives the bf16 copy of the final dx.  With beta_dx != 0 the
// earlier gradient is read from dx_src (null: dx itself) and the sum written to dx.
// dxsum (optional, [C]) receives the column sums of the final dx where the fused
// path runs; *dxsum_written says whether it did.  gbf (optional, g then unused): the
// upstream gradient held as bf16, read by the fused path only (hipErrorInvalidValue
// where layernorm_bwd_bf16_fits is false; gamma, dx_src and the workspace must then
// be 16-byte aligned as well)
bool layernorm_bwd_bf16_fits(const float* x, const float* dx, const uint16_t* gbf, int64_t rows, int64_t C);
hipError_t layernorm_bwd(const float* g, const float* x, const float* gamma, const float* mean, const float* rstd,
                         float* dx, const float* dx_src, uint16_t* dxbf, float* dgamma, float* dbeta, int64_t rows,
                         int64_t C, float beta_dx, float beta_dg, float beta_db, void* ws, hipStream_t s,
                         float* dxsum = nullptr, bool* dxsum_written = nullptr, const uint16_t* gbf = nullptr,
                         ReduceJob* defer = nullptr);
// full == true: every element of the [rows, T] view is written (zeros where masked);
// full == false: only the visible prefix of each row is touched.
hipError_t causal_softmax_fwd(const float* x, float* p, int64_t rows, int64_t T, bool full, hipStream_t s);
hipError_t causal_softmax_bwd(const float* g, const float* p, float* d, int64_t rows, int64_t T, float scale,
                              float beta, bool full, hipStream_t s);
size_t softmax_ce_workspace_bytes(int64_t rows);
// logits rows have V valid columns at a row stride of ld >= V.  dlbf (optional):
// the bf16 gradient of the logits for an upstream gradient of 1 is also written
// there, in softmax_ce_bwd's expression, where the one-pass path runs
// (*dlbf_written says whether it did).  logits_bf (optional, logits then unused):
// the logits stored as bf16, read by the one-pass kernel (hipErrorInvalidValue
// where softmax_ce_bf16_fits is false); dlbf may be null then
bool softmax_ce_bf16_fits(int64_t ld, int64_t V, const uint16_t* logits_bf);
hipError_t softmax_ce_fwd(const float* logits, int64_t ld, const int32_t* targets, int64_t rows, int64_t V,
                          float* lse, float* loss, void* ws, hipStream_t s, uint16_t* dlbf = nullptr,
                          bool* dlbf_written = nullptr, const uint16_t* logits_bf = nullptr);
// dl may be null when dlbf is given (and beta == 0): only the bf16 copy is written.
// skip_if_unit: nothing is done when g_scalar[0] == 1 (checked on the device): the
// forward already wrote that gradient into dlbf.  logits_bf: as in softmax_ce_fwd.
hipError_t softmax_ce_bwd(const float* logits, int64_t ld, const int32_t* targets, const float* lse,
                          const float* g_scalar, float* dl, uint16_t* dlbf, int64_t rows, int64_t V, float beta,
                          hipStream_t s, bool skip_if_unit = false, const uint16_t* logits_bf = nullptr);

// ---- fused causal attention, bf16 variant (attention.hip)
// qkv: bf16 [B, T, 3C] (q | k | v thirds, head h = columns h*hs .. h*hs+hs-1 of each third)
// y: fp32 [B, T, C] (null: only its bf16 copy ybf is written); lse: [B*H, T] base-2
// log-sum-exp of the scaled scores (saved for backward)
bool flash_attention_supported(int hs, int64_t C, int64_t T);
hipError_t flash_attention_fwd(const uint16_t* qkv, float* y, uint16_t* ybf, float* lse, int B, int T, int H, int C,
                               float scale, hipStream_t s);
// dqkv = beta*dqkv + d(qkv) (dqkv null with beta 0: the bf16 copy alone); D: [B*H, T]
// scratch, rowsum(dy * y) from y and dyf, or from ybf and dy where either is null
hipError_t flash_attention_bwd(const uint16_t* qkv, const float* y, const float* dyf, const uint16_t* dy,
                               const float* lse, float* D, float* dqkv, uint16_t* dqkv_bf, float beta, int B, int T,
                               int H, int C, float scale, hipStream_t s, const uint16_t* ybf = nullptr);

// ---- KV-cached inference (decode.hip); cache [L][2][B][Tmax][C], fp32 or (kv_bf16) bf16
hipError_t kv_store(const float* qkv, int64_t T, int C, void* kv, bool kv_bf16, int layer, int B, int Tmax, int pos0,
                    hipStream_t s);
// ws: kv_attend_workspace_bytes(B, C, H, pos) bytes of scratch (partial results per block of positions)
size_t kv_attend_workspace_bytes(int B, int C, int H, int pos);
// qkv_part (optional; qkv then unused): qkv is the sum over qkv_chunks chunks of
// qkv_part[c][B][3C] plus qkv_bias, the partials of the few-row c_attn product
// (POST_PARTIALS); taken only where kv_attend_takes_parts(C, H)
bool kv_attend_takes_parts(int C, int H);
// y null (only where kv_attend_takes_parts(C, H), with ws): the attention stops at
// its per-block results, which stay in ws as acc [B*H][S][C/H] then (M, l) [B*H][S][2]
// with S = kv_attend_blocks(kv_bf16, pos); a few-row product merges them as it loads
// them (GemmArgs::att_acc)
int kv_attend_blocks(bool kv_bf16, int pos);
hipError_t kv_attend(const float* qkv, void* kv, bool kv_bf16, float* y, int layer, int B, int Tmax, int C, int H,
                     int pos, float scale, void* ws, hipStream_t s, const float* qkv_part = nullptr, int qkv_chunks = 0,
                     const float* qkv_bias = nullptr);
hipError_t sample_topk(const float* logits, int64_t ld, int B, int V, int k, float temperature, const double* u,
                       int32_t* out, hipStream_t s);

// ---- embedding (embedding.hip)
// ids outside [0, rows) give zero rows forward and are skipped backward
hipError_t embedding_fwd(const float* table, int64_t rows, const int32_t* ids, float* y, int64_t n, int64_t C,
                         hipStream_t s);
size_t embedding_bwd_workspace_bytes(int64_t n);
// dtable[ids[r]] += g[r] for every r; sums per table row in ascending r order
hipError_t embedding_bwd(const float* g, const int32_t* ids, int64_t n, int64_t C, float* dtable, int64_t rows,
                         void* ws, hipStream_t s);

// ---- optimizers (optim.hip)
struct AdamSeg {
  float* p;
  const float* g;
  float* m;
  float* v;
  uint16_t* pbf;  // bf16 copy of p refreshed by the step, or null
  int64_t n;
  float wd;
  int pad;
};
struct AdamChunk {
  int seg;
  int pad;
  int64_t off;
};
hipError_t adamw_step(const AdamSeg* segs, const AdamChunk* chunks, int nchunks, int64_t chunk_elems, float lr,
                      float b1, float b2, float eps, float bc1, float bc2, hipStream_t s);
hipError_t sgd_step(float* p, const float* g, float lr, int64_t n, hipStream_t s);

// ---- runtime (tfb_runtime.cpp): sets the calling thread's tfb_last_error text, returns code
int set_last_error(int code, const char* msg);

}  // namespace tfb
