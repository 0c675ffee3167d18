/*
 * tfb.h -- C ABI of the MI355X (gfx950) tensor-autograd hot path.
 *
 * The operations are those of the tensor autograd engine described in
 *   [Autograd-1] arabroot.io, "Build a language model in C# from scratch (1):
 *                the Autograd engine"
 *   [GPT2-4]     arabroot.io, "Build a language model in C# from scratch (4):
 *                running the GPT-2 weights"
 * Each forward call computes its output on the GPU and, unless gradients are
 * disabled, records one entry on the context's tape; tfb_backward replays the
 * entries' backward rules in reverse order.
 *
 * Conventions
 *  - Every function returns 0 (TFB_OK) or a negative TFB_ERR_* code.  The text
 *    of the last error of the calling thread is available from tfb_last_error().
 *    Argument and shape checks happen on the host before anything is enqueued;
 *    a failed call enqueues nothing and leaves the context usable.
 *  - All work is enqueued asynchronously on the HIP stream given to tfb_init.
 *    GPU faults surface as TFB_ERR_HIP from tfb_sync or a later call.
 *  - Tensors are float32, row-major, contiguous.  A tensor's "rows" are the
 *    product of all dimensions but the last ([Autograd-1, "The Tensor class"]).
 *  - Pointers named dev_* are device pointers; host_* are host pointers.
 *  - Handles (tfb_tensor) are small non-negative integers owned by the context.
 *
 * Memory
 *  - The caller gives tfb_init one device buffer (the arena).  The library never
 *    calls hipMalloc for tensors: persistent allocations (parameters created with
 *    dev_ptr == NULL, parameter gradients, optimizer moments) grow from the low
 *    end, per-step allocations (op outputs, saved tensors, non-leaf gradients,
 *    scratch) from the high end.  Exhaustion returns TFB_ERR_OOM.
 *  - Op outputs and everything the tape saved are valid until tfb_tape_reset.
 */
#ifndef TFB_H
#define TFB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tfb_ctx tfb_ctx;
typedef struct tfb_opt tfb_opt;
typedef int32_t tfb_tensor;

#define TFB_OK 0
#define TFB_ERR_ARG (-1)    /* bad argument: null pointer, unknown handle, bad enum */
#define TFB_ERR_SHAPE (-2)  /* shapes do not fit the op */
#define TFB_ERR_STATE (-3)  /* e.g. backward from a non-scalar, released tensor in use */
#define TFB_ERR_OOM (-4)    /* arena exhausted */
#define TFB_ERR_HIP (-5)    /* a HIP runtime call failed */

/* Arithmetic of the contractions (MatMul family and the attention products). */
#define TFB_FP32 0       /* fp32 operands, fp32 MFMA, fp32 accumulation */
#define TFB_BF16_MFMA 1  /* operands rounded to bf16 (nearest-even), fp32 accumulation;
                            every other op and all stored tensors stay fp32 */

#define TFB_MAX_DIMS 6
#define TFB_MAX_NAME 128  /* a tensor name is kept up to 127 bytes */

/* ---------------------------------------------------------------- context */

/* Create a context on `device` that enqueues on `hip_stream` (a hipStream_t;
 * NULL = the null stream) and sub-allocates from [arena, arena + arena_bytes)
 * (device memory owned by the caller, at least 256-byte aligned).  The context
 * holds what the pages keep in the Tensor objects and the graph they link:
 * every tensor's data and gradient, and the recorded backward rules
 * ([Autograd-1, "The Tensor class"; "How each op records itself in the
 * graph"]).  precision: TFB_FP32 or TFB_BF16_MFMA.  Errors: TFB_ERR_ARG for a
 * null out/arena, an unknown precision or a missing device. */
int tfb_init(tfb_ctx** out, int device, void* hip_stream, void* arena, size_t arena_bytes, int precision);
/* Destroy the context and every handle it owns; the arena itself stays the
 * caller's.  Work still queued on the stream must not be running after this
 * returns, so it synchronises first.  (The pages' objects are garbage
 * collected; here the owner ends them: [Autograd-1, "The Tensor class"].) */
int tfb_destroy(tfb_ctx* ctx);
/* Text of the calling thread's last error (valid until its next call): the
 * counterpart of the pages' exception messages, e.g. the shape message of
 * MatMul or "Backward() starts from a scalar loss" ([Autograd-1, "Ops";
 * "How each op records itself in the graph"]).  Never NULL. */
const char* tfb_last_error(void);
/* Switch the contraction arithmetic for ops recorded from now on (TFB_FP32 or
 * TFB_BF16_MFMA).  The pages compute in float ([Autograd-1, "Why fast
 * MatMul"]); the bf16 variant rounds the contraction operands only. */
int tfb_set_precision(tfb_ctx* ctx, int precision);
/* Inference mode: with enabled == 0 ops record nothing ([Autograd-1, "The
 * Tensor class": the NoGrad flag]).  Per context. */
int tfb_set_grad_enabled(tfb_ctx* ctx, int enabled);
/* Wait for all enqueued work; returns TFB_ERR_HIP if any of it failed.  The
 * pages' calls return finished values ([Autograd-1, "The Tensor class"]);
 * here results are final once this returns (tfb_tensor_read also waits). */
int tfb_sync(tfb_ctx* ctx);
/* Bytes in use at the low (persistent) and high (step) ends of the arena
 * (the persistent figure includes ranges given back below its top that later
 * persistent allocations reuse).  Either pointer may be NULL.  Memory
 * bookkeeping of the tensors the pages allocate per op ([Autograd-1, "The
 * Tensor class": Grad created on demand]). */
int tfb_arena_usage(tfb_ctx* ctx, size_t* persistent, size_t* step);

/* ---------------------------------------------------------------- tensors */

/* A leaf tensor ([Autograd-1, "The Tensor class": op "leaf", flat row-major
 * Data with a Shape, and a Name for parameters]).  shape: ndim (1..6)
 * positive sizes.  With dev_ptr != NULL the tensor borrows that device memory
 * (the caller keeps it alive and 256-byte aligned); with NULL it is allocated
 * in the persistent arena and zero-filled.  is_param marks optimizer
 * parameters (informational).  name: NULL or a NUL-terminated string, copied
 * (up to TFB_MAX_NAME - 1 bytes); it appears in shape error messages.
 * Errors: TFB_ERR_SHAPE (bad rank or size), TFB_ERR_ARG (misaligned dev_ptr),
 * TFB_ERR_OOM. */
int tfb_tensor_create(tfb_ctx* ctx, const int64_t* shape, int ndim, void* dev_ptr, int is_param, const char* name,
                      tfb_tensor* out);
/* The tensor's name, NUL-terminated, truncated to cap - 1 bytes (empty for op
 * outputs and unnamed leaves).  [Autograd-1, "The Tensor class": Name] */
int tfb_tensor_name(tfb_ctx* ctx, tfb_tensor t, char* buf, size_t cap);
/* Shape, rank and device pointers of a tensor; *grad is NULL while the tensor
 * has no gradient buffer ([Autograd-1, "The Tensor class": Grad is created on
 * demand]).  Any output pointer may be NULL.  The pointers stay owned by the
 * context. */
int tfb_tensor_info(tfb_ctx* ctx, tfb_tensor t, int64_t* shape, int* ndim, void** data, void** grad);
/* Copy n floats (n == the tensor's size, else TFB_ERR_SHAPE) between host
 * memory and the tensor's Data (which == 0) or Grad (which == 1; reading a
 * gradient that was cleared returns zeros, reading one that never existed or
 * that is kept only as bf16 is TFB_ERR_STATE).  Synchronous: the read waits
 * for the work queued before it.  [Autograd-1, "The Tensor class": Data and
 * Grad, same size] */
int tfb_tensor_write(tfb_ctx* ctx, tfb_tensor t, const float* host_src, int64_t n);
int tfb_tensor_read(tfb_ctx* ctx, tfb_tensor t, int which, float* host_dst, int64_t n);
/* Release a leaf tensor (TFB_ERR_STATE while the tape still references it).
 * Op outputs are released by tfb_tape_reset.  [Autograd-1, "The Tensor
 * class"] */
int tfb_tensor_release(tfb_ctx* ctx, tfb_tensor t);

/* ---------------------------------------------------------------- ops
 * Each op writes its new output handle to *y.  Backward rules add into the
 * inputs' gradients ([Autograd-1, "Why += and not ="]). */

/* y = a + b; b equals the trailing dims of a (bias broadcast); db sums over the
 * leading dims.  [Autograd-1, table of ops: Add with broadcast] */
int tfb_add(tfb_ctx* ctx, tfb_tensor a, tfb_tensor b, tfb_tensor* y);
/* y = a * b elementwise; sizes must match.  [Autograd-1, "Ops": Mul] */
int tfb_mul(tfb_ctx* ctx, tfb_tensor a, tfb_tensor b, tfb_tensor* y);
/* y = s * a.  [Autograd-1, table of ops: Scale] */
int tfb_scale(tfb_ctx* ctx, tfb_tensor a, float s, tfb_tensor* y);
/* y[0] = sum of all elements of a.  [Autograd-1, table of ops: Sum] */
int tfb_sum(tfb_ctx* ctx, tfb_tensor a, tfb_tensor* y);
/* Same data, new shape of equal size.  [Autograd-1, table of ops: Reshape] */
int tfb_reshape(tfb_ctx* ctx, tfb_tensor a, const int64_t* shape, int ndim, tfb_tensor* y);
/* y = tanh(a); backward g(1 - y^2).  [Autograd-1, table of ops: Tanh] */
int tfb_tanh(tfb_ctx* ctx, tfb_tensor a, tfb_tensor* y);
/* y = 0.5 a (1 + tanh(sqrt(2/pi)(a + 0.044715 a^3))), GPT-2's tanh form.
 * [GPT2-4, "Common mistakes"] */
int tfb_gelu(tfb_ctx* ctx, tfb_tensor a, tfb_tensor* y);
/* tfb_gelu with flags (TFB_OUT_BF16_ONLY; unknown flags: TFB_ERR_ARG).
 * [GPT2-4, "Common mistakes"] */
int tfb_gelu_ex(tfb_ctx* ctx, tfb_tensor a, int flags, tfb_tensor* y);
/* y = x[..., K] @ w[K, M] (rows of x flattened).  Backward dx = g w^T,
 * dw = x^T g.  [Autograd-1, "Ops": MatMul] */
int tfb_matmul(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, tfb_tensor* y);
/* y = x[..., C] @ w[V, C]^T, the weight-tied LM head.  Backward dx = g w,
 * dw = g^T x.  [GPT2-4, "Loading the weights": weight tying] */
int tfb_matmul_t(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, tfb_tensor* y);
/* tfb_matmul_t with flags (TFB_OUT_BF16_COPY, TFB_OUT_BF16_ONLY below; unknown
 * flags: TFB_ERR_ARG).  With TFB_OUT_BF16_ONLY the logits are stored as bf16
 * alone and tfb_softmax_cross_entropy reads them as such. */
int tfb_matmul_t_ex(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, int flags, tfb_tensor* y);
/* y = x @ w + b as one op (MatMul followed by the bias Add, fused into the
 * contraction's epilogue); w is [in, out] as GPT-2 stores it.
 * [GPT2-4, "Loading the weights": Linear weights stored [in, out]] */
int tfb_linear(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, tfb_tensor b, tfb_tensor* y);
/* tfb_linear with flags.  TFB_OUT_BF16_COPY: in the bf16 variant the product's
 * epilogue also writes the bf16 copy of y that bf16 consumers (the contraction
 * and attention kernels) read, sparing them a conversion pass; it changes no
 * value and is ignored in the fp32 variant.  Unknown flags: TFB_ERR_ARG.
 * [GPT2-4, "Loading the weights": Linear weights stored [in, out]] */
#define TFB_OUT_BF16_COPY 1
/* Output flag of tfb_linear_ex, tfb_matmul_t_ex, tfb_layernorm_ex, tfb_gelu_ex and tfb_causal_attention_ex (bf16 variant):
 * only the bf16 copy of y is written, for an output whose readers take bf16
 * (the contractions, the fused attention).  A reader that needs fp32 data (any
 * other op, tfb_tensor_read, tfb_tensor_info) gets the exact float values of
 * those bf16 numbers, converted on first use.  In the backward, where y's
 * gradient has one contribution and its only reader takes bf16 (the contraction
 * that produced y, with column sums for the bias gradient, or the GELU or fused
 * attention that produced y), that gradient too may be written only as bf16;
 * reading it then gives TFB_ERR_STATE.  Ignored in the fp32 variant. */
#define TFB_OUT_BF16_ONLY 2
/* y = r + (x @ w + b): a Linear and the residual Add that follows it, with the
 * Add done in the product's epilogue (r is read there, once).  r has the
 * output's shape [rows(x), cols(w)].  One op on the tape; its backward gives r
 * the output's gradient and x, w, b the Linear's gradients.
 * [Autograd-1, "Ops": MatMul, the bias Add and Add; GPT2-4, "Loading the
 * weights": the residual stream x = x + attn(ln_1(x)), x = x + mlp(ln_2(x))] */
int tfb_linear_residual(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, tfb_tensor b, tfb_tensor r, tfb_tensor* y);
/* tfb_linear with flags (TFB_OUT_BF16_COPY, TFB_OUT_BF16_ONLY above).
 * [GPT2-4, "Loading the weights": Linear weights stored [in, out]] */
int tfb_linear_ex(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, tfb_tensor b, int flags, tfb_tensor* y);
/* Inference only (gradients disabled, else TFB_ERR_STATE; nothing is recorded):
 * y = gelu(x @ w + b), the Linear and the GELU that follows it in GPT-2's MLP, as one
 * call.  In a product of at most 16 rows (a decode step) the GELU is applied where
 * the few-row kernel sums its partial products, so no separate pass reads and
 * writes the product; otherwise it runs as tfb_linear_ex then tfb_gelu_ex.  Flags:
 * TFB_OUT_BF16_ONLY (y kept as bf16 alone, bf16 variant).
 * [GPT2-4, "Loading the weights": the MLP c_fc then GELU; "Common mistakes"] */
int tfb_linear_gelu(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, tfb_tensor b, int flags, tfb_tensor* y);
/* Inference only (as above): y = r + (x @ w + b) and h = LayerNorm(y) with gamma,
 * beta, eps (biased variance) -- a block's projection with its residual Add and the
 * LayerNorm that reads the result next (the following block's ln_1, or ln_f), as
 * one call.  In a product of at most 16 rows the few-row kernel's chunk sum adds
 * bias and residual and normalises each row; otherwise it runs as
 * tfb_linear_residual then tfb_layernorm_ex.  y [rows, N] fp32; h the same shape
 * (TFB_OUT_BF16_ONLY: bf16 alone in the bf16 variant); N <= 2048.
 * [GPT2-4, "Loading the weights": x = x + attn(ln_1(x)), x = x + mlp(ln_2(x));
 * Autograd-1, table of ops: LayerNorm] */
int tfb_linear_residual_layernorm(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, tfb_tensor b, tfb_tensor r,
                                  tfb_tensor gamma, tfb_tensor beta, float eps, int flags, tfb_tensor* y,
                                  tfb_tensor* h);
/* Inference only (as above): a whole MLP sub-block of a pre-LN block and the
 * LayerNorm after it: y = r + gelu(x @ w_fc + b_fc) @ w_proj + b_proj and
 * h = LayerNorm(y) with gamma, beta, eps.  For at most 16 rows the c_fc product's
 * partial sums are read straight by the projection, which adds them with the bias
 * and applies the GELU as it loads its input (the values tfb_linear_gelu would
 * have stored, bf16 in the bf16 variant), so neither the hidden activation nor its
 * chunk sum is a pass of its own; otherwise tfb_linear_gelu then
 * tfb_linear_residual_layernorm.  Flags as there (TFB_OUT_BF16_ONLY for h).
 * [GPT2-4, "Loading the weights": x = x + mlp(ln_2(x)), MLP C -> 4C -> C] */
int tfb_mlp_residual_layernorm(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w_fc, tfb_tensor b_fc, tfb_tensor w_proj,
                               tfb_tensor b_proj, tfb_tensor r, tfb_tensor gamma, tfb_tensor beta, float eps, int flags,
                               tfb_tensor* y, tfb_tensor* h);
/* Per row over the last dim: (x - mean)/sqrt(var + eps) * gamma + beta with the
 * biased variance.  [Autograd-1, table of ops: LayerNorm] */
int tfb_layernorm(tfb_ctx* ctx, tfb_tensor x, tfb_tensor gamma, tfb_tensor beta, float eps, tfb_tensor* y);
/* tfb_layernorm with flags (TFB_OUT_BF16_ONLY; unknown flags: TFB_ERR_ARG).
 * [Autograd-1, table of ops: LayerNorm] */
int tfb_layernorm_ex(tfb_ctx* ctx, tfb_tensor x, tfb_tensor gamma, tfb_tensor beta, float eps, int flags,
                     tfb_tensor* y);
/* y[b, t, :] = table[ids[b*T + t], :], y shape [batch, n/batch, C]; backward
 * scatter-adds rows into table's gradient (sorted segment sum: deterministic).
 * dev_ids: n int32 device values in [0, rows(table)), copied by the call.
 * [Autograd-1, table of ops: Embedding; GPT2-4, "Generation with KV cache"] */
int tfb_embedding(tfb_ctx* ctx, tfb_tensor table, const int32_t* dev_ids, int64_t n, int64_t batch,
                  tfb_tensor* y);
/* Slice [start, start+len) of the last dim.  [Autograd-1, table of ops: Narrow] */
int tfb_narrow(tfb_ctx* ctx, tfb_tensor x, int64_t start, int64_t len, tfb_tensor* y);
/* [B, T, H*hs] -> [B, H, T, hs], head h = columns h*hs..h*hs+hs-1; and back.
 * [Autograd-1, table of ops: SplitHeads, MergeHeads] */
int tfb_split_heads(tfb_ctx* ctx, tfb_tensor x, int heads, tfb_tensor* y);
int tfb_merge_heads(tfb_ctx* ctx, tfb_tensor x, tfb_tensor* y);
/* a[Z, n, k] @ b[Z, k, m] and a[Z, n, k] @ b[Z, m, k]^T per batch entry.
 * [Autograd-1, table of ops: BatchMatMul, BatchMatMulT] */
int tfb_batch_matmul(tfb_ctx* ctx, tfb_tensor a, tfb_tensor b, tfb_tensor* y);
int tfb_batch_matmul_t(tfb_ctx* ctx, tfb_tensor a, tfb_tensor b, tfb_tensor* y);
/* Row r of the [rows, T] view sees columns j <= r mod T; softmax over those,
 * exact zeros elsewhere.  [GPT2-4, "The 12 unused tensors": the mask is
 * computed, visible = r % t + 1] */
int tfb_causal_softmax(tfb_ctx* ctx, tfb_tensor s, tfb_tensor* y);
/* The attention core as one tape entry: from qkv [B, T, 3C] (q, k, v = the
 * three column thirds, heads = hs-column slices) compute
 * y = MergeHeads(CausalSoftmax(q k^T / sqrt(hs)) v), y [B, T, C].  Same
 * arithmetic as Narrow/SplitHeads/BatchMatMulT/Scale/CausalSoftmax/
 * BatchMatMul/MergeHeads; the head split is folded into the products'
 * addressing and the masked upper triangle is never computed.
 * [Autograd-1, table of ops; GPT2-4, "Generation with KV cache"] */
int tfb_causal_attention(tfb_ctx* ctx, tfb_tensor qkv, int heads, tfb_tensor* y);
/* tfb_causal_attention with flags (TFB_OUT_BF16_ONLY, bf16 variant with the fused
 * kernels: y kept as bf16 alone; its backward then takes rowsum(dy * y) from the
 * bf16 copies.  Unknown flags: TFB_ERR_ARG). */
int tfb_causal_attention_ex(tfb_ctx* ctx, tfb_tensor qkv, int heads, int flags, tfb_tensor* y);
/* loss[0] = mean over rows of -log(max(softmax(logits_row)[target], 1e-30));
 * backward (g/n)(p - onehot).  dev_targets: n = rows(logits) int32 device
 * values in [0, cols), copied by the call.  [Autograd-1, "Ops":
 * SoftmaxCrossEntropy] */
int tfb_softmax_cross_entropy(tfb_ctx* ctx, tfb_tensor logits, const int32_t* dev_targets, int64_t n,
                              tfb_tensor* loss);
/* tfb_softmax_cross_entropy with flags.  TFB_CE_GRAD_BF16_ONLY (bf16 variant):
 * when the logits come from a contraction and nothing else reads them, their
 * gradient is written only as the bf16 copy that the contraction's backward
 * reads; the fp32 gradient of the logits is not kept (reading it gives
 * TFB_ERR_STATE).  Every other gradient is unchanged.  Ignored in the fp32
 * variant or when those conditions do not hold.  Unknown flags: TFB_ERR_ARG.
 * [Autograd-1, "Ops": SoftmaxCrossEntropy] */
#define TFB_CE_GRAD_BF16_ONLY 1
int tfb_softmax_cross_entropy_ex(tfb_ctx* ctx, tfb_tensor logits, const int32_t* dev_targets, int64_t n, int flags,
                                 tfb_tensor* loss);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the forward
 * of tfb_softmax_cross_entropy on plain device pointers, with no context and no
 * arena.  dev_loss[0] = mean over the rows of -log(max(softmax(row)[target],
 * 1e-30)) -- the same kernels and the same value as tfb_softmax_cross_entropy's
 * loss for fp32 logits.  dev_logits: rows x cols fp32 at a row stride of ld >=
 * cols floats; dev_targets: rows int32 in [0, cols) (an id outside gives a NaN
 * loss, never an access outside the row); all three device pointers are the
 * caller's.  Enqueued on hip_stream (a hipStream_t, NULL = the null stream) of
 * the current device.  Its scratch (2 * rows floats) is a fixed array on each
 * GPU the library runs on, held until the process ends: rows above
 * TFB_NOALLOC_MAX_ROWS give TFB_ERR_SHAPE, and calls that overlap on one GPU
 * (other streams or threads) race on it.  Calls no allocating routine.
 * Errors: TFB_ERR_ARG (null pointer), TFB_ERR_SHAPE (sizes), TFB_ERR_HIP. */
#define TFB_NOALLOC_MAX_ROWS 65536
int tfb_softmax_cross_entropy_noalloc(const float* dev_logits, int64_t ld, const int32_t* dev_targets, int64_t rows,
                                      int64_t cols, float* dev_loss, void* hip_stream);

/* ---------------------------------------------------------------- autograd */

/* [Autograd-1, "How each op records itself in the graph"]: loss must have one
 * element (else TFB_ERR_STATE); gradients of op outputs start at zero, the
 * loss's gradient is seeded with 1 and the recorded rules run from the last
 * entry to the first.  Leaf gradients keep accumulating across calls until
 * tfb_zero_grad. */
int tfb_backward(tfb_ctx* ctx, tfb_tensor loss);
/* Clear the gradients of the given leaf tensors ([Autograd-1, "The
 * Optimizer": ZeroGrad]).  Tensors that never had a gradient are skipped. */
int tfb_zero_grad(tfb_ctx* ctx, const tfb_tensor* params, int n);
/* End of step: drop the tape, release every op output and free the step end
 * of the arena.  The pages' graph is dropped with the loss tensor that roots
 * it ([Autograd-1, "How each op records itself in the graph": the graph is
 * the parents and backward fields of each output]); here it is dropped
 * explicitly.  Leaf tensors and their gradients are kept.  Work already queued
 * that reads the freed memory completes before later work reuses it. */
int tfb_tape_reset(tfb_ctx* ctx);

/* ---------------------------------------------------------------- optimizers */

/* AdamW ([Autograd-1, "The Optimizer": AdamW]): per step t += 1, bc1 = 1 -
 * beta1^t, bc2 = 1 - beta2^t; for every parameter that has a gradient,
 * m = b1 m + (1-b1) g, v = b2 v + (1-b2) g^2,
 * p -= lr * ((m/bc1) / (sqrt(v/bc2) + eps) + wd_k p) with wd_k = wd for
 * tensors of rank >= 2 and 0 otherwise.  m and v live in the persistent arena.
 * One fused launch updates all parameters. */
int tfb_adamw_create(tfb_ctx* ctx, const tfb_tensor* params, int n, float lr, float weight_decay, float beta1,
                     float beta2, float eps, tfb_opt** out);
/* One AdamW step over every parameter given at creation ([Autograd-1, "The
 * Optimizer": Step]). */
int tfb_adamw_step(tfb_opt* opt);
/* Change the learning rate of later steps ([Autograd-1, "The Optimizer": the
 * lr field]). */
int tfb_adamw_set_lr(tfb_opt* opt, float lr);
/* Read the moments m and v of parameter i (n floats each, n == its size;
 * NULL skips one).  Synchronous.  [Autograd-1, "The Optimizer": AdamW's m, v] */
int tfb_adamw_moments(tfb_opt* opt, int i, float* host_m, float* host_v, int64_t n);
/* Free the optimizer handle; its moments' arena memory stays reserved until the
 * context is destroyed.  [Autograd-1, "The Optimizer"] */
int tfb_adamw_destroy(tfb_opt* opt);
/* w -= lr * g for every given parameter that has a gradient.
 * [Autograd-1, "The Optimizer": SGD] */
int tfb_sgd_step(tfb_ctx* ctx, const tfb_tensor* params, int n, float lr);

/* ---------------------------------------------------------------- KV-cached inference
 * [GPT2-4, "Generation with KV cache"; "Temperature and Top-k"].  None of these
 * calls is recorded on the tape. */

typedef struct tfb_kv tfb_kv;
/* A key/value cache of `layers` x 2 x batch x tmax x channels values in the
 * persistent arena, zero-filled (tmax <= 16384): fp32, or bf16 (round to nearest
 * even) when the context is in the bf16 variant at creation -- keys and values are
 * operands of the q.k and p.v products, and the bf16 variant rounds every
 * contraction operand to bf16; the attention arithmetic stays fp32. */
int tfb_kv_create(tfb_ctx* ctx, int layers, int batch, int tmax, int channels, tfb_kv** out);
/* Frees the handle and gives the cache's arena memory back: to the top of the
 * persistent end when nothing was allocated there after it, otherwise as a hole
 * that later persistent allocations (the next cache, a parameter, a bf16 weight
 * copy) take first.  Queued work that reads the cache still completes before
 * later work on the stream reuses it.  [GPT2-4, "Generation with KV cache"] */
int tfb_kv_destroy(tfb_kv* kv);
/* Copy the keys and values (the second and third column thirds) of qkv
 * [batch, T, 3C] into positions pos0 .. pos0+T-1 of `layer` (a batched prompt). */
int tfb_kv_store(tfb_ctx* ctx, tfb_kv* kv, int layer, tfb_tensor qkv, int pos0);
/* One new token per sequence: qkv [batch, 1, 3C].  Appends its key and value at
 * `pos`, then y[b, 0, head slice] = sum_j softmax_j(q . k_j / sqrt(hs)) v_j over
 * positions 0..pos -- no mask, the cache holds only the past.  y [batch, 1, C]. */
int tfb_kv_attend(tfb_ctx* ctx, tfb_kv* kv, int layer, tfb_tensor qkv, int pos, int heads, tfb_tensor* y);
/* The c_attn Linear of one new token per sequence and tfb_kv_attend as one call:
 * qkv = x @ w + b with x [batch, 1, K] and w [K, 3C], then the append and the
 * single-query attention of tfb_kv_attend; y [batch, 1, C].  With gradients
 * disabled, at most 16 sequences and head size 32, 64 or 128 the attention kernel
 * sums the product's partials (plus the bias) as it reads q, k and v, so qkv is
 * never stored; otherwise it runs as tfb_linear then tfb_kv_attend.  Not recorded.
 * [GPT2-4, "Generation with KV cache"] */
int tfb_kv_attend_linear(tfb_ctx* ctx, tfb_kv* kv, int layer, tfb_tensor x, tfb_tensor w, tfb_tensor b, int pos,
                         int heads, tfb_tensor* y);
/* The attention half of a transformer block for one new token per sequence, as
 * one call: a = tfb_kv_attend_linear(x, w_attn, b_attn) (append at `pos`, then the
 * single-query attention), y = r + a @ w_proj + b_proj and h = LayerNorm(y; gamma,
 * beta, eps), y and h [batch, 1, N] with w_proj [C, N].  Inference only: gradients
 * enabled -> TFB_ERR_STATE; nothing recorded.  Where the fused kernels apply (at
 * most 16 sequences, head size 32, 64 or 128, N <= 2048 and a multiple of 4) the
 * attention leaves its per-block results and the projection merges them as it
 * loads its input, so `a` is never stored; otherwise it runs as
 * tfb_kv_attend_linear then tfb_linear_residual_layernorm.  Flags: as there
 * (TFB_OUT_BF16_ONLY for h).  Errors: as those two calls.
 * [GPT2-4, "Generation with KV cache"; "Loading the weights": x = x + attn(ln_1(x))] */
int tfb_kv_attention_block(tfb_ctx* ctx, tfb_kv* kv, int layer, tfb_tensor x, tfb_tensor w_attn, tfb_tensor b_attn,
                           int pos, int heads, tfb_tensor w_proj, tfb_tensor b_proj, tfb_tensor r, tfb_tensor gamma,
                           tfb_tensor beta, float eps, int flags, tfb_tensor* y, tfb_tensor* h);
/* One id per row of logits [..., V]: keep every logit >= the k-th largest (ties
 * kept; k = 0 or k >= V keeps all), p = softmax((l - max)/temperature) summed in
 * double, and return the first id (ascending) whose cumulative p exceeds u[row].
 * dev_uniforms: rows doubles in [0, 1); dev_out: rows int32 (device memory). */
int tfb_sample_topk(tfb_ctx* ctx, tfb_tensor logits, int k, float temperature, const double* dev_uniforms,
                    int32_t* dev_out);

/* ---------------------------------------------------------------- measurement */

/* Measurement of the pages' claim that matrix multiplication takes most of
 * the time ([Autograd-1, "Why fast MatMul"]) and that cached generation is
 * bound by memory ([GPT2-4, "Generation with KV cache"]).
 * Between begin and end, the launches of the kernel families below are each
 * bracketed by HIP events on the context's stream, and each family adds up the
 * algorithmic work of its launches: flops (2*M*N*K, causal
 * products counted over the needed triangle only) for the contractions, bytes
 * (each operand read once, each output written once, in the form it is stored)
 * for the others.  end() synchronises and returns the contraction family's
 * summed time in milliseconds, its flops and its launch count; after it,
 * tfb_profile_kind gives the same three figures for any family. */
#define TFB_PROF_GEMM 0       /* MatMul family (MFMA tiles), flops */
#define TFB_PROF_ATTN_FWD 1   /* fused causal attention forward: QK^T and PV, flops */
#define TFB_PROF_ATTN_BWD 2   /* fused attention backward (dQ and dK/dV kernels): the four
                                 products dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q, flops */
#define TFB_PROF_CE 3         /* SoftmaxCrossEntropy forward (with the fused gradient) and backward, bytes */
#define TFB_PROF_ADAMW 4      /* the fused AdamW pass, bytes */
#define TFB_PROF_LN_FWD 5     /* LayerNorm forward, bytes */
#define TFB_PROF_LN_BWD 6     /* LayerNorm backward (dx and the column partials), bytes */
#define TFB_PROF_GELU_FWD 7   /* GELU forward, bytes */
#define TFB_PROF_GELU_BWD 8   /* GELU backward, bytes */
#define TFB_PROF_GEMV 9       /* products of at most 16 rows (the decode Linears), bytes */
#define TFB_PROF_KV_ATTEND 10 /* cached single-query attention, bytes */
#define TFB_PROF_SAMPLE 11    /* top-k / temperature sampler, bytes */
#define TFB_PROF_KINDS 12
int tfb_profile_begin(tfb_ctx* ctx);
int tfb_profile_end(tfb_ctx* ctx, double* gemm_ms, double* gemm_flops, int* launches);
/* After tfb_profile_end: summed milliseconds, work and launches of one family
 * (TFB_ERR_ARG for an unknown kind, TFB_ERR_STATE while profiling runs). */
int tfb_profile_kind(tfb_ctx* ctx, int kind, double* ms, double* work, int* launches);

#ifdef __cplusplus
}
#endif
#endif /* TFB_H */
