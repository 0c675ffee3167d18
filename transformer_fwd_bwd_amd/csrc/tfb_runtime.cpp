// Host runtime of the C ABI declared in include/tfb.h: tensor table, arena,
// tape and the backward replay.
//
// The tape follows [Autograd-1, "How each op records itself in the graph"]:
// each op appends one record (inputs, output, saved values) after it has
// enqueued its forward kernels; backward() walks the records from the last to
// the first.  Records are appended in execution order, which is a topological
// order of the graph, so the reverse walk visits a node only after everything
// that consumed it.  A record whose output never received a gradient cannot
// reach the loss and is skipped (its contribution would be zero).
//
// Gradient buffers carry a state: NONE (no buffer), ZERO (cleared, contents
// not yet materialised) or VALID.  The first backward rule that writes a
// ZERO/NONE gradient overwrites it (beta = 0), every later one adds (beta = 1),
// which is the "+=" rule without a separate clearing pass.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <deque>
#include <stdexcept>
#include <string>
#include <vector>

#include "../../include/tfb.h"
#include "kernels.h"

using namespace tfb;

namespace {

thread_local std::string g_last_error;

struct Err {
  int code;
  std::string msg;
};

[[noreturn]] void fail(int code, const std::string& msg) { throw Err{code, msg}; }

void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) fail(TFB_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// G_BF16: the gradient exists only as its bf16 copy (gbf); no fp32 gradient is kept
enum GradState { G_NONE = 0, G_ZERO = 1, G_VALID = 2, G_BF16 = 3 };

struct TensorRec {
  std::string name;  // a leaf's name as given at creation (may be empty)
  bool live = false;
  bool leaf = true;
  bool is_param = false;
  bool owns_persistent = false;
  int ndim = 0;
  int64_t shape[TFB_MAX_DIMS] = {0};
  int64_t numel = 0;
  float* data = nullptr;
  float* grad = nullptr;
  int gstate = G_NONE;
  size_t persist_off = 0, persist_bytes = 0;
  // bf16 copies of data / grad used as contraction operands in the bf16 variant
  uint16_t* bf = nullptr;
  bool bf_valid = false;
  // false: only the bf16 copy was written (an output whose readers take bf16); any
  // fp32 reader first converts it back (Ctx::f32), exactly, from the bf16 values
  bool f32_valid = true;
  // made with the bf16-only output flag: where the contraction that produced it is
  // the only reader of its gradient, that gradient too may be kept as bf16 alone
  bool bf16_out = false;
  uint16_t* gbf = nullptr;
  bool gbf_valid = false;
  // column sums (over every row of the [rows, cols] view) of the finished gradient,
  // left by the kernel that wrote it: a Linear reading this as its output gradient
  // takes its bias gradient from here
  float* gcol = nullptr;
  bool gcol_valid = false;

  int64_t ld = 0;  // row stride of the last dim when rows are padded (0: dense)
  int uses = 0;    // ops on the tape that read this tensor
  int producer = -1;  // tape index of the op that wrote it (-1: none on the tape)
  // During backward: the gradient so far equals this finished gradient of
  // another tensor (a copy not yet made).  The next contribution reads it as
  // its accumulation source, or it is copied into `grad` before anyone reads
  // `grad`.  The buffer it points to is never written again in the pass.
  const float* gpend = nullptr;

  int64_t cols() const { return ndim ? shape[ndim - 1] : 1; }
  int64_t rows() const { return cols() ? numel / cols() : 0; }
  bool padded() const { return ld != 0 && ld != cols(); }
  int64_t stride() const { return padded() ? ld : cols(); }
  int64_t storage() const { return padded() ? rows() * ld : numel; }
};

enum OpKind {
  OP_ADD,
  OP_MUL,
  OP_SCALE,
  OP_SUM,
  OP_RESHAPE,
  OP_TANH,
  OP_GELU,
  OP_MATMUL,
  OP_MATMUL_T,
  OP_LINEAR,
  OP_LAYERNORM,
  OP_EMBEDDING,
  OP_NARROW,
  OP_SPLIT_HEADS,
  OP_MERGE_HEADS,
  OP_BMM,
  OP_BMM_T,
  OP_CSOFTMAX,
  OP_ATTENTION,
  OP_SOFTMAX_CE,
  OP_COMPACT,  // dense copy of a row-padded tensor (inserted by the library)
  OP_LINEAR_RES,  // x @ w + b + r: a Linear and the residual Add that follows it
};

struct Rec {
  OpKind op;
  int in[4] = {-1, -1, -1, -1};
  int out = -1;
  float f = 0.f;
  int64_t i0 = 0, i1 = 0, i2 = 0, i3 = 0;
  void* s0 = nullptr;  // saved buffers (step arena)
  void* s1 = nullptr;
};

constexpr size_t ALIGN = 256;

struct Arena {
  char* base = nullptr;
  size_t size = 0;
  size_t lo = 0;   // persistent allocations: [0, lo)
  size_t hi = 0;   // step allocations: [hi, size)
  // ranges below lo given back out of stack order (offset, bytes), sorted by
  // offset and coalesced; persistent allocations take the first that fits
  std::vector<std::pair<size_t, size_t>> holes;

  static size_t up(size_t n) { return (n + ALIGN - 1) / ALIGN * ALIGN; }
  size_t alloc_persist(size_t n) {
    n = up(std::max<size_t>(n, 1));
    for (size_t i = 0; i < holes.size(); ++i) {
      if (holes[i].second < n) continue;
      const size_t off = holes[i].first;
      holes[i].first += n, holes[i].second -= n;
      if (holes[i].second == 0) holes.erase(holes.begin() + i);
      return off;
    }
    if (lo + n > hi) fail(TFB_ERR_OOM, "arena exhausted (persistent allocation of " + std::to_string(n) + " bytes)");
    size_t off = lo;
    lo += n;
    return off;
  }
  // Give back [off, off + n) of the persistent end.  Work already queued on the
  // stream that uses the range runs before any later-queued work can reuse it.
  void release_persist(size_t off, size_t n) {
    n = up(std::max<size_t>(n, 1));
    size_t i = 0;
    while (i < holes.size() && holes[i].first < off) ++i;
    holes.insert(holes.begin() + i, {off, n});
    // coalesce with the neighbours, then let a hole that reaches lo lower it
    if (i + 1 < holes.size() && holes[i].first + holes[i].second == holes[i + 1].first) {
      holes[i].second += holes[i + 1].second;
      holes.erase(holes.begin() + i + 1);
    }
    if (i > 0 && holes[i - 1].first + holes[i - 1].second == holes[i].first) {
      holes[i - 1].second += holes[i].second;
      holes.erase(holes.begin() + i);
    }
    if (!holes.empty() && holes.back().first + holes.back().second == lo) {
      lo = holes.back().first;
      holes.pop_back();
    }
  }
  void* alloc_step(size_t n) {
    n = up(std::max<size_t>(n, 1));
    if (hi < lo + n) fail(TFB_ERR_OOM, "arena exhausted (step allocation of " + std::to_string(n) + " bytes)");
    hi -= n;
    return base + hi;
  }
};

}  // namespace

// Launch timing by kernel family (tfb_profile_*): each bracketed launch gets an
// event pair on the context's stream and adds its algorithmic work (flops or
// bytes, per TFB_PROF_*) to its family.
struct ProfileState {
  bool on = false;
  std::vector<hipEvent_t> pool;
  int used = 0;
  struct Span {
    int ev, kind;
    double work;
  };
  std::vector<Span> spans;
  double ms[TFB_PROF_KINDS] = {0}, work[TFB_PROF_KINDS] = {0};
  int launches[TFB_PROF_KINDS] = {0};
};

struct tfb_ctx {
  ProfileState prof;
  int device = 0;
  hipStream_t stream = nullptr;
  Arena arena;
  int precision = TFB_FP32;
  bool grad_enabled = true;
  std::deque<TensorRec> tensors;  // deque: handles' references survive growth
  std::vector<int> free_handles;
  std::vector<Rec> tape;
  // bias gradients taken from column sums, added in one launch at the end of the
  // backward pass (nothing reads a leaf's gradient before then)
  AxpbyJobs bias_jobs;
  // second stages of column reductions (LayerNorm parameter gradients, column sums of
  // gradients), run in one launch before the bias jobs; their partials live in the
  // step arena until then
  ReduceJobs reduce_jobs;
};

struct tfb_kv {
  tfb_ctx* ctx = nullptr;
  int layers = 0, batch = 0, tmax = 0, channels = 0;
  void* data = nullptr;  // persistent arena: [layers][2][batch][tmax][channels], fp32 or bf16
  bool bf16 = false;     // made in the bf16 variant: keys and values stored as bf16
  size_t off = 0, end = 0;  // its arena range [off, end)
};

struct tfb_opt {
  tfb_ctx* ctx = nullptr;
  std::vector<int> params;
  std::vector<float*> m, v;
  float lr, wd, b1, b2, eps;
  int t = 0;
  int64_t chunk_elems = 1 << 16;
  AdamSeg* d_segs = nullptr;
  AdamChunk* d_chunks = nullptr;
  int d_nseg_cap = 0, d_nchunk_cap = 0;
  std::vector<int> uploaded_active;
  std::vector<uint16_t*> uploaded_shadows;
  int nchunks = 0;
};

namespace {

// ------------------------------------------------------------------ helpers
struct Ctx {
  tfb_ctx* c;
  explicit Ctx(tfb_ctx* ctx) : c(ctx) {
    if (!ctx) fail(TFB_ERR_ARG, "null context");
    hip_check(hipSetDevice(ctx->device), "hipSetDevice");
  }
  TensorRec& T(int h) {
    if (h < 0 || h >= (int)c->tensors.size() || !c->tensors[h].live)
      fail(TFB_ERR_ARG, "invalid or released tensor handle " + std::to_string(h));
    return c->tensors[h];
  }
  hipStream_t s() const { return c->stream; }

  // Bracket the launches made by f() with events when profiling is on, counting
  // `work` (flops or bytes: TFB_PROF_*) for family `kind`.
  template <typename F>
  void timed(int kind, double work, F&& f) {
    ProfileState& pf = c->prof;
    if (!pf.on) {
      f();
      return;
    }
    while ((int)pf.pool.size() < pf.used + 2) {
      hipEvent_t e;
      hip_check(hipEventCreate(&e), "hipEventCreate");
      pf.pool.push_back(e);
    }
    // the kernels' own dispatches carry the events (tfb::run_kernel); a launch made
    // some other way (a copy) falls back to events recorded on the stream around it
    hip_check(hipEventRecord(pf.pool[pf.used], s()), "hipEventRecord");
    LaunchEvents& le = launch_events();
    le.start = pf.pool[pf.used], le.stop = pf.pool[pf.used + 1], le.launches = 0;
    try {
      f();
    } catch (...) {
      le = LaunchEvents();
      throw;
    }
    const int n = le.launches;
    le = LaunchEvents();
    if (n == 0) hip_check(hipEventRecord(pf.pool[pf.used + 1], s()), "hipEventRecord");
    pf.spans.push_back({pf.used, kind, work});
    pf.used += 2;
  }

  int new_handle() {
    if (!c->free_handles.empty()) {
      int h = c->free_handles.back();
      c->free_handles.pop_back();
      c->tensors[h] = TensorRec();
      return h;
    }
    c->tensors.emplace_back();
    return (int)c->tensors.size() - 1;
  }

  static int64_t numel_of(const int64_t* shape, int ndim) {
    if (ndim < 1 || ndim > TFB_MAX_DIMS) fail(TFB_ERR_SHAPE, "rank must be 1.." + std::to_string(TFB_MAX_DIMS));
    int64_t n = 1;
    for (int i = 0; i < ndim; ++i) {
      if (shape[i] < 0) fail(TFB_ERR_SHAPE, "negative dimension");
      n *= shape[i];
    }
    return n;
  }

  // an op output in the step arena; ld > last dim pads every row to ld floats
  int make_output(const std::vector<int64_t>& shape, int64_t ld = 0) {
    int64_t n = numel_of(shape.data(), (int)shape.size());
    const int64_t cols = shape.back();
    const int64_t stor = (ld > cols && cols > 0) ? n / cols * ld : n;
    float* p = static_cast<float*>(c->arena.alloc_step((size_t)stor * sizeof(float)));
    int h = new_handle();
    TensorRec& t = c->tensors[h];
    t.live = true;
    t.leaf = false;
    t.ndim = (int)shape.size();
    for (int i = 0; i < t.ndim; ++i) t.shape[i] = shape[i];
    t.numel = n;
    t.ld = ld > cols ? ld : 0;
    t.data = p;
    return h;
  }

  // fp32 data of t: converted from its bf16 copy first when only that was written
  const float* f32(TensorRec& t) {
    if (!t.f32_valid) {
      hip_check(to_f32(t.bf, t.data, t.storage(), s()), "to_f32");
      t.f32_valid = true;
    }
    return t.data;
  }

  // ops other than the cross-entropy read dense fp32 rows: a padded input is first
  // copied to a dense tensor by a recorded compaction op, and an input held only as
  // bf16 is converted (bf16_ok: the op reads bf16 copies itself, so it is not)
  int dense_in(int h, bool bf16_ok = false) {
    TensorRec& t = T(h);
    if (!bf16_ok || t.padded()) f32(t);
    if (!t.padded()) return h;
    const int64_t rows = t.rows(), cols = t.cols(), ld = t.ld;
    const float* src = t.data;
    int o = make_output(std::vector<int64_t>(t.shape, t.shape + t.ndim));
    hip_check(copy_pitched(src, ld, c->tensors[o].data, cols, rows, cols, 0.f, s()), "compact");
    Rec r{OP_COMPACT};
    r.in[0] = h, r.out = o;
    record(r);
    return o;
  }

  void ensure_grad_buffer(TensorRec& t) {
    if (t.grad) return;
    const size_t bytes = (size_t)t.storage() * sizeof(float);
    if (t.leaf) {
      size_t off = c->arena.alloc_persist(bytes);
      t.grad = reinterpret_cast<float*>(c->arena.base + off);
    } else {
      t.grad = static_cast<float*>(c->arena.alloc_step(bytes));
    }
    t.gstate = G_ZERO;
  }

  // destination of a gradient contribution: (pointer, beta)
  std::pair<float*, float> gdst(int h) {
    TensorRec& t = T(h);
    settle(t);
    ensure_grad_buffer(t);
    flush_bias_into(t.grad);
    t.gbf_valid = false;
    t.gcol_valid = false;
    if (t.gstate == G_VALID) return {t.grad, 1.f};
    t.gstate = G_VALID;
    return {t.grad, 0.f};
  }

  // the same for a kernel that reads the earlier gradient from a separate
  // pointer: (destination, beta, source of the earlier gradient)
  struct GradDst {
    float* dst;
    float beta;
    const float* src;
  };
  GradDst gdst_src(int h) {
    TensorRec& t = T(h);
    flush_bias_into(t.grad);
    if (t.gpend) {
      ensure_grad_buffer(t);
      const float* src = t.gpend;
      t.gpend = nullptr;
      t.gstate = G_VALID;
      t.gbf_valid = false;
      t.gcol_valid = false;
      return {t.grad, 1.f, src};
    }
    const auto d = gdst(h);
    return {d.first, d.second, d.first};
  }

  // make a pending first contribution real
  void settle(TensorRec& t) {
    if (!t.gpend) return;
    const float* src = t.gpend;
    t.gpend = nullptr;
    ensure_grad_buffer(t);
    hip_check(axpby(t.grad, src, 1.f, 0.f, t.numel, s()), "gradient copy");
    t.gstate = G_VALID;
    t.gbf_valid = false;
    t.gcol_valid = false;
  }

  // x's gradient so far is the finished gradient of `out` (a residual
  // branch): remember the buffer instead of copying it.  Only for a
  // gradient with no contribution yet, of the same dense shape.
  bool defer_grad(TensorRec& x, const TensorRec& out) {
    if (x.leaf || x.is_param || x.gpend || x.gstate == G_VALID) return false;
    if (x.padded() || out.padded() || x.numel != out.numel || !out.grad || out.gpend) return false;
    x.gpend = out.grad;
    x.gbf_valid = false;
    return true;
  }

  bool bf16_mode() const { return c->precision == TFB_BF16_MFMA; }

  uint16_t* alloc_bf16(const TensorRec& t) {
    const size_t bytes = (size_t)std::max<int64_t>(t.storage(), 1) * sizeof(uint16_t);
    if (t.leaf) return reinterpret_cast<uint16_t*>(c->arena.base + c->arena.alloc_persist(bytes));
    return static_cast<uint16_t*>(c->arena.alloc_step(bytes));
  }

  // bf16 copy written by the producing kernel beside its fp32 output (bf16
  // variant only; null otherwise).  The caller marks it valid after the launch.
  uint16_t* twin_data(TensorRec& t) {
    if (!bf16_mode()) return nullptr;
    if (!t.bf) t.bf = alloc_bf16(t);
    return t.bf;
  }
  uint16_t* twin_grad(TensorRec& t) {
    if (!bf16_mode()) return nullptr;
    if (!t.gbf) t.gbf = alloc_bf16(t);
    return t.gbf;
  }

  // Before a backward rule: the tensors it reads as fp32 data, converted where only
  // their bf16 copy exists.  The contraction rules read their inputs through
  // op_data (bf16 copies, or converted fp32 in the fp32 variant) and the fused
  // attention reads q, k, v as bf16 and its output in fp32.
  void f32_for_bwd(const Rec& r) {
    switch (r.op) {
      case OP_LINEAR:
      case OP_LINEAR_RES:
      case OP_MATMUL:
      case OP_MATMUL_T:
      case OP_ADD:
      case OP_SCALE:
      case OP_SUM:
      case OP_RESHAPE:
      case OP_EMBEDDING:
      case OP_NARROW:
      case OP_SPLIT_HEADS:
      case OP_MERGE_HEADS:
      case OP_COMPACT:
        return;  // these read gradients only (or inputs through op_data)
      case OP_TANH:
      case OP_CSOFTMAX:
        f32(T(r.out));
        return;
      case OP_GELU:
        return;  // the rule reads its input's bf16 copy or converts it
      case OP_SOFTMAX_CE:
        return;  // the rule reads bf16-only logits as such or converts them
      case OP_LAYERNORM:
        f32(T(r.in[0]));
        f32(T(r.in[1]));
        return;
      case OP_ATTENTION:
        if (r.i1 == 1) return;  // the fused backward reads the output's fp32 form or its bf16 copy
        break;
      default:
        break;
    }
    for (int h : r.in)
      if (h >= 0) f32(T(h));
    f32(T(r.out));
  }

  // buffer for t's gradient column sums (non-leaf tensors only)
  // a queued job must land before any other contribution to the same gradient
  void flush_bias_into(const float* g) {
    if (!g) return;
    for (int i = 0; i < c->reduce_jobs.count; ++i)
      for (float* o : c->reduce_jobs.j[i].out)
        if (o == g) {
          flush_bias();  // the reductions first, then the bias jobs that read their sums
          return;
        }
    for (int i = 0; i < c->bias_jobs.count; ++i)
      if (c->bias_jobs.j[i].dst == g) {
        flush_bias();
        return;
      }
  }
  void flush_reduce() {
    hip_check(reduce_batch(c->reduce_jobs, s()), "column reductions");
    c->reduce_jobs.count = 0;
  }
  // queue a described reduction (kind 0: nothing was deferred); a job writing an output
  // that a queued one writes first lets the queue run
  void defer_reduce(const ReduceJob& j) {
    if (j.kind == 0) return;
    ReduceJobs& q = c->reduce_jobs;
    bool clash = q.count == REDUCE_BATCH;
    for (int i = 0; i < q.count && !clash; ++i)
      for (float* a : q.j[i].out)
        for (float* b : j.out) clash = clash || (a && a == b);
    if (clash) flush_reduce();
    q.j[q.count++] = j;
  }
  // workspace for partials that a deferred reduction reads later: the step arena
  void* keep(size_t bytes) { return c->arena.alloc_step(std::max<size_t>(bytes, 256)); }
  void flush_bias() {
    flush_reduce();
    hip_check(axpby_batch(c->bias_jobs, s()), "bias gradients");
    c->bias_jobs.count = 0;
  }
  // dst = src + beta * dst at the end of the pass (earlier if dst is already queued:
  // a second contribution must see the first)
  void defer_bias(float* dst, const float* src, int64_t n, float beta) {
    AxpbyJobs& q = c->bias_jobs;
    bool clash = q.count == AXPBY_BATCH;
    for (int i = 0; i < q.count && !clash; ++i) clash = q.j[i].dst == dst;
    if (clash) flush_bias();
    q.j[q.count++] = AxpbyJob{dst, src, n, beta};
  }

  float* gcol_buf(TensorRec& t) {
    if (t.leaf || t.cols() <= 0) return nullptr;
    if (!t.gcol) t.gcol = static_cast<float*>(c->arena.alloc_step((size_t)t.cols() * sizeof(float)));
    return t.gcol;
  }

  // bf16 copy of a tensor's data, converted once and reused until the data changes
  const uint16_t* data_bf16(TensorRec& t) {
    if (!t.bf_valid) {
      if (!t.bf) t.bf = alloc_bf16(t);
      hip_check(to_bf16(t.data, t.bf, t.storage(), s()), "to_bf16");
      t.bf_valid = true;
    }
    return t.bf;
  }

  // bf16 copy of a finished gradient (all contributions already added)
  const uint16_t* grad_bf16(TensorRec& t) {
    materialize_zero(t);
    if (!t.gbf_valid) {
      if (!t.gbf) t.gbf = alloc_bf16(t);
      hip_check(to_bf16(t.grad, t.gbf, t.storage(), s()), "to_bf16");
      t.gbf_valid = true;
    }
    return t.gbf;
  }

  void materialize_zero(TensorRec& t) {
    if (t.grad && t.gstate == G_ZERO) {
      hip_check(fill(t.grad, 0.f, t.storage(), s()), "fill");
      t.gstate = G_VALID;
    }
  }

  void record(const Rec& r) {
    if (!c->grad_enabled) return;
    c->tape.push_back(r);
    for (int h : r.in)
      if (h >= 0) c->tensors[h].uses += 1;
    c->tensors[r.out].producer = (int)c->tape.size() - 1;
  }

  // t is a bf16-only GELU output whose backward can read t's gradient as bf16 alone
  // (the row-slab kernel, whose shape and alignment conditions are checked here)
  bool gelu_takes_bf16_grad(const TensorRec& t) const {
    if (!bf16_mode() || !t.bf16_out || t.producer < 0 || t.producer >= (int)c->tape.size()) return false;
    const Rec& p = c->tape[t.producer];
    if (&c->tensors[p.out] != &t || p.op != OP_GELU) return false;
    const TensorRec& a = c->tensors[p.in[0]];
    return !a.padded() && !t.padded() && !a.leaf && a.rows() >= 128 && a.cols() % 4 == 0;
  }

  // t is a bf16-only LayerNorm output whose backward can read t's gradient as bf16
  // (the fused kernel; its shape and alignment conditions are checked here)
  bool layernorm_takes_bf16_grad(const TensorRec& t) const {
    if (!bf16_mode() || !t.bf16_out || t.padded() || t.producer < 0 || t.producer >= (int)c->tape.size()) return false;
    const Rec& p = c->tape[t.producer];
    if (&c->tensors[p.out] != &t || p.op != OP_LAYERNORM) return false;
    const TensorRec& x = c->tensors[p.in[0]];
    const TensorRec& gm = c->tensors[p.in[1]];
    return !x.padded() && (reinterpret_cast<uintptr_t>(x.data) & 15) == 0 &&
           (reinterpret_cast<uintptr_t>(gm.data) & 15) == 0 && x.cols() % 4 == 0 && x.cols() <= 1024 && x.rows() > 0;
  }

  // t is a bf16-only output of the fused attention (whose backward reads its
  // gradient as bf16 and can take D from the bf16 copies)
  bool attention_out_bf16(const TensorRec& t) const {
    if (!bf16_mode() || !t.bf16_out || t.producer < 0 || t.producer >= (int)c->tape.size()) return false;
    const Rec& p = c->tape[t.producer];
    return &c->tensors[p.out] == &t && p.op == OP_ATTENTION && p.i1 == 1;
  }

  // the backward of t's producer reads t's gradient as the bf16 copy
  bool grad_read_as_bf16(const TensorRec& t) const {
    if (!bf16_mode() || t.producer < 0 || t.producer >= (int)c->tape.size()) return false;
    const Rec& p = c->tape[t.producer];
    if (&c->tensors[p.out] != &t) return false;
    return p.op == OP_LINEAR || p.op == OP_LINEAR_RES || p.op == OP_MATMUL || p.op == OP_MATMUL_T ||
           (p.op == OP_ATTENTION && p.i1 == 1);
  }

  // An op output read by exactly one op (this one, during its backward) whose
  // gradient is a plain copy of `out`'s finished gradient can use out's
  // gradient buffer itself: no later contribution can reach it.
  bool share_grad(TensorRec& x, const TensorRec& out) {
    if (x.leaf || x.is_param || x.uses != 1 || x.grad || x.gstate != G_NONE) return false;
    if (x.padded() || out.padded() || x.numel != out.numel || !out.grad) return false;
    x.grad = out.grad;
    x.gstate = G_VALID;
    x.gbf = out.gbf_valid ? out.gbf : nullptr;
    x.gbf_valid = out.gbf_valid;
    x.gcol = out.gcol_valid && x.cols() == out.cols() ? out.gcol : nullptr;
    x.gcol_valid = x.gcol != nullptr;
    return true;
  }

  GemmArgs gemm_base() const {
    GemmArgs g;
    g.prec = c->precision == TFB_BF16_MFMA ? PREC_BF16 : PREC_F32;
    return g;
  }

  void run_gemm(const GemmArgs& g) {
    size_t ws = gemm_workspace_bytes(g);
    size_t mark = c->arena.hi;
    void* w = ws ? c->arena.alloc_step(ws) : nullptr;
    // a product of at most 16 rows is a weight stream (the decode Linears): bytes
    const bool few = g.M <= 16 && g.batch == 1;
    const double work = few ? gemv_bytes(g) : needed_flops(g);
    timed(few ? TFB_PROF_GEMV : TFB_PROF_GEMM, work, [&] { hip_check(gemm(g, w, ws, s()), "gemm launch"); });
    c->arena.hi = mark;  // scratch: later work on the same stream runs after this gemm
  }

  // a few-row product whose workspace (its partial products) the caller keeps for a
  // later kernel: no scratch of its own
  void run_gemm_ws(const GemmArgs& g, void* ws, size_t bytes) {
    hipError_t e = hipSuccess;
    timed(TFB_PROF_GEMV, gemv_bytes(g), [&] {
      if (!gemv(g, ws, bytes, s(), &e)) fail(TFB_ERR_STATE, "few-row product declined");
      hip_check(e, "gemv launch");
    });
  }

  // bytes a few-row product must move: its operands once, its output once
  static double gemv_bytes(const GemmArgs& g) {
    const double ea = g.a_bf16 ? 2 : 4, eb = g.b_bf16 ? 2 : 4;
    double b = (g.a_part ? 4.0 * g.a_chunks : g.att_acc ? 4.0 * g.att_blocks : ea) * g.M * (double)g.K +
               eb * (double)g.K * g.N;
    b += (g.c_bf16_only ? 2.0 : 4.0 + (g.Cbf ? 2.0 : 0.0)) * g.M * (double)g.N;
    if (g.bias) b += 4.0 * g.N;
    if (g.resid) b += 4.0 * g.M * (double)g.N;
    if (g.beta != 0.f) b += 4.0 * g.M * (double)g.N;
    return b;
  }

  // multiply-adds the contraction must do, x2; a causal product needs only the
  // triangle j <= i: T(T+1)/2 of the T*T (query, key) pairs
  static double needed_flops(const GemmArgs& g) {
    double f = 2.0 * g.M * (double)g.N * g.K * g.batch;
    if (g.causal_out) f = 2.0 * g.K * (g.M * (g.M + 1.0) / 2.0) * g.batch;
    if (g.causal_a != CAUSAL_NONE) f = 2.0 * g.N * (g.M * (g.M + 1.0) / 2.0) * g.batch;
    return f;
  }

  void* scratch(size_t n) { return c->arena.alloc_step(n); }
};

template <typename F>
int guarded(F&& f) {
  try {
    f();
    return TFB_OK;
  } catch (const Err& e) {
    g_last_error = e.msg;
    return e.code;
  } catch (const std::exception& e) {
    g_last_error = e.what();
    return TFB_ERR_STATE;
  }
}

void need(bool cond, int code, const std::string& msg) {
  if (!cond) fail(code, msg);
}

std::string shape_str(const TensorRec& t) {
  std::string s = "[";
  for (int i = 0; i < t.ndim; ++i) s += (i ? "," : "") + std::to_string(t.shape[i]);
  // a named leaf (a parameter) is named in shape errors, as the pages' messages do
  return s + "]" + (t.name.empty() ? "" : " (" + t.name + ")");
}

std::vector<int64_t> shape_vec(const TensorRec& t) { return std::vector<int64_t>(t.shape, t.shape + t.ndim); }

// ------------------------------------------------------------------ contraction layouts
// A contraction operand: fp32 data, or its bf16 copy in the bf16 variant.
struct Opnd {
  const void* p;
  bool bf;
};

Opnd op_data(Ctx& C, TensorRec& t) {
  if (C.bf16_mode()) return {C.data_bf16(t), true};
  return {C.f32(t), false};
}
Opnd op_grad(Ctx& C, TensorRec& t) {
  if (C.bf16_mode()) return {C.grad_bf16(t), true};
  C.materialize_zero(t);
  return {t.grad, false};
}

void set_a(GemmArgs& g, Opnd o) {
  g.A = static_cast<const float*>(o.p);
  g.a_bf16 = o.bf;
}
void set_b(GemmArgs& g, Opnd o) {
  g.B = static_cast<const float*>(o.p);
  g.b_bf16 = o.bf;
}

// y[rows, N] = x[rows, K] @ w[K, N] (+ bias)
void gemm_nn(Ctx& C, Opnd x, Opnd w, float* y, int64_t rows, int64_t K, int64_t N, float beta, const float* bias,
             int64_t lda = -1, uint16_t* ybf = nullptr, const float* resid = nullptr, bool ybf_only = false) {
  GemmArgs g = C.gemm_base();
  g.M = (int)rows, g.N = (int)N, g.K = (int)K;
  set_a(g, x), g.lda = lda < 0 ? K : lda;
  set_b(g, w), g.ldb = N;
  g.C = y, g.ldc = N, g.Cbf = ybf, g.resid = resid, g.c_bf16_only = ybf_only && ybf;
  g.beta = beta, g.bias = bias;
  C.run_gemm(g);
}
// y[rows, N] = x[rows, K] @ w[N, K]^T
void gemm_nt(Ctx& C, Opnd x, Opnd w, float* y, int64_t rows, int64_t K, int64_t N, float beta, int64_t ldc = -1,
             uint16_t* ybf = nullptr, bool bf16_only = false) {
  GemmArgs g = C.gemm_base();
  g.M = (int)rows, g.N = (int)N, g.K = (int)K;
  set_a(g, x), g.lda = K;
  set_b(g, w), g.ldb = K, g.b_kcontig = true;
  g.C = y, g.ldc = ldc < 0 ? N : ldc, g.Cbf = ybf, g.c_bf16_only = bf16_only;
  g.beta = beta;
  C.run_gemm(g);
}
// y[M, N] = x[K, M]^T @ g[K, N]
void gemm_tn(Ctx& C, Opnd x, Opnd gr, float* y, int64_t M, int64_t K, int64_t N, float beta, int64_t lda = -1) {
  GemmArgs g = C.gemm_base();
  g.M = (int)M, g.N = (int)N, g.K = (int)K;
  set_a(g, x), g.lda = lda < 0 ? M : lda, g.a_mcontig = true;
  set_b(g, gr), g.ldb = N;
  g.C = y, g.ldc = N;
  g.beta = beta;
  C.run_gemm(g);
}

void check_gemm_dims(int64_t a, int64_t b, int64_t c) {
  need(a < (1ll << 31) && b < (1ll << 31) && c < (1ll << 31), TFB_ERR_SHAPE, "contraction dimension too large");
}

// ------------------------------------------------------------------ backward rules
void backward_rec(Ctx& C, const Rec& r) {
  TensorRec& out = C.T(r.out);
  const float* g = out.grad;
  hipStream_t s = C.s();
  switch (r.op) {
    case OP_ADD: {
      TensorRec& a = C.T(r.in[0]);
      TensorRec& b = C.T(r.in[1]);
      if (r.in[0] == r.in[1] || !(C.share_grad(a, out) || C.defer_grad(a, out))) {
        auto da = C.gdst(r.in[0]);
        hip_check(axpby(da.first, g, 1.f, da.second, a.numel, s), "add bwd");
      }
      if (b.numel == out.numel && r.in[0] != r.in[1] && C.share_grad(b, out)) break;
      auto db = C.gdst(r.in[1]);
      const int64_t rows = b.numel ? a.numel / b.numel : 0;
      size_t mark = C.c->arena.hi;
      void* ws = C.scratch(colsum_workspace_bytes(rows, b.numel));
      hip_check(colsum(g, rows, b.numel, db.first, db.second, ws, s), "add bwd colsum");
      C.c->arena.hi = mark;
      break;
    }
    case OP_MUL: {
      TensorRec& a = C.T(r.in[0]);
      TensorRec& b = C.T(r.in[1]);
      auto da = C.gdst(r.in[0]);
      hip_check(mul_bwd(g, b.data, da.first, da.second, a.numel, s), "mul bwd a");
      auto db = C.gdst(r.in[1]);
      hip_check(mul_bwd(g, a.data, db.first, db.second, b.numel, s), "mul bwd b");
      break;
    }
    case OP_SCALE: {
      auto da = C.gdst(r.in[0]);
      hip_check(axpby(da.first, g, r.f, da.second, out.numel, s), "scale bwd");
      break;
    }
    case OP_SUM: {
      TensorRec& a = C.T(r.in[0]);
      auto da = C.gdst(r.in[0]);
      hip_check(bcast_scalar_bwd(g, da.first, da.second, a.numel, s), "sum bwd");
      break;
    }
    case OP_RESHAPE: {
      auto da = C.gdst(r.in[0]);
      hip_check(axpby(da.first, g, 1.f, da.second, out.numel, s), "reshape bwd");
      break;
    }
    case OP_TANH: {
      auto da = C.gdst(r.in[0]);
      hip_check(tanh_bwd(g, out.data, da.first, da.second, out.numel, s), "tanh bwd");
      break;
    }
    case OP_GELU: {
      TensorRec& a = C.T(r.in[0]);
      float* dcol = a.padded() ? nullptr : C.gcol_buf(a);
      // the upstream gradient held only as bf16 (see gelu_takes_bf16_grad): read as such
      const uint16_t* gb = out.gstate == G_BF16 ? out.gbf : nullptr;
      // A bf16-only input whose one gradient is read by its producer as bf16 (with the
      // bias gradient from the column sums below): that copy alone, no fp32 gradient
      if (dcol && a.bf16_out && a.uses == 1 && !a.gpend && a.gstate != G_VALID && C.grad_read_as_bf16(a)) {
        uint16_t* db = C.twin_grad(a);
        void* ws = C.keep(colsum_workspace_bytes(a.rows(), a.cols()));  // read by the deferred reduction
        const void* xin = a.f32_valid ? (const void*)a.data : (const void*)a.bf;
        if (db && gelu_bwd_cols_fits(gb ? reinterpret_cast<const float*>(gb) : g, xin, nullptr, db, a.rows(), a.cols(), ws) &&
            (!a.f32_valid || (reinterpret_cast<uintptr_t>(a.data) & 15) == 0)) {
          bool written = false;
          ReduceJob job;
          const double bytes = (double)a.numel * ((gb ? 2 : 4) + (a.f32_valid ? 4 : 2) + 2);
          C.timed(TFB_PROF_GELU_BWD, bytes, [&] {
            hip_check(gelu_bwd_cols(g, a.f32_valid ? a.data : nullptr, nullptr, db, 0.f, a.rows(), a.cols(), dcol, ws,
                                    s, &written, a.f32_valid ? nullptr : a.bf, gb, &job),
                      "gelu bwd");
          });
          C.defer_reduce(job);
          a.gstate = G_BF16;
          a.gbf_valid = true;
          a.gcol_valid = written;
          break;
        }
      }
      if (gb) {  // the general paths read fp32: convert the upstream gradient
        hip_check(to_f32(gb, out.grad, out.storage(), s), "gelu upstream gradient");
        out.gstate = G_VALID;
        gb = nullptr;
      }
      auto da = C.gdst(r.in[0]);
      uint16_t* db = C.twin_grad(a);
      if (dcol) {  // with the column sums a reading Linear takes as its bias gradient
        void* ws = C.keep(colsum_workspace_bytes(a.rows(), a.cols()));  // read by the deferred reduction
        // an input held only as bf16 is read as such where the row-slab kernel fits
        const bool abf = !a.f32_valid && gelu_bwd_cols_fits(g, a.bf, da.first, db, a.rows(), a.cols(), ws);
        bool written = false;
        ReduceJob job;
        const float* xa = abf ? nullptr : C.f32(a);
        const double bytes = (double)a.numel * (4 + (abf ? 2 : 4) + 4 + (da.second != 0.f ? 4 : 0) + (db ? 2 : 0));
        C.timed(TFB_PROF_GELU_BWD, bytes, [&] {
          hip_check(gelu_bwd_cols(g, xa, da.first, db, da.second, a.rows(), a.cols(), dcol, ws, s, &written,
                                  abf ? a.bf : nullptr, nullptr, &job),
                    "gelu bwd");
        });
        C.defer_reduce(job);
        a.gcol_valid = written;
      } else {
        const float* xa = C.f32(a);
        const double bytes = (double)out.numel * (4 + 4 + 4 + (da.second != 0.f ? 4 : 0) + (db ? 2 : 0));
        C.timed(TFB_PROF_GELU_BWD, bytes,
                [&] { hip_check(gelu_bwd(g, xa, da.first, db, da.second, out.numel, s), "gelu bwd"); });
      }
      if (db) a.gbf_valid = true;
      break;
    }
    case OP_LINEAR_RES: {
      // the residual input's gradient is the output's gradient itself
      TensorRec& res = C.T(r.in[3]);
      if (!(C.share_grad(res, out) || C.defer_grad(res, out))) {
        auto dr = C.gdst(r.in[3]);
        hip_check(axpby(dr.first, g, 1.f, dr.second, res.numel, s), "residual bwd");
      }
    }
      [[fallthrough]];
    case OP_MATMUL:
    case OP_LINEAR: {
      TensorRec& x = C.T(r.in[0]);
      TensorRec& w = C.T(r.in[1]);
      const int64_t rows = x.rows(), K = w.shape[0], N = w.shape[1];
      const Opnd go = op_grad(C, out);
      auto dx = C.gdst(r.in[0]);
      // a first and only contribution read as bf16 by x's producer: the product writes that copy too
      const bool first_only = dx.second == 0.f && x.uses == 1 && !x.leaf;
      uint16_t* dxb = first_only && C.grad_read_as_bf16(x) ? C.twin_grad(x) : nullptr;
      // ... or that copy alone, for a bf16-only GELU output (the GELU backward reads bf16)
      // or a bf16-only attention output (its backward then takes D from bf16 copies)
      const bool only = first_only && ((!dxb && (C.gelu_takes_bf16_grad(x) || C.layernorm_takes_bf16_grad(x))) ||
                                        (dxb && C.attention_out_bf16(x)));
      if (only) dxb = C.twin_grad(x);
      gemm_nt(C, go, op_data(C, w), dx.first, rows, N, K, dx.second, -1, dxb, only);   // dx = g @ w^T
      if (dxb) x.gbf_valid = true;
      if (only) x.gstate = G_BF16;
      auto dw = C.gdst(r.in[1]);
      gemm_tn(C, op_data(C, x), go, dw.first, K, rows, N, dw.second);   // dw = x^T @ g
      if (r.op != OP_MATMUL) {
        auto db = C.gdst(r.in[2]);
        if (out.gcol_valid && out.cols() == N) {  // summed by the kernel that finished g
          C.defer_bias(db.first, out.gcol, N, db.second);
        } else {
          void* ws = C.keep(colsum_workspace_bytes(rows, N));  // read by the deferred reduction
          ReduceJob job;
          hip_check(colsum(g, rows, N, db.first, db.second, ws, s, out.gstate == G_BF16 ? out.gbf : nullptr, &job),
                    "linear bias bwd");
          C.defer_reduce(job);
        }
      }
      break;
    }
    case OP_MATMUL_T: {
      TensorRec& x = C.T(r.in[0]);
      TensorRec& w = C.T(r.in[1]);
      const int64_t rows = x.rows(), V = w.shape[0], Cc = w.shape[1];
      const Opnd go = op_grad(C, out);
      const int64_t ldg = out.stride();
      auto dx = C.gdst(r.in[0]);
      gemm_nn(C, go, op_data(C, w), dx.first, rows, V, Cc, dx.second, nullptr, ldg);  // dx = g @ w
      auto dw = C.gdst(r.in[1]);
      gemm_tn(C, go, op_data(C, x), dw.first, V, rows, Cc, dw.second, ldg);           // dw = g^T @ x
      break;
    }
    case OP_LAYERNORM: {
      TensorRec& x = C.T(r.in[0]);
      TensorRec& gm = C.T(r.in[1]);
      const int64_t rows = x.rows(), Cc = x.cols();
      const auto dx = C.gdst_src(r.in[0]);
      auto dg = C.gdst(r.in[1]);
      auto db = C.gdst(r.in[2]);
      // the bf16 copy of dx serves the contractions when this is the gradient's last
      // contribution (a later one invalidates it); a residual-stream gradient is one
      uint16_t* dxb = x.leaf ? nullptr : C.twin_grad(x);
      // and its column sums: the bias gradient of a Linear whose output this gradient also is
      float* dxs = C.gcol_buf(x);
      void* ws = C.keep(layernorm_bwd_workspace_bytes(rows, Cc));  // read by the deferred reduction
      bool summed = false;
      // an upstream gradient held only as bf16 is read as such where the fused kernel runs
      const uint16_t* gb = out.gstate == G_BF16 ? out.gbf : nullptr;
      if (gb && !(layernorm_bwd_bf16_fits(x.data, dx.dst, gb, rows, Cc) && (reinterpret_cast<uintptr_t>(gm.data) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(dx.src ? dx.src : dx.dst) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(ws) & 15) == 0)) {
        hip_check(to_f32(gb, out.grad, out.storage(), s), "layernorm upstream gradient");
        out.gstate = G_VALID;
        gb = nullptr;
      }
      ReduceJob job;
      // g, x, dx (and the earlier dx it adds to), its bf16 copy, the row statistics
      const double bytes = (double)rows * Cc * ((gb ? 2 : 4) + 4 + 4 + ((dx.src || dx.beta != 0.f) ? 4 : 0) +
                                                (dxb ? 2 : 0)) + 8.0 * rows;
      C.timed(TFB_PROF_LN_BWD, bytes, [&] {
        hip_check(layernorm_bwd(g, x.data, gm.data, static_cast<float*>(r.s0), static_cast<float*>(r.s1), dx.dst,
                                dx.src, dxb, dg.first, db.first, rows, Cc, dx.beta, dg.second, db.second, ws, s, dxs,
                                &summed, gb, &job),
                  "layernorm bwd");
      });
      C.defer_reduce(job);
      if (dxb) x.gbf_valid = true;
      x.gcol_valid = summed;
      break;
    }
    case OP_EMBEDDING: {
      TensorRec& tab = C.T(r.in[0]);
      auto dt = C.gdst(r.in[0]);
      if (dt.second == 0.f) hip_check(fill(dt.first, 0.f, tab.numel, s), "embedding bwd clear");
      size_t mark = C.c->arena.hi;
      void* ws = C.scratch(embedding_bwd_workspace_bytes(r.i0));
      hip_check(embedding_bwd(g, static_cast<const int32_t*>(r.s0), r.i0, tab.cols(), dt.first, tab.rows(), ws, s),
                "embedding bwd");
      C.c->arena.hi = mark;
      break;
    }
    case OP_NARROW: {
      TensorRec& x = C.T(r.in[0]);
      auto dx = C.gdst(r.in[0]);
      hip_check(narrow_bwd(g, dx.first, x.rows(), x.cols(), r.i0, r.i1, dx.second, s), "narrow bwd");
      break;
    }
    case OP_SPLIT_HEADS: {  // out [B, H, T, hs] -> dx [B, T, H, hs]
      auto dx = C.gdst(r.in[0]);
      hip_check(permute_heads(g, dx.first, out.shape[0], out.shape[2], out.shape[1], out.shape[3], false, dx.second, s),
                "split_heads bwd");
      break;
    }
    case OP_MERGE_HEADS: {  // in [B, H, T, hs]
      TensorRec& x = C.T(r.in[0]);
      auto dx = C.gdst(r.in[0]);
      hip_check(permute_heads(g, dx.first, x.shape[0], x.shape[2], x.shape[1], x.shape[3], true, dx.second, s),
                "merge_heads bwd");
      break;
    }
    case OP_BMM:
    case OP_BMM_T: {
      TensorRec& a = C.T(r.in[0]);
      TensorRec& b = C.T(r.in[1]);
      const int64_t Z = a.shape[0], n = a.shape[1], k = a.shape[2];
      const int64_t m = out.shape[2];
      auto da = C.gdst(r.in[0]);
      {
        GemmArgs q = C.gemm_base();
        q.M = (int)n, q.N = (int)k, q.K = (int)m;
        q.A = g, q.lda = m, q.sa1 = n * m;
        q.B = b.data;
        if (r.op == OP_BMM) {  // da = g @ b^T, b [Z, k, m]
          q.ldb = m, q.b_kcontig = true, q.sb1 = k * m;
        } else {               // da = g @ b, b [Z, m, k]
          q.ldb = k, q.sb1 = m * k;
        }
        q.C = da.first, q.ldc = k, q.sc1 = n * k;
        q.beta = da.second, q.batch = (int)Z;
        C.run_gemm(q);
      }
      auto db = C.gdst(r.in[1]);
      {
        GemmArgs q = C.gemm_base();
        q.batch = (int)Z;
        q.beta = db.second;
        if (r.op == OP_BMM) {  // db [k, m] = a^T @ g
          q.M = (int)k, q.N = (int)m, q.K = (int)n;
          q.A = a.data, q.lda = k, q.a_mcontig = true, q.sa1 = n * k;
          q.B = g, q.ldb = m, q.sb1 = n * m;
          q.C = db.first, q.ldc = m, q.sc1 = k * m;
        } else {               // db [m, k] = g^T @ a
          q.M = (int)m, q.N = (int)k, q.K = (int)n;
          q.A = g, q.lda = m, q.a_mcontig = true, q.sa1 = n * m;
          q.B = a.data, q.ldb = k, q.sb1 = n * k;
          q.C = db.first, q.ldc = k, q.sc1 = m * k;
        }
        C.run_gemm(q);
      }
      break;
    }
    case OP_CSOFTMAX: {
      auto dx = C.gdst(r.in[0]);
      hip_check(causal_softmax_bwd(g, out.data, dx.first, out.rows(), out.cols(), 1.f, dx.second, true, s),
                "causal_softmax bwd");
      break;
    }
    case OP_ATTENTION: {
      TensorRec& qkv = C.T(r.in[0]);
      const int64_t B = qkv.shape[0], T = qkv.shape[1], C3 = qkv.shape[2], Cc = C3 / 3, H = r.i0, hs = Cc / H;
      const float scale = r.f;
      if (r.i1 == 1) {  // fused kernels: recompute probabilities from the saved log-sum-exp
        const uint16_t* qb = C.data_bf16(qkv);
        const uint16_t* dyb = C.grad_bf16(out);
        // D from the fp32 output and gradient where both exist, else from their bf16 copies
        const float* yf = out.f32_valid ? out.data : nullptr;
        const float* dyf = out.gstate == G_BF16 ? nullptr : g;
        auto dq = C.gdst(r.in[0]);
        uint16_t* dqb = C.twin_grad(qkv);
        // a bf16-only qkv whose one gradient its Linear reads as bf16 (with the bias
        // gradient summed from that copy): the copy alone
        const bool only = dqb && dq.second == 0.f && qkv.uses == 1 && !qkv.leaf && qkv.bf16_out &&
                          qkv.cols() % 4 == 0 && C.grad_read_as_bf16(qkv);
        size_t mark = C.c->arena.hi;
        float* D = static_cast<float*>(C.scratch((size_t)B * H * T * sizeof(float)));
        // the method's four backward products over the causal triangle
        const double flops = 4.0 * 2.0 * hs * (T * (T + 1.0) / 2.0) * B * H;
        C.timed(TFB_PROF_ATTN_BWD, flops, [&] {
          hip_check(flash_attention_bwd(qb, yf, dyf, dyb, static_cast<const float*>(r.s1), D,
                                        only ? nullptr : dq.first, dqb, dq.second, (int)B, (int)T, (int)H, (int)Cc,
                                        scale, s, out.bf),
                    "attention bwd");
        });
        C.c->arena.hi = mark;
        qkv.gbf_valid = true;
        if (only) qkv.gstate = G_BF16;
        break;
      }
      float* P = static_cast<float*>(r.s0);
      // the gradient buffer first: it must outlive the scratch released below
      auto dq = C.gdst(r.in[0]);
      float* dqkv = dq.first;
      size_t mark = C.c->arena.hi;
      float* dP = static_cast<float*>(C.scratch((size_t)B * H * T * T * sizeof(float)));
      const float* q = qkv.data;
      {  // dP = dY_h @ V_h^T (lower triangle of tiles)
        GemmArgs a = C.gemm_base();
        a.M = (int)T, a.N = (int)T, a.K = (int)hs;
        a.A = g, a.lda = Cc, a.sa1 = T * Cc, a.sa2 = hs;
        a.B = q + 2 * Cc, a.ldb = C3, a.b_kcontig = true, a.sb1 = T * C3, a.sb2 = hs;
        a.C = dP, a.ldc = T, a.sc1 = H * T * T, a.sc2 = T * T;
        a.batch = (int)(B * H), a.batch_div = (int)H;
        a.causal_out = true;
        C.run_gemm(a);
      }
      // dS = scale * P (dP - rowsum(P dP)), in place, visible part only
      hip_check(causal_softmax_bwd(dP, P, dP, B * H * T, T, scale, 0.f, false, s), "attention softmax bwd");
      {  // dQ = dS @ K
        GemmArgs a = C.gemm_base();
        a.M = (int)T, a.N = (int)hs, a.K = (int)T;
        a.A = dP, a.lda = T, a.sa1 = H * T * T, a.sa2 = T * T, a.causal_a = CAUSAL_UPTO;
        a.B = q + Cc, a.ldb = C3, a.sb1 = T * C3, a.sb2 = hs;
        a.C = dqkv, a.ldc = C3, a.sc1 = T * C3, a.sc2 = hs;
        a.beta = dq.second, a.batch = (int)(B * H), a.batch_div = (int)H;
        C.run_gemm(a);
      }
      {  // dK = dS^T @ Q
        GemmArgs a = C.gemm_base();
        a.M = (int)T, a.N = (int)hs, a.K = (int)T;
        a.A = dP, a.lda = T, a.a_mcontig = true, a.sa1 = H * T * T, a.sa2 = T * T, a.causal_a = CAUSAL_FROM;
        a.B = q, a.ldb = C3, a.sb1 = T * C3, a.sb2 = hs;
        a.C = dqkv + Cc, a.ldc = C3, a.sc1 = T * C3, a.sc2 = hs;
        a.beta = dq.second, a.batch = (int)(B * H), a.batch_div = (int)H;
        C.run_gemm(a);
      }
      {  // dV = P^T @ dY_h
        GemmArgs a = C.gemm_base();
        a.M = (int)T, a.N = (int)hs, a.K = (int)T;
        a.A = P, a.lda = T, a.a_mcontig = true, a.sa1 = H * T * T, a.sa2 = T * T, a.causal_a = CAUSAL_FROM;
        a.B = g, a.ldb = Cc, a.sb1 = T * Cc, a.sb2 = hs;
        a.C = dqkv + 2 * Cc, a.ldc = C3, a.sc1 = T * C3, a.sc2 = hs;
        a.beta = dq.second, a.batch = (int)(B * H), a.batch_div = (int)H;
        C.run_gemm(a);
      }
      C.c->arena.hi = mark;
      break;
    }
    case OP_SOFTMAX_CE: {
      TensorRec& lg = C.T(r.in[0]);
      // logits held only as bf16 are read as such
      const uint16_t* lgb = !lg.f32_valid && softmax_ce_bf16_fits(lg.stride(), lg.cols(), lg.bf) ? lg.bf : nullptr;
      const float* lgd = lgb ? nullptr : C.f32(lg);
      if ((r.i0 & TFB_CE_GRAD_BF16_ONLY) && lg.uses == 1 && !lg.leaf && !lg.gpend && lg.gstate != G_VALID &&
          C.grad_read_as_bf16(lg)) {
        // the logits' only gradient, read by their producer as bf16: that copy alone
        // (written by the forward already when r.i1 == 1: then only for g != 1)
        uint16_t* dlb = C.twin_grad(lg);
        // when the forward wrote the gradient this launch only checks g == 1 on the device
        const double bytes = r.i1 == 1 ? 0.0 : (double)lg.rows() * lg.cols() * ((lgb ? 2 : 4) + 2);
        C.timed(TFB_PROF_CE, bytes, [&] {
          hip_check(softmax_ce_bwd(lgd, lg.stride(), static_cast<const int32_t*>(r.s0),
                                   static_cast<const float*>(r.s1), g, nullptr, dlb, lg.rows(), lg.cols(), 0.f, s,
                                   r.i1 == 1, lgb),
                    "softmax_ce bwd");
        });
        lg.gstate = G_BF16;
        lg.gbf_valid = true;
        break;
      }
      auto dl = C.gdst(r.in[0]);
      uint16_t* dlb = C.twin_grad(lg);
      const double bytes = (double)lg.rows() * lg.cols() *
                           ((lgb ? 2 : 4) + 4 + (dl.second != 0.f ? 4 : 0) + (dlb ? 2 : 0));
      C.timed(TFB_PROF_CE, bytes, [&] {
        hip_check(softmax_ce_bwd(lgd, lg.stride(), static_cast<const int32_t*>(r.s0),
                                 static_cast<const float*>(r.s1), g, dl.first, dlb, lg.rows(), lg.cols(), dl.second,
                                 s, false, lgb),
                  "softmax_ce bwd");
      });
      if (dlb) lg.gbf_valid = true;
      break;
    }
    case OP_COMPACT: {
      TensorRec& x = C.T(r.in[0]);
      auto dx = C.gdst(r.in[0]);
      hip_check(copy_pitched(g, out.cols(), dx.first, x.stride(), x.rows(), x.cols(), dx.second, s), "compact bwd");
      break;
    }
  }
}

}  // namespace

// ==================================================================== C ABI
// for entry points defined in other sources (noalloc.hip): record the calling
// thread's error text and return the code
LaunchEvents& tfb::launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}

int tfb::set_last_error(int code, const char* msg) {
  g_last_error = msg ? msg : "";
  return code;
}

extern "C" {

const char* tfb_last_error(void) { return g_last_error.c_str(); }

int tfb_init(tfb_ctx** out, int device, void* hip_stream, void* arena, size_t arena_bytes, int precision) {
  return guarded([&] {
    need(out != nullptr, TFB_ERR_ARG, "null output pointer");
    need(arena != nullptr && arena_bytes >= ALIGN, TFB_ERR_ARG, "arena must be a device buffer of at least 256 bytes");
    need((reinterpret_cast<uintptr_t>(arena) & (ALIGN - 1)) == 0, TFB_ERR_ARG, "arena must be 256-byte aligned");
    need(precision == TFB_FP32 || precision == TFB_BF16_MFMA, TFB_ERR_ARG, "unknown precision");
    int n = 0;
    hip_check(hipGetDeviceCount(&n), "hipGetDeviceCount");
    need(device >= 0 && device < n, TFB_ERR_ARG, "no such device");
    hip_check(hipSetDevice(device), "hipSetDevice");
    tfb_ctx* c = new tfb_ctx();
    c->device = device;
    c->stream = static_cast<hipStream_t>(hip_stream);
    c->arena.base = static_cast<char*>(arena);
    c->arena.size = arena_bytes / ALIGN * ALIGN;
    c->arena.lo = 0;
    c->arena.hi = c->arena.size;
    c->precision = precision;
    *out = c;
  });
}

int tfb_destroy(tfb_ctx* ctx) {
  return guarded([&] {
    need(ctx != nullptr, TFB_ERR_ARG, "null context");
    (void)hipSetDevice(ctx->device);
    (void)hipStreamSynchronize(ctx->stream);
    for (hipEvent_t e : ctx->prof.pool) (void)hipEventDestroy(e);
    delete ctx;
  });
}

int tfb_set_precision(tfb_ctx* ctx, int precision) {
  return guarded([&] {
    need(ctx != nullptr, TFB_ERR_ARG, "null context");
    need(precision == TFB_FP32 || precision == TFB_BF16_MFMA, TFB_ERR_ARG, "unknown precision");
    ctx->precision = precision;
  });
}

int tfb_set_grad_enabled(tfb_ctx* ctx, int enabled) {
  return guarded([&] {
    need(ctx != nullptr, TFB_ERR_ARG, "null context");
    ctx->grad_enabled = enabled != 0;
  });
}

int tfb_sync(tfb_ctx* ctx) {
  return guarded([&] {
    Ctx C(ctx);
    hip_check(hipStreamSynchronize(C.s()), "stream synchronize");
    hip_check(hipGetLastError(), "last error");
  });
}

int tfb_arena_usage(tfb_ctx* ctx, size_t* persistent, size_t* step) {
  return guarded([&] {
    need(ctx != nullptr, TFB_ERR_ARG, "null context");
    if (persistent) *persistent = ctx->arena.lo;
    if (step) *step = ctx->arena.size - ctx->arena.hi;
  });
}

int tfb_tensor_create(tfb_ctx* ctx, const int64_t* shape, int ndim, void* dev_ptr, int is_param, const char* name,
                      tfb_tensor* out) {
  return guarded([&] {
    Ctx C(ctx);
    need(shape != nullptr && out != nullptr, TFB_ERR_ARG, "null argument");
    int64_t n = Ctx::numel_of(shape, ndim);
    need(dev_ptr == nullptr || (reinterpret_cast<uintptr_t>(dev_ptr) & (ALIGN - 1)) == 0, TFB_ERR_ARG,
         "borrowed tensor memory must be 256-byte aligned");
    float* p;
    size_t off = 0, bytes = 0;
    if (dev_ptr) {
      p = static_cast<float*>(dev_ptr);
    } else {
      bytes = (size_t)n * sizeof(float);
      off = ctx->arena.alloc_persist(bytes);
      p = reinterpret_cast<float*>(ctx->arena.base + off);
      hip_check(fill(p, 0.f, n, C.s()), "zero fill");
    }
    int h = C.new_handle();
    TensorRec& t = ctx->tensors[h];
    t.live = true;
    t.leaf = true;
    t.is_param = is_param != 0;
    t.ndim = ndim;
    for (int i = 0; i < ndim; ++i) t.shape[i] = shape[i];
    t.numel = n;
    t.data = p;
    t.owns_persistent = dev_ptr == nullptr;
    t.persist_off = off;
    t.persist_bytes = Arena::up(std::max<size_t>(bytes, 1));
    t.name = name ? std::string(name).substr(0, TFB_MAX_NAME - 1) : std::string();
    *out = h;
  });
}

int tfb_tensor_name(tfb_ctx* ctx, tfb_tensor h, char* buf, size_t cap) {
  return guarded([&] {
    Ctx C(ctx);
    need(buf != nullptr && cap > 0, TFB_ERR_ARG, "null or empty name buffer");
    const std::string& n = C.T(h).name;
    const size_t k = std::min(n.size(), cap - 1);
    std::memcpy(buf, n.data(), k);
    buf[k] = 0;
  });
}

int tfb_tensor_info(tfb_ctx* ctx, tfb_tensor h, int64_t* shape, int* ndim, void** data, void** grad) {
  return guarded([&] {
    Ctx C(ctx);
    TensorRec& t = C.T(h);
    if (shape)
      for (int i = 0; i < t.ndim; ++i) shape[i] = t.shape[i];
    if (ndim) *ndim = t.ndim;
    if (data) *data = const_cast<float*>(C.f32(t));
    if (grad) {
      C.materialize_zero(t);
      *grad = t.grad;
    }
  });
}

int tfb_tensor_write(tfb_ctx* ctx, tfb_tensor h, const float* src, int64_t n) {
  return guarded([&] {
    Ctx C(ctx);
    TensorRec& t = C.T(h);
    need(src != nullptr && n == t.numel, TFB_ERR_SHAPE, "write of " + std::to_string(n) + " floats into " +
                                                            shape_str(t));
    if (t.padded())
      hip_check(hipMemcpy2DAsync(t.data, t.ld * sizeof(float), src, t.cols() * sizeof(float),
                                 t.cols() * sizeof(float), t.rows(), hipMemcpyHostToDevice, C.s()),
                "copy in");
    else
      hip_check(hipMemcpyAsync(t.data, src, (size_t)n * sizeof(float), hipMemcpyHostToDevice, C.s()), "copy in");
    t.bf_valid = false;
    t.f32_valid = true;
    hip_check(hipStreamSynchronize(C.s()), "sync");
  });
}

int tfb_tensor_read(tfb_ctx* ctx, tfb_tensor h, int which, float* dst, int64_t n) {
  return guarded([&] {
    Ctx C(ctx);
    TensorRec& t = C.T(h);
    need(dst != nullptr && n == t.numel, TFB_ERR_SHAPE, "read of " + std::to_string(n) + " floats from " +
                                                            shape_str(t));
    need(which == 0 || which == 1, TFB_ERR_ARG, "which must be 0 (data) or 1 (grad)");
    const float* src = which == 0 ? C.f32(t) : t.data;
    if (which == 1) {
      need(t.gstate != G_BF16, TFB_ERR_STATE, "the gradient was kept only as its bf16 copy");
      need(t.grad != nullptr, TFB_ERR_STATE, "tensor has no gradient");
      C.materialize_zero(t);
      src = t.grad;
    }
    if (t.padded())
      hip_check(hipMemcpy2DAsync(dst, t.cols() * sizeof(float), src, t.ld * sizeof(float), t.cols() * sizeof(float),
                                 t.rows(), hipMemcpyDeviceToHost, C.s()),
                "copy out");
    else
      hip_check(hipMemcpyAsync(dst, src, (size_t)n * sizeof(float), hipMemcpyDeviceToHost, C.s()), "copy out");
    hip_check(hipStreamSynchronize(C.s()), "sync");
  });
}

int tfb_tensor_release(tfb_ctx* ctx, tfb_tensor h) {
  return guarded([&] {
    Ctx C(ctx);
    TensorRec& t = C.T(h);
    need(t.leaf, TFB_ERR_STATE, "op outputs are released by tfb_tape_reset");
    for (const Rec& r : ctx->tape)
      for (int i : r.in)
        need(i != h, TFB_ERR_STATE, "tensor is still referenced by the tape");
    // a leaf's memory returns only from the top of the persistent end (an optimizer
    // may still hold its address); a hole it leaves below is never reused
    if (t.owns_persistent && t.persist_off + t.persist_bytes == ctx->arena.lo)
      ctx->arena.release_persist(t.persist_off, t.persist_bytes);
    t.live = false;
    ctx->free_handles.push_back(h);
  });
}

// ------------------------------------------------------------------ ops
int tfb_add(tfb_ctx* ctx, tfb_tensor a, tfb_tensor b, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    a = C.dense_in(a), b = C.dense_in(b);
    TensorRec& A = C.T(a);
    TensorRec& B = C.T(b);
    need(y != nullptr, TFB_ERR_ARG, "null output");
    bool ok = B.ndim <= A.ndim;
    for (int i = 0; ok && i < B.ndim; ++i) ok = A.shape[A.ndim - B.ndim + i] == B.shape[i];
    need(ok, TFB_ERR_SHAPE, "add: " + shape_str(B) + " must equal the trailing dims of " + shape_str(A));
    int h = C.make_output(shape_vec(A));
    TensorRec& Y = ctx->tensors[h];
    const float* ad = ctx->tensors[a].data;
    const float* bd = ctx->tensors[b].data;
    hip_check(add_bcast(ad, bd, Y.data, Y.numel, ctx->tensors[b].numel, C.s()), "add");
    Rec r{OP_ADD};
    r.in[0] = a, r.in[1] = b, r.out = h;
    C.record(r);
    *y = h;
  });
}

int tfb_mul(tfb_ctx* ctx, tfb_tensor a, tfb_tensor b, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    a = C.dense_in(a), b = C.dense_in(b);
    TensorRec& A = C.T(a);
    TensorRec& B = C.T(b);
    need(y != nullptr, TFB_ERR_ARG, "null output");
    need(A.numel == B.numel, TFB_ERR_SHAPE, "shapes differ: " + shape_str(A) + " " + shape_str(B));
    int h = C.make_output(shape_vec(A));
    hip_check(mul_fwd(ctx->tensors[a].data, ctx->tensors[b].data, ctx->tensors[h].data, ctx->tensors[h].numel, C.s()),
              "mul");
    Rec r{OP_MUL};
    r.in[0] = a, r.in[1] = b, r.out = h;
    C.record(r);
    *y = h;
  });
}

int tfb_scale(tfb_ctx* ctx, tfb_tensor a, float sc, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    a = C.dense_in(a);
    TensorRec& A = C.T(a);
    need(y != nullptr, TFB_ERR_ARG, "null output");
    int h = C.make_output(shape_vec(A));
    hip_check(scale_fwd(ctx->tensors[a].data, sc, ctx->tensors[h].data, ctx->tensors[h].numel, C.s()), "scale");
    Rec r{OP_SCALE};
    r.in[0] = a, r.out = h, r.f = sc;
    C.record(r);
    *y = h;
  });
}

int tfb_sum(tfb_ctx* ctx, tfb_tensor a, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    a = C.dense_in(a);
    C.T(a);
    need(y != nullptr, TFB_ERR_ARG, "null output");
    int h = C.make_output({1});
    size_t mark = ctx->arena.hi;
    void* ws = C.scratch(sum_workspace_bytes(ctx->tensors[a].numel));
    hip_check(sum_all(ctx->tensors[a].data, ctx->tensors[a].numel, ctx->tensors[h].data, ws, C.s()), "sum");
    ctx->arena.hi = mark;
    Rec r{OP_SUM};
    r.in[0] = a, r.out = h;
    C.record(r);
    *y = h;
  });
}

int tfb_reshape(tfb_ctx* ctx, tfb_tensor a, const int64_t* shape, int ndim, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    a = C.dense_in(a);
    TensorRec& A = C.T(a);
    need(y != nullptr && shape != nullptr, TFB_ERR_ARG, "null argument");
    int64_t n = Ctx::numel_of(shape, ndim);
    need(n == A.numel, TFB_ERR_SHAPE, "reshape changes the size of " + shape_str(A));
    float* data = A.data;
    int h = C.new_handle();
    TensorRec& t = ctx->tensors[h];
    t.live = true;
    t.leaf = false;
    t.ndim = ndim;
    for (int i = 0; i < ndim; ++i) t.shape[i] = shape[i];
    t.numel = n;
    t.data = data;  // a view of the same data
    Rec r{OP_RESHAPE};
    r.in[0] = a, r.out = h;
    C.record(r);
    *y = h;
  });
}

int tfb_tanh(tfb_ctx* ctx, tfb_tensor a, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    a = C.dense_in(a);
    TensorRec& A = C.T(a);
    need(y != nullptr, TFB_ERR_ARG, "null output");
    int h = C.make_output(shape_vec(A));
    hip_check(tanh_fwd(ctx->tensors[a].data, ctx->tensors[h].data, ctx->tensors[h].numel, C.s()), "tanh");
    Rec r{OP_TANH};
    r.in[0] = a, r.out = h;
    C.record(r);
    *y = h;
  });
}

int tfb_gelu(tfb_ctx* ctx, tfb_tensor a, tfb_tensor* y) { return tfb_gelu_ex(ctx, a, 0, y); }

int tfb_gelu_ex(tfb_ctx* ctx, tfb_tensor a, int flags, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    need((flags & ~TFB_OUT_BF16_ONLY) == 0, TFB_ERR_ARG, "unknown tfb_gelu_ex flags");
    a = C.dense_in(a, C.bf16_mode());  // an input held only as bf16 is read as such
    TensorRec& A = C.T(a);
    need(y != nullptr, TFB_ERR_ARG, "null output");
    int h = C.make_output(shape_vec(A));
    uint16_t* yb = C.twin_data(ctx->tensors[h]);
    const bool only = yb && (flags & TFB_OUT_BF16_ONLY);
    float* yd = only ? nullptr : ctx->tensors[h].data;
    const bool abf = !ctx->tensors[a].f32_valid;
    const double bytes = (double)ctx->tensors[h].numel * ((abf ? 2 : 4) + (yd ? 4 : 0) + (yb ? 2 : 0));
    C.timed(TFB_PROF_GELU_FWD, bytes, [&] {
      if (abf)
        hip_check(gelu_fwd_bf(ctx->tensors[a].bf, yd, yb, ctx->tensors[h].numel, C.s()), "gelu");
      else
        hip_check(gelu_fwd(ctx->tensors[a].data, yd, yb, ctx->tensors[h].numel, C.s()), "gelu");
    });
    if (yb) ctx->tensors[h].bf_valid = true;
    if (only) ctx->tensors[h].f32_valid = false, ctx->tensors[h].bf16_out = true;
    Rec r{OP_GELU};
    r.in[0] = a, r.out = h;
    C.record(r);
    *y = h;
  });
}

static int matmul_impl(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, tfb_tensor b, tfb_tensor* y, OpKind kind,
                       int out_flags = 0, tfb_tensor res = -1) {
  return guarded([&] {
    Ctx C(ctx);
    // the contraction reads x and w as bf16 copies in the bf16 variant
    x = C.dense_in(x, C.bf16_mode()), w = C.dense_in(w, C.bf16_mode());
    if (kind != OP_MATMUL && kind != OP_MATMUL_T) b = C.dense_in(b);
    if (kind == OP_LINEAR_RES) res = C.dense_in(res);
    TensorRec& X = C.T(x);
    TensorRec& W = C.T(w);
    need(y != nullptr, TFB_ERR_ARG, "null output");
    need(W.ndim == 2, TFB_ERR_SHAPE, "matmul weight must be 2-D, got " + shape_str(W));
    const int64_t K = X.cols(), rows = X.rows();
    int64_t N;
    if (kind == OP_MATMUL_T) {
      need(W.shape[1] == K, TFB_ERR_SHAPE, "matmul_t " + shape_str(X) + " @ " + shape_str(W) + "^T");
      N = W.shape[0];
    } else {
      need(W.shape[0] == K, TFB_ERR_SHAPE, "matmul " + shape_str(X) + " @ " + shape_str(W));
      N = W.shape[1];
    }
    const float* bias = nullptr;
    if (kind == OP_LINEAR || kind == OP_LINEAR_RES) {
      TensorRec& Bv = C.T(b);
      need(Bv.numel == N && Bv.ndim == 1, TFB_ERR_SHAPE, "linear bias must be [" + std::to_string(N) + "]");
      bias = Bv.data;
    }
    const float* rd = nullptr;
    if (kind == OP_LINEAR_RES) {
      TensorRec& R = C.T(res);
      need(R.numel == X.rows() * N && R.cols() == N, TFB_ERR_SHAPE,
           "residual must have the output's shape: " + shape_str(R) + " for [" + std::to_string(X.rows()) + ", " +
               std::to_string(N) + "]");
      rd = R.data;
    }
    check_gemm_dims(rows, K, N);
    std::vector<int64_t> shp = shape_vec(X);
    shp.back() = N;
    // a vocabulary-sized LM-head output gets rows padded to a multiple of 64
    // floats so that its rows (and its gradient's) stay 16-byte aligned
    const int64_t ld = (kind == OP_MATMUL_T && N % 64 != 0 && N >= 1024) ? (N + 63) / 64 * 64 : 0;
    int h = C.make_output(shp, ld);
    float* yd = ctx->tensors[h].data;
    const float* xd = ctx->tensors[x].data;
    const float* wd = ctx->tensors[w].data;
    // a product of at most 16 rows whose input has no bf16 copy yet (the cached
    // attention's output in decoding) rounds the fp32 input as it loads it: the same
    // values without a conversion launch
    const bool round_on_load = C.bf16_mode() && kind != OP_MATMUL_T && rows <= 16 && !ctx->tensors[x].bf_valid &&
                               ctx->tensors[x].f32_valid;
    const Opnd xo = round_on_load ? Opnd{C.f32(ctx->tensors[x]), false} : op_data(C, ctx->tensors[x]);
    const Opnd wo = op_data(C, ctx->tensors[w]);
    (void)xd, (void)wd;
    uint16_t* yb = out_flags ? C.twin_data(ctx->tensors[h]) : nullptr;
    const bool only = yb && (out_flags & TFB_OUT_BF16_ONLY);
    if (kind == OP_MATMUL_T)
      gemm_nt(C, xo, wo, yd, rows, K, N, 0.f, ld ? ld : N, yb, only);
    else
      gemm_nn(C, xo, wo, yd, rows, K, N, 0.f, bias, -1, yb, rd, only);
    if (yb) ctx->tensors[h].bf_valid = true;
    if (only) ctx->tensors[h].f32_valid = false, ctx->tensors[h].bf16_out = true;
    Rec r{kind};
    r.in[0] = x, r.in[1] = w, r.in[2] = (kind == OP_LINEAR || kind == OP_LINEAR_RES) ? b : -1, r.out = h;
    if (kind == OP_LINEAR_RES) r.in[3] = res;
    C.record(r);
    *y = h;
  });
}

int tfb_matmul(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, tfb_tensor* y) {
  return matmul_impl(ctx, x, w, -1, y, OP_MATMUL);
}
int tfb_matmul_t(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, tfb_tensor* y) {
  return matmul_impl(ctx, x, w, -1, y, OP_MATMUL_T);
}
int tfb_matmul_t_ex(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, int flags, tfb_tensor* y) {
  if (flags & ~(TFB_OUT_BF16_COPY | TFB_OUT_BF16_ONLY))
    return guarded([&] { need(false, TFB_ERR_ARG, "unknown tfb_matmul_t_ex flags"); });
  return matmul_impl(ctx, x, w, -1, y, OP_MATMUL_T, flags);
}
int tfb_linear(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, tfb_tensor b, tfb_tensor* y) {
  return matmul_impl(ctx, x, w, b, y, OP_LINEAR);
}

int tfb_linear_residual(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, tfb_tensor b, tfb_tensor r, tfb_tensor* y) {
  return matmul_impl(ctx, x, w, b, y, OP_LINEAR_RES, 0, r);
}

int tfb_linear_ex(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, tfb_tensor b, int flags, tfb_tensor* y) {
  if (flags & ~(TFB_OUT_BF16_COPY | TFB_OUT_BF16_ONLY))
    return guarded([&] { need(false, TFB_ERR_ARG, "unknown tfb_linear_ex flags"); });
  return matmul_impl(ctx, x, w, b, y, OP_LINEAR, flags);
}

// ------------------------------------------------------------------ inference fusions
// A Linear of at most 16 rows with its consumer folded into the chunk sum of the
// few-row product (gemv.hip): GELU, or the residual Add followed by LayerNorm.  Both
// are inference-only (nothing is recorded); where the few-row kernel does not take
// the product they run as the separate ops, with the same results up to rounding.
}  // extern "C"

namespace {

// The few-row product y = x @ w + b (+ resid) with the epilogue `post`, its output
// pointers still unset; `ok` says whether the few-row kernel takes it (checked with
// 256-byte aligned stand-ins for the outputs, which the step arena gives them).
GemmArgs linear_post_args(Ctx& C, int x, int w, int b, int res, int post, const float* ln_gamma,
                          const float* ln_beta, bool* ok) {
  TensorRec& X = C.T(x);
  TensorRec& W = C.T(w);
  const int64_t K = X.cols(), rows = X.rows(), N = W.shape[1];
  const bool round_on_load = C.bf16_mode() && rows <= 16 && !X.bf_valid && X.f32_valid;
  const Opnd xo = round_on_load ? Opnd{C.f32(X), false} : op_data(C, X);
  const Opnd wo = op_data(C, W);
  GemmArgs g = C.gemm_base();
  g.M = (int)rows, g.N = (int)N, g.K = (int)K;
  set_a(g, xo), g.lda = K;
  set_b(g, wo), g.ldb = N;
  g.ldc = N;
  g.bias = C.T(b).data;
  g.resid = res >= 0 ? C.f32(C.T(res)) : nullptr;
  g.post = post, g.ln_gamma = ln_gamma, g.ln_beta = ln_beta;
  float* stand_in = reinterpret_cast<float*>(C.c->arena.base);
  g.C = stand_in;
  if (post == POST_LN) g.ln_y = stand_in;
  *ok = gemv_accepts(g);
  return g;
}

void check_linear(Ctx& C, int x, int w, int b) {
  TensorRec& X = C.T(x);
  TensorRec& W = C.T(w);
  need(W.ndim == 2 && W.shape[0] == X.cols(), TFB_ERR_SHAPE, "matmul " + shape_str(X) + " @ " + shape_str(W));
  need(C.T(b).numel == W.shape[1] && C.T(b).ndim == 1, TFB_ERR_SHAPE,
       "linear bias must be [" + std::to_string(W.shape[1]) + "]");
  check_gemm_dims(X.rows(), X.cols(), W.shape[1]);
}

[[noreturn]] void rethrow(int rc) { fail(rc, g_last_error); }

}  // namespace

extern "C" {

int tfb_linear_gelu(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, tfb_tensor b, int flags, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    need((flags & ~TFB_OUT_BF16_ONLY) == 0, TFB_ERR_ARG, "unknown tfb_linear_gelu flags");
    need(!ctx->grad_enabled, TFB_ERR_STATE, "tfb_linear_gelu is inference-only: disable gradients first");
    need(y != nullptr, TFB_ERR_ARG, "null output");
    x = C.dense_in(x, C.bf16_mode()), w = C.dense_in(w, C.bf16_mode()), b = C.dense_in(b);
    check_linear(C, x, w, b);
    std::vector<int64_t> shp = shape_vec(C.T(x));
    shp.back() = C.T(w).shape[1];
    bool ok = false;
    GemmArgs g = linear_post_args(C, x, w, b, -1, POST_GELU, nullptr, nullptr, &ok);
    if (ok) {
      int h = C.make_output(shp);
      uint16_t* yb = C.twin_data(ctx->tensors[h]);
      const bool only = yb && (flags & TFB_OUT_BF16_ONLY);
      g.C = ctx->tensors[h].data, g.Cbf = yb, g.c_bf16_only = only;
      C.run_gemm(g);
      if (yb) ctx->tensors[h].bf_valid = true;
      if (only) ctx->tensors[h].f32_valid = false, ctx->tensors[h].bf16_out = true;
      *y = h;
      return;
    }
    tfb_tensor l;
    int rc = tfb_linear_ex(ctx, x, w, b, flags, &l);
    if (rc) rethrow(rc);
    rc = tfb_gelu_ex(ctx, l, flags, y);
    if (rc) rethrow(rc);
  });
}

int tfb_linear_residual_layernorm(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w, tfb_tensor b, tfb_tensor r,
                                  tfb_tensor gamma, tfb_tensor beta, float eps, int flags, tfb_tensor* y,
                                  tfb_tensor* h) {
  return guarded([&] {
    Ctx C(ctx);
    need((flags & ~TFB_OUT_BF16_ONLY) == 0, TFB_ERR_ARG, "unknown tfb_linear_residual_layernorm flags");
    need(!ctx->grad_enabled, TFB_ERR_STATE,
         "tfb_linear_residual_layernorm is inference-only: disable gradients first");
    need(y != nullptr && h != nullptr, TFB_ERR_ARG, "null output");
    x = C.dense_in(x, C.bf16_mode()), w = C.dense_in(w, C.bf16_mode()), b = C.dense_in(b);
    r = C.dense_in(r), gamma = C.dense_in(gamma), beta = C.dense_in(beta);
    check_linear(C, x, w, b);
    const int64_t N = C.T(w).shape[1];
    need(C.T(r).numel == C.T(x).rows() * N && C.T(r).cols() == N, TFB_ERR_SHAPE,
         "residual must have the output's shape, got " + shape_str(C.T(r)));
    need(C.T(gamma).numel == N && C.T(beta).numel == N, TFB_ERR_SHAPE,
         "layernorm gain/shift must have " + std::to_string(N) + " elements");
    need(N <= 2048, TFB_ERR_SHAPE, "layernorm rows longer than 2048 are not supported");
    std::vector<int64_t> shp = shape_vec(C.T(x));
    shp.back() = N;
    bool ok = false;
    GemmArgs g = linear_post_args(C, x, w, b, r, POST_LN, C.T(gamma).data, C.T(beta).data, &ok);
    if (ok) {
      int yh = C.make_output(shp);
      int hh = C.make_output(shp);
      uint16_t* hb = C.twin_data(ctx->tensors[hh]);
      const bool only = hb && (flags & TFB_OUT_BF16_ONLY);
      g.C = ctx->tensors[yh].data;
      g.ln_eps = eps;
      g.ln_y = only ? nullptr : ctx->tensors[hh].data, g.ln_ybf = hb;
      C.run_gemm(g);
      if (hb) ctx->tensors[hh].bf_valid = true;
      if (only) ctx->tensors[hh].f32_valid = false, ctx->tensors[hh].bf16_out = true;
      *y = yh, *h = hh;
      return;
    }
    int rc = tfb_linear_residual(ctx, x, w, b, r, y);
    if (rc) rethrow(rc);
    rc = tfb_layernorm_ex(ctx, *y, gamma, beta, eps, flags, h);
    if (rc) rethrow(rc);
  });
}

int tfb_mlp_residual_layernorm(tfb_ctx* ctx, tfb_tensor x, tfb_tensor w_fc, tfb_tensor b_fc, tfb_tensor w_proj,
                               tfb_tensor b_proj, tfb_tensor r, tfb_tensor gamma, tfb_tensor beta, float eps, int flags,
                               tfb_tensor* y, tfb_tensor* h) {
  return guarded([&] {
    Ctx C(ctx);
    need((flags & ~TFB_OUT_BF16_ONLY) == 0, TFB_ERR_ARG, "unknown tfb_mlp_residual_layernorm flags");
    need(!ctx->grad_enabled, TFB_ERR_STATE, "tfb_mlp_residual_layernorm is inference-only: disable gradients first");
    need(y != nullptr && h != nullptr, TFB_ERR_ARG, "null output");
    x = C.dense_in(x, C.bf16_mode()), w_fc = C.dense_in(w_fc, C.bf16_mode()), b_fc = C.dense_in(b_fc);
    w_proj = C.dense_in(w_proj, C.bf16_mode()), b_proj = C.dense_in(b_proj);
    r = C.dense_in(r), gamma = C.dense_in(gamma), beta = C.dense_in(beta);
    check_linear(C, x, w_fc, b_fc);
    const int64_t F = C.T(w_fc).shape[1];
    need(C.T(w_proj).ndim == 2 && C.T(w_proj).shape[0] == F, TFB_ERR_SHAPE,
         "mlp projection must be [" + std::to_string(F) + ", N], got " + shape_str(C.T(w_proj)));
    const int64_t N = C.T(w_proj).shape[1];
    need(C.T(b_proj).numel == N && C.T(b_proj).ndim == 1, TFB_ERR_SHAPE,
         "linear bias must be [" + std::to_string(N) + "]");
    need(C.T(r).numel == C.T(x).rows() * N && C.T(r).cols() == N, TFB_ERR_SHAPE,
         "residual must have the output's shape, got " + shape_str(C.T(r)));
    need(C.T(gamma).numel == N && C.T(beta).numel == N, TFB_ERR_SHAPE,
         "layernorm gain/shift must have " + std::to_string(N) + " elements");
    need(N <= 2048, TFB_ERR_SHAPE, "layernorm rows longer than 2048 are not supported");
    // the c_fc product leaves its partials; the projection sums them (+ bias, GELU) as
    // it loads its input, then normalises its own chunk sum
    bool ok1 = false;
    GemmArgs g1 = linear_post_args(C, x, w_fc, b_fc, -1, POST_PARTIALS, nullptr, nullptr, &ok1);
    g1.bias = nullptr;
    ok1 = gemv_accepts(g1);
    GemmArgs g2 = C.gemm_base();
    const int64_t rows = C.T(x).rows();
    g2.M = (int)rows, g2.N = (int)N, g2.K = (int)F;
    set_b(g2, op_data(C, C.T(w_proj))), g2.ldb = N;
    g2.ldc = N, g2.bias = C.T(b_proj).data, g2.resid = C.f32(C.T(r));
    g2.post = POST_LN, g2.ln_gamma = C.T(gamma).data, g2.ln_beta = C.T(beta).data, g2.ln_eps = eps;
    float* stand_in = reinterpret_cast<float*>(C.c->arena.base);
    g2.C = stand_in, g2.ln_y = stand_in;
    g2.a_part = stand_in, g2.a_bias = C.T(b_fc).data, g2.a_chunks = ok1 ? gemv_chunks(g1) : 0;
    if (ok1 && gemv_accepts(g2)) {
      const size_t wb = gemv_workspace_bytes(g1);
      void* parts = C.scratch(wb);  // kept until the projection below has read it (stream order)
      std::vector<int64_t> shp = shape_vec(C.T(x));
      shp.back() = N;
      int yh = C.make_output(shp);
      int hh = C.make_output(shp);
      uint16_t* hb = C.twin_data(ctx->tensors[hh]);
      const bool only = hb && (flags & TFB_OUT_BF16_ONLY);
      g1.C = nullptr;
      C.run_gemm_ws(g1, parts, wb);
      g2.a_part = static_cast<const float*>(parts);
      g2.C = ctx->tensors[yh].data;
      g2.ln_y = only ? nullptr : ctx->tensors[hh].data, g2.ln_ybf = hb;
      C.run_gemm(g2);
      if (hb) ctx->tensors[hh].bf_valid = true;
      if (only) ctx->tensors[hh].f32_valid = false, ctx->tensors[hh].bf16_out = true;
      *y = yh, *h = hh;
      return;
    }
    tfb_tensor f;
    int rc = tfb_linear_gelu(ctx, x, w_fc, b_fc, TFB_OUT_BF16_ONLY, &f);
    if (rc) rethrow(rc);
    rc = tfb_linear_residual_layernorm(ctx, f, w_proj, b_proj, r, gamma, beta, eps, flags, y, h);
    if (rc) rethrow(rc);
  });
}

int tfb_kv_attend_linear(tfb_ctx* ctx, tfb_kv* kv, int layer, tfb_tensor x, tfb_tensor w, tfb_tensor b, int pos,
                         int heads, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    need(kv != nullptr && kv->ctx == ctx, TFB_ERR_ARG, "cache of another context");
    need(y != nullptr, TFB_ERR_ARG, "null output");
    x = C.dense_in(x, C.bf16_mode()), w = C.dense_in(w, C.bf16_mode()), b = C.dense_in(b);
    check_linear(C, x, w, b);
    const int Cc = kv->channels;
    TensorRec& X = C.T(x);
    need(X.ndim == 3 && X.shape[0] == kv->batch && X.shape[1] == 1 && C.T(w).shape[1] == 3LL * Cc, TFB_ERR_SHAPE,
         "kv_attend_linear needs x [batch, 1, K] and w [K, 3C]");
    need(layer >= 0 && layer < kv->layers, TFB_ERR_ARG, "no such layer");
    need(pos >= 0 && pos < kv->tmax, TFB_ERR_SHAPE, "position past the cache length");
    need(heads > 0 && Cc % heads == 0, TFB_ERR_SHAPE, "channels not divisible by heads");
    bool ok = false;
    GemmArgs g = linear_post_args(C, x, w, b, -1, POST_PARTIALS, nullptr, nullptr, &ok);
    g.bias = nullptr;
    ok = gemv_accepts(g) && kv_attend_takes_parts(Cc, heads) && !ctx->grad_enabled;
    if (!ok) {
      tfb_tensor qkv;
      int rc = tfb_linear(ctx, x, w, b, &qkv);
      if (rc) rethrow(rc);
      rc = tfb_kv_attend(ctx, kv, layer, qkv, pos, heads, y);
      if (rc) rethrow(rc);
      return;
    }
    const size_t wb = gemv_workspace_bytes(g);
    void* parts = C.scratch(wb);
    g.C = nullptr;
    C.run_gemm_ws(g, parts, wb);
    const float scale = 1.f / std::sqrt((float)(Cc / heads));
    int h = C.make_output({kv->batch, 1, Cc});
    void* ws = C.scratch(std::max<size_t>(kv_attend_workspace_bytes(kv->batch, Cc, heads, pos), 256));
    const double e = kv->bf16 ? 2.0 : 4.0;
    const double bytes = (double)kv->batch * Cc * (2 * e * (pos + 1) + 2 * e + 4.0 + 4.0);
    const float* bias = C.T(b).data;
    const int chunks = gemv_chunks(g);
    C.timed(TFB_PROF_KV_ATTEND, bytes, [&] {
      hip_check(kv_attend(nullptr, kv->data, kv->bf16, ctx->tensors[h].data, layer, kv->batch, kv->tmax, Cc, heads,
                          pos, scale, ws, C.s(), static_cast<const float*>(parts), chunks, bias),
                "kv_attend");
    });
    *y = h;  // inference only: not recorded on the tape
  });
}

int tfb_kv_attention_block(tfb_ctx* ctx, tfb_kv* kv, int layer, tfb_tensor x, tfb_tensor w_attn, tfb_tensor b_attn,
                           int pos, int heads, tfb_tensor w_proj, tfb_tensor b_proj, tfb_tensor r, tfb_tensor gamma,
                           tfb_tensor beta, float eps, int flags, tfb_tensor* y, tfb_tensor* h) {
  return guarded([&] {
    Ctx C(ctx);
    need((flags & ~TFB_OUT_BF16_ONLY) == 0, TFB_ERR_ARG, "unknown tfb_kv_attention_block flags");
    need(kv != nullptr && kv->ctx == ctx, TFB_ERR_ARG, "cache of another context");
    need(!ctx->grad_enabled, TFB_ERR_STATE, "tfb_kv_attention_block is inference-only: disable gradients first");
    need(y != nullptr && h != nullptr, TFB_ERR_ARG, "null output");
    x = C.dense_in(x, C.bf16_mode()), w_attn = C.dense_in(w_attn, C.bf16_mode()), b_attn = C.dense_in(b_attn);
    w_proj = C.dense_in(w_proj, C.bf16_mode()), b_proj = C.dense_in(b_proj);
    r = C.dense_in(r), gamma = C.dense_in(gamma), beta = C.dense_in(beta);
    check_linear(C, x, w_attn, b_attn);
    const int Cc = kv->channels;
    TensorRec& X = C.T(x);
    need(X.ndim == 3 && X.shape[0] == kv->batch && X.shape[1] == 1 && C.T(w_attn).shape[1] == 3LL * Cc,
         TFB_ERR_SHAPE, "kv_attention_block needs x [batch, 1, K] and w_attn [K, 3C]");
    need(layer >= 0 && layer < kv->layers, TFB_ERR_ARG, "no such layer");
    need(pos >= 0 && pos < kv->tmax, TFB_ERR_SHAPE, "position past the cache length");
    need(heads > 0 && Cc % heads == 0, TFB_ERR_SHAPE, "channels not divisible by heads");
    need(C.T(w_proj).ndim == 2 && C.T(w_proj).shape[0] == Cc, TFB_ERR_SHAPE,
         "attention projection must be [" + std::to_string(Cc) + ", N], got " + shape_str(C.T(w_proj)));
    const int64_t N = C.T(w_proj).shape[1];
    need(C.T(b_proj).numel == N && C.T(b_proj).ndim == 1, TFB_ERR_SHAPE,
         "linear bias must be [" + std::to_string(N) + "]");
    need(C.T(r).numel == (int64_t)kv->batch * N && C.T(r).cols() == N, TFB_ERR_SHAPE,
         "residual must have the output's shape, got " + shape_str(C.T(r)));
    need(C.T(gamma).numel == N && C.T(beta).numel == N, TFB_ERR_SHAPE,
         "layernorm gain/shift must have " + std::to_string(N) + " elements");
    need(N <= 2048, TFB_ERR_SHAPE, "layernorm rows longer than 2048 are not supported");
    // c_attn leaves its partials, the attention sums them as it reads q, k and v and
    // leaves its per-block results, and the projection merges those as it loads its
    // input, then its chunk sum adds bias and residual and normalises the row
    bool ok1 = false;
    GemmArgs g1 = linear_post_args(C, x, w_attn, b_attn, -1, POST_PARTIALS, nullptr, nullptr, &ok1);
    g1.bias = nullptr;
    ok1 = gemv_accepts(g1) && kv_attend_takes_parts(Cc, heads);
    const int hs = Cc / heads, S = kv_attend_blocks(kv->bf16, pos);
    GemmArgs g2 = C.gemm_base();
    g2.M = kv->batch, g2.N = (int)N, g2.K = Cc;
    set_b(g2, op_data(C, C.T(w_proj))), g2.ldb = N;
    g2.ldc = N, g2.bias = C.T(b_proj).data, g2.resid = C.f32(C.T(r));
    g2.post = POST_LN, g2.ln_gamma = C.T(gamma).data, g2.ln_beta = C.T(beta).data, g2.ln_eps = eps;
    float* stand_in = reinterpret_cast<float*>(C.c->arena.base);
    g2.C = stand_in, g2.ln_y = stand_in;
    g2.att_acc = stand_in, g2.att_ml = stand_in, g2.att_blocks = S, g2.att_hs = hs, g2.att_heads = heads;
    if (ok1 && gemv_accepts(g2)) {
      const size_t wb = gemv_workspace_bytes(g1);
      void* parts = C.scratch(wb);  // kept until the attention below has read it (stream order)
      float* ws = static_cast<float*>(
          C.scratch(std::max<size_t>(kv_attend_workspace_bytes(kv->batch, Cc, heads, pos), 256)));
      std::vector<int64_t> shp = shape_vec(X);
      shp.back() = N;
      int yh = C.make_output(shp);
      int hh = C.make_output(shp);
      uint16_t* hb = C.twin_data(ctx->tensors[hh]);
      const bool only = hb && (flags & TFB_OUT_BF16_ONLY);
      g1.C = nullptr;
      C.run_gemm_ws(g1, parts, wb);
      const float scale = 1.f / std::sqrt((float)hs);
      const double e = kv->bf16 ? 2.0 : 4.0;
      const double bytes = (double)kv->batch * Cc * (2 * e * (pos + 1) + 2 * e + 4.0 + 4.0);
      const float* bias = C.T(b_attn).data;
      const int chunks = gemv_chunks(g1);
      C.timed(TFB_PROF_KV_ATTEND, bytes, [&] {
        hip_check(kv_attend(nullptr, kv->data, kv->bf16, nullptr, layer, kv->batch, kv->tmax, Cc, heads, pos, scale,
                            ws, C.s(), static_cast<const float*>(parts), chunks, bias),
                  "kv_attend");
      });
      g2.att_acc = ws, g2.att_ml = ws + (int64_t)kv->batch * heads * S * hs;
      g2.C = ctx->tensors[yh].data;
      g2.ln_y = only ? nullptr : ctx->tensors[hh].data, g2.ln_ybf = hb;
      C.run_gemm(g2);
      if (hb) ctx->tensors[hh].bf_valid = true;
      if (only) ctx->tensors[hh].f32_valid = false, ctx->tensors[hh].bf16_out = true;
      *y = yh, *h = hh;
      return;
    }
    tfb_tensor a;
    int rc = tfb_kv_attend_linear(ctx, kv, layer, x, w_attn, b_attn, pos, heads, &a);
    if (rc) rethrow(rc);
    rc = tfb_linear_residual_layernorm(ctx, a, w_proj, b_proj, r, gamma, beta, eps, flags, y, h);
    if (rc) rethrow(rc);
  });
}

int tfb_layernorm(tfb_ctx* ctx, tfb_tensor x, tfb_tensor gamma, tfb_tensor beta, float eps, tfb_tensor* y) {
  return tfb_layernorm_ex(ctx, x, gamma, beta, eps, 0, y);
}

int tfb_layernorm_ex(tfb_ctx* ctx, tfb_tensor x, tfb_tensor gamma, tfb_tensor beta, float eps, int flags,
                     tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    need((flags & ~TFB_OUT_BF16_ONLY) == 0, TFB_ERR_ARG, "unknown tfb_layernorm_ex flags");
    x = C.dense_in(x), gamma = C.dense_in(gamma), beta = C.dense_in(beta);
    TensorRec& X = C.T(x);
    TensorRec& G = C.T(gamma);
    TensorRec& Bt = C.T(beta);
    need(y != nullptr, TFB_ERR_ARG, "null output");
    const int64_t Cc = X.cols(), rows = X.rows();
    need(G.numel == Cc && Bt.numel == Cc, TFB_ERR_SHAPE, "layernorm gain/shift must have " + std::to_string(Cc) +
                                                             " elements");
    need(Cc <= 2048, TFB_ERR_SHAPE, "layernorm rows longer than 2048 are not supported");
    int h = C.make_output(shape_vec(X));
    float* mean = static_cast<float*>(C.scratch((size_t)rows * sizeof(float)));
    float* rstd = static_cast<float*>(C.scratch((size_t)rows * sizeof(float)));
    uint16_t* yb = C.twin_data(ctx->tensors[h]);
    const bool only = yb && (flags & TFB_OUT_BF16_ONLY);
    const double bytes = (double)rows * Cc * (4 + (only ? 0 : 4) + (yb ? 2 : 0)) + 8.0 * rows;
    C.timed(TFB_PROF_LN_FWD, bytes, [&] {
      hip_check(layernorm_fwd(ctx->tensors[x].data, ctx->tensors[gamma].data, ctx->tensors[beta].data,
                              only ? nullptr : ctx->tensors[h].data, yb, mean, rstd, rows, Cc, eps, C.s()),
                "layernorm");
    });
    if (yb) ctx->tensors[h].bf_valid = true;
    if (only) ctx->tensors[h].f32_valid = false, ctx->tensors[h].bf16_out = true;
    Rec r{OP_LAYERNORM};
    r.in[0] = x, r.in[1] = gamma, r.in[2] = beta, r.out = h, r.f = eps;
    r.s0 = mean, r.s1 = rstd;
    C.record(r);
    *y = h;
  });
}

int tfb_embedding(tfb_ctx* ctx, tfb_tensor table, const int32_t* dev_ids, int64_t n, int64_t batch, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    table = C.dense_in(table);
    TensorRec& Tb = C.T(table);
    need(y != nullptr && dev_ids != nullptr, TFB_ERR_ARG, "null argument");
    need(Tb.ndim == 2, TFB_ERR_SHAPE, "embedding table must be 2-D");
    need(n >= 0 && batch > 0 && n % batch == 0, TFB_ERR_SHAPE, "ids count must be a multiple of batch");
    need(n < (1ll << 31), TFB_ERR_SHAPE, "too many ids");
    const int64_t Cc = Tb.shape[1], trows = Tb.shape[0];
    int h = C.make_output({batch, n / batch, Cc});
    int32_t* ids = static_cast<int32_t*>(C.scratch((size_t)std::max<int64_t>(n, 1) * sizeof(int32_t)));
    if (n)
      hip_check(hipMemcpyAsync(ids, dev_ids, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToDevice, C.s()),
                "copy ids");
    hip_check(embedding_fwd(ctx->tensors[table].data, trows, ids, ctx->tensors[h].data, n, Cc, C.s()), "embedding");
    Rec r{OP_EMBEDDING};
    r.in[0] = table, r.out = h, r.i0 = n;
    r.s0 = ids;
    C.record(r);
    *y = h;
  });
}

int tfb_narrow(tfb_ctx* ctx, tfb_tensor x, int64_t start, int64_t len, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    x = C.dense_in(x);
    TensorRec& X = C.T(x);
    need(y != nullptr, TFB_ERR_ARG, "null output");
    need(start >= 0 && len >= 0 && start + len <= X.cols(), TFB_ERR_SHAPE, "narrow out of range");
    const int64_t rows = X.rows(), cols = X.cols();
    std::vector<int64_t> shp = shape_vec(X);
    shp.back() = len;
    int h = C.make_output(shp);
    hip_check(narrow_fwd(ctx->tensors[x].data, ctx->tensors[h].data, rows, cols, start, len, C.s()), "narrow");
    Rec r{OP_NARROW};
    r.in[0] = x, r.out = h, r.i0 = start, r.i1 = len;
    C.record(r);
    *y = h;
  });
}

int tfb_split_heads(tfb_ctx* ctx, tfb_tensor x, int heads, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    x = C.dense_in(x);
    TensorRec& X = C.T(x);
    need(y != nullptr, TFB_ERR_ARG, "null output");
    need(X.ndim == 3 && heads > 0 && X.shape[2] % heads == 0, TFB_ERR_SHAPE,
         "split_heads needs [B, T, H*hs], got " + shape_str(X));
    const int64_t B = X.shape[0], T = X.shape[1], hs = X.shape[2] / heads;
    int h = C.make_output({B, heads, T, hs});
    hip_check(permute_heads(ctx->tensors[x].data, ctx->tensors[h].data, B, T, heads, hs, true, 0.f, C.s()),
              "split_heads");
    Rec r{OP_SPLIT_HEADS};
    r.in[0] = x, r.out = h;
    C.record(r);
    *y = h;
  });
}

int tfb_merge_heads(tfb_ctx* ctx, tfb_tensor x, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    x = C.dense_in(x);
    TensorRec& X = C.T(x);
    need(y != nullptr, TFB_ERR_ARG, "null output");
    need(X.ndim == 4, TFB_ERR_SHAPE, "merge_heads needs [B, H, T, hs], got " + shape_str(X));
    const int64_t B = X.shape[0], H = X.shape[1], T = X.shape[2], hs = X.shape[3];
    int h = C.make_output({B, T, H * hs});
    hip_check(permute_heads(ctx->tensors[x].data, ctx->tensors[h].data, B, T, H, hs, false, 0.f, C.s()),
              "merge_heads");
    Rec r{OP_MERGE_HEADS};
    r.in[0] = x, r.out = h;
    C.record(r);
    *y = h;
  });
}

static int bmm_impl(tfb_ctx* ctx, tfb_tensor a, tfb_tensor b, tfb_tensor* y, bool transb) {
  return guarded([&] {
    Ctx C(ctx);
    a = C.dense_in(a), b = C.dense_in(b);
    TensorRec& A = C.T(a);
    TensorRec& B = C.T(b);
    need(y != nullptr, TFB_ERR_ARG, "null output");
    need(A.ndim == 3 && B.ndim == 3 && A.shape[0] == B.shape[0], TFB_ERR_SHAPE,
         "batch_matmul needs [Z, n, k] and [Z, ., .]: " + shape_str(A) + " " + shape_str(B));
    const int64_t Z = A.shape[0], n = A.shape[1], k = A.shape[2];
    int64_t m;
    if (transb) {
      need(B.shape[2] == k, TFB_ERR_SHAPE, "batch_matmul_t " + shape_str(A) + " @ " + shape_str(B) + "^T");
      m = B.shape[1];
    } else {
      need(B.shape[1] == k, TFB_ERR_SHAPE, "batch_matmul " + shape_str(A) + " @ " + shape_str(B));
      m = B.shape[2];
    }
    check_gemm_dims(n, k, m);
    int h = C.make_output({Z, n, m});
    GemmArgs q = C.gemm_base();
    q.M = (int)n, q.N = (int)m, q.K = (int)k;
    q.A = ctx->tensors[a].data, q.lda = k, q.sa1 = n * k;
    q.B = ctx->tensors[b].data;
    if (transb)
      q.ldb = k, q.b_kcontig = true, q.sb1 = m * k;
    else
      q.ldb = m, q.sb1 = k * m;
    q.C = ctx->tensors[h].data, q.ldc = m, q.sc1 = n * m;
    q.batch = (int)Z;
    C.run_gemm(q);
    Rec r{transb ? OP_BMM_T : OP_BMM};
    r.in[0] = a, r.in[1] = b, r.out = h;
    C.record(r);
    *y = h;
  });
}

int tfb_batch_matmul(tfb_ctx* ctx, tfb_tensor a, tfb_tensor b, tfb_tensor* y) { return bmm_impl(ctx, a, b, y, false); }
int tfb_batch_matmul_t(tfb_ctx* ctx, tfb_tensor a, tfb_tensor b, tfb_tensor* y) { return bmm_impl(ctx, a, b, y, true); }

int tfb_causal_softmax(tfb_ctx* ctx, tfb_tensor sx, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    sx = C.dense_in(sx);
    TensorRec& S = C.T(sx);
    need(y != nullptr, TFB_ERR_ARG, "null output");
    const int64_t rows = S.rows(), T = S.cols();
    int h = C.make_output(shape_vec(S));
    hip_check(causal_softmax_fwd(ctx->tensors[sx].data, ctx->tensors[h].data, rows, T, true, C.s()),
              "causal_softmax");
    Rec r{OP_CSOFTMAX};
    r.in[0] = sx, r.out = h;
    C.record(r);
    *y = h;
  });
}

int tfb_causal_attention(tfb_ctx* ctx, tfb_tensor qkv, int heads, tfb_tensor* y) {
  return tfb_causal_attention_ex(ctx, qkv, heads, 0, y);
}

int tfb_causal_attention_ex(tfb_ctx* ctx, tfb_tensor qkv, int heads, int flags, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    need((flags & ~TFB_OUT_BF16_ONLY) == 0, TFB_ERR_ARG, "unknown tfb_causal_attention_ex flags");
    qkv = C.dense_in(qkv, true);  // the fused kernels read the bf16 copy; the fp32 path converts below
    TensorRec& Q = C.T(qkv);
    need(y != nullptr, TFB_ERR_ARG, "null output");
    need(Q.ndim == 3 && Q.shape[2] % 3 == 0 && heads > 0 && (Q.shape[2] / 3) % heads == 0, TFB_ERR_SHAPE,
         "causal_attention needs qkv [B, T, 3C] with C divisible by heads, got " + shape_str(Q));
    const int64_t B = Q.shape[0], T = Q.shape[1], C3 = Q.shape[2], Cc = C3 / 3, H = heads, hs = Cc / H;
    check_gemm_dims(T, T, hs);
    need(B * H < 65536, TFB_ERR_SHAPE, "too many (batch, head) pairs");
    const float scale = 1.f / std::sqrt((float)hs);
    int h = C.make_output({B, T, Cc});
    if (C.bf16_mode() && flash_attention_supported((int)hs, Cc, T)) {
      // bf16 variant: fused kernels, no T x T buffers
      const uint16_t* qb = C.data_bf16(ctx->tensors[qkv]);
      float* lse = static_cast<float*>(C.scratch((size_t)B * H * T * sizeof(float)));
      uint16_t* yb = C.twin_data(ctx->tensors[h]);
      const bool only = yb && (flags & TFB_OUT_BF16_ONLY);
      // QK^T and PV over the causal triangle
      const double flops = 2.0 * 2.0 * hs * (T * (T + 1.0) / 2.0) * B * H;
      C.timed(TFB_PROF_ATTN_FWD, flops, [&] {
        hip_check(flash_attention_fwd(qb, only ? nullptr : ctx->tensors[h].data, yb, lse, (int)B, (int)T, (int)H,
                                      (int)Cc, scale, C.s()),
                  "attention");
      });
      ctx->tensors[h].bf_valid = true;
      if (only) ctx->tensors[h].f32_valid = false, ctx->tensors[h].bf16_out = true;
      Rec r{OP_ATTENTION};
      r.in[0] = qkv, r.out = h, r.i0 = H, r.i1 = 1, r.f = scale;
      r.s1 = lse;
      C.record(r);
      *y = h;
      return;
    }
    float* P = static_cast<float*>(C.scratch((size_t)B * H * T * T * sizeof(float)));
    const float* q = C.f32(ctx->tensors[qkv]);
    float* yd = ctx->tensors[h].data;
    {  // S = (Q_h K_h^T) * scale, tiles on or below the diagonal
      GemmArgs a = C.gemm_base();
      a.M = (int)T, a.N = (int)T, a.K = (int)hs;
      a.A = q, a.lda = C3, a.sa1 = T * C3, a.sa2 = hs;
      a.B = q + Cc, a.ldb = C3, a.b_kcontig = true, a.sb1 = T * C3, a.sb2 = hs;
      a.C = P, a.ldc = T, a.sc1 = H * T * T, a.sc2 = T * T;
      a.alpha = scale, a.batch = (int)(B * H), a.batch_div = (int)H;
      a.causal_out = true;
      C.run_gemm(a);
    }
    hip_check(causal_softmax_fwd(P, P, B * H * T, T, false, C.s()), "attention softmax");
    {  // Y_h = P V_h, written straight into the merged [B, T, C] layout
      GemmArgs a = C.gemm_base();
      a.M = (int)T, a.N = (int)hs, a.K = (int)T;
      a.A = P, a.lda = T, a.sa1 = H * T * T, a.sa2 = T * T, a.causal_a = CAUSAL_UPTO;
      a.B = q + 2 * Cc, a.ldb = C3, a.sb1 = T * C3, a.sb2 = hs;
      a.C = yd, a.ldc = Cc, a.sc1 = T * Cc, a.sc2 = hs;
      a.batch = (int)(B * H), a.batch_div = (int)H;
      C.run_gemm(a);
    }
    Rec r{OP_ATTENTION};
    r.in[0] = qkv, r.out = h, r.i0 = H, r.f = scale;
    r.s0 = P;
    C.record(r);
    *y = h;
  });
}

int tfb_softmax_cross_entropy(tfb_ctx* ctx, tfb_tensor logits, const int32_t* dev_targets, int64_t n,
                              tfb_tensor* loss) {
  return tfb_softmax_cross_entropy_ex(ctx, logits, dev_targets, n, 0, loss);
}

int tfb_softmax_cross_entropy_ex(tfb_ctx* ctx, tfb_tensor logits, const int32_t* dev_targets, int64_t n, int flags,
                                 tfb_tensor* loss) {
  return guarded([&] {
    need((flags & ~TFB_CE_GRAD_BF16_ONLY) == 0, TFB_ERR_ARG, "unknown tfb_softmax_cross_entropy_ex flags");
    Ctx C(ctx);
    TensorRec& L = C.T(logits);
    need(loss != nullptr && dev_targets != nullptr, TFB_ERR_ARG, "null argument");
    need(n == L.rows(), TFB_ERR_SHAPE, "one target per row");
    const int64_t rows = L.rows(), V = L.cols();
    int h = C.make_output({1});
    int32_t* tg = static_cast<int32_t*>(C.scratch((size_t)std::max<int64_t>(rows, 1) * sizeof(int32_t)));
    float* lse = static_cast<float*>(C.scratch((size_t)std::max<int64_t>(rows, 1) * sizeof(float)));
    if (rows)
      hip_check(hipMemcpyAsync(tg, dev_targets, (size_t)rows * sizeof(int32_t), hipMemcpyDeviceToDevice, C.s()),
                "copy targets");
    // with the bf16-only option the logits' bf16 gradient for an upstream gradient of 1
    // comes out of the same pass over the logits (allocated before the scratch below)
    uint16_t* pre = nullptr;
    if ((flags & TFB_CE_GRAD_BF16_ONLY) && ctx->grad_enabled && !ctx->tensors[logits].leaf &&
        C.grad_read_as_bf16(ctx->tensors[logits]))
      pre = C.twin_grad(ctx->tensors[logits]);
    size_t mark = ctx->arena.hi;
    void* ws = C.scratch(softmax_ce_workspace_bytes(rows));
    bool pre_written = false;
    // logits held only as bf16 are read as such
    TensorRec& LG = ctx->tensors[logits];
    const bool lbf = !LG.f32_valid && softmax_ce_bf16_fits(LG.stride(), V, LG.bf);
    if (!lbf) C.f32(LG);
    // the logits once, and the fused gradient where it is written in the same pass
    const double bytes = (double)rows * V * ((lbf ? 2 : 4) + (pre ? 2 : 0));
    C.timed(TFB_PROF_CE, bytes, [&] {
      hip_check(softmax_ce_fwd(lbf ? nullptr : LG.data, LG.stride(), tg, rows, V, lse, ctx->tensors[h].data, ws,
                               C.s(), pre, &pre_written, lbf ? LG.bf : nullptr),
                "softmax_ce");
    });
    ctx->arena.hi = mark;
    Rec r{OP_SOFTMAX_CE};
    r.in[0] = logits, r.out = h;
    r.s0 = tg, r.s1 = lse;
    r.i0 = flags;
    r.i1 = pre_written ? 1 : 0;
    C.record(r);
    *loss = h;
  });
}

// ------------------------------------------------------------------ autograd
int tfb_backward(tfb_ctx* ctx, tfb_tensor loss) {
  return guarded([&] {
    Ctx C(ctx);
    TensorRec& L = C.T(loss);
    need(L.numel == 1, TFB_ERR_STATE, "backward() starts from a scalar loss");
    for (TensorRec& t : ctx->tensors) {
      if (t.live && !t.leaf && t.grad) t.gstate = G_ZERO;
      if (t.gstate == G_BF16) t.gstate = t.grad ? G_ZERO : G_NONE;
      t.gbf_valid = false;
      t.gcol_valid = false;
      t.gpend = nullptr;
    }
    C.ensure_grad_buffer(L);
    hip_check(fill(L.grad, 1.f, 1, C.s()), "seed");
    L.gstate = G_VALID;
    ctx->bias_jobs.count = 0;
    ctx->reduce_jobs.count = 0;
    for (int i = (int)ctx->tape.size() - 1; i >= 0; --i) {
      const Rec& r = ctx->tape[i];
      TensorRec& out = ctx->tensors[r.out];
      if (!out.live) continue;
      C.settle(out);  // its gradient is complete: nothing else contributes
      if (out.gstate != G_VALID && out.gstate != G_BF16) continue;
      C.f32_for_bwd(r);
      backward_rec(C, r);
    }
    C.flush_bias();
    for (TensorRec& t : ctx->tensors)
      if (t.live) C.settle(t);
  });
}

int tfb_zero_grad(tfb_ctx* ctx, const tfb_tensor* params, int n) {
  return guarded([&] {
    Ctx C(ctx);
    need(n == 0 || params != nullptr, TFB_ERR_ARG, "null parameter list");
    for (int i = 0; i < n; ++i) {
      TensorRec& t = C.T(params[i]);
      if (t.grad) t.gstate = G_ZERO;
      t.gbf_valid = false;
    }
  });
}

int tfb_tape_reset(tfb_ctx* ctx) {
  return guarded([&] {
    Ctx C(ctx);
    ctx->tape.clear();
    for (int h = 0; h < (int)ctx->tensors.size(); ++h) {
      TensorRec& t = ctx->tensors[h];
      if (t.live && !t.leaf) {
        t.live = false;
        ctx->free_handles.push_back(h);
      }
    }
    ctx->arena.hi = ctx->arena.size;
  });
}

// ------------------------------------------------------------------ optimizers
int tfb_adamw_create(tfb_ctx* ctx, const tfb_tensor* params, int n, float lr, float weight_decay, float beta1,
                     float beta2, float eps, tfb_opt** out) {
  return guarded([&] {
    Ctx C(ctx);
    need(out != nullptr && (n == 0 || params != nullptr), TFB_ERR_ARG, "null argument");
    tfb_opt* o = new tfb_opt();
    o->ctx = ctx;
    o->lr = lr, o->wd = weight_decay, o->b1 = beta1, o->b2 = beta2, o->eps = eps;
    try {
      int64_t nchunks = 0;
      for (int i = 0; i < n; ++i) {
        TensorRec& t = C.T(params[i]);
        o->params.push_back(params[i]);
        size_t mo = ctx->arena.alloc_persist((size_t)t.numel * sizeof(float));
        size_t vo = ctx->arena.alloc_persist((size_t)t.numel * sizeof(float));
        o->m.push_back(reinterpret_cast<float*>(ctx->arena.base + mo));
        o->v.push_back(reinterpret_cast<float*>(ctx->arena.base + vo));
        hip_check(fill(o->m.back(), 0.f, t.numel, C.s()), "zero m");
        hip_check(fill(o->v.back(), 0.f, t.numel, C.s()), "zero v");
        nchunks += (t.numel + o->chunk_elems - 1) / o->chunk_elems;
      }
      o->d_nseg_cap = std::max(n, 1);
      o->d_nchunk_cap = (int)std::max<int64_t>(nchunks, 1);
      o->d_segs = reinterpret_cast<AdamSeg*>(ctx->arena.base +
                                             ctx->arena.alloc_persist(sizeof(AdamSeg) * o->d_nseg_cap));
      o->d_chunks = reinterpret_cast<AdamChunk*>(ctx->arena.base +
                                                 ctx->arena.alloc_persist(sizeof(AdamChunk) * o->d_nchunk_cap));
    } catch (...) {
      delete o;
      throw;
    }
    *out = o;
  });
}

int tfb_adamw_set_lr(tfb_opt* opt, float lr) {
  return guarded([&] {
    need(opt != nullptr, TFB_ERR_ARG, "null optimizer");
    opt->lr = lr;
  });
}

int tfb_adamw_step(tfb_opt* o) {
  return guarded([&] {
    need(o != nullptr, TFB_ERR_ARG, "null optimizer");
    Ctx C(o->ctx);
    tfb_ctx* ctx = o->ctx;
    // parameters without a gradient are skipped; a cleared gradient reads as zeros
    std::vector<int> active;
    std::vector<uint16_t*> shadows;
    for (int i = 0; i < (int)o->params.size(); ++i) {
      TensorRec& t = C.T(o->params[i]);
      if (!t.grad) continue;
      C.materialize_zero(t);
      active.push_back(i);
      shadows.push_back(t.bf);
    }
    o->t += 1;
    const float bc1 = 1.f - std::pow(o->b1, (float)o->t);
    const float bc2 = 1.f - std::pow(o->b2, (float)o->t);
    if (active != o->uploaded_active || shadows != o->uploaded_shadows) {
      std::vector<AdamSeg> segs;
      std::vector<AdamChunk> chunks;
      for (int i : active) {
        TensorRec& t = C.T(o->params[i]);
        AdamSeg sg;
        sg.p = t.data, sg.g = t.grad, sg.m = o->m[i], sg.v = o->v[i], sg.n = t.numel;
        sg.pbf = t.bf;  // the step keeps an existing bf16 copy current
        sg.wd = t.ndim >= 2 ? o->wd : 0.f;
        sg.pad = 0;
        for (int64_t off = 0; off < t.numel; off += o->chunk_elems) {
          AdamChunk ch;
          ch.seg = (int)segs.size(), ch.pad = 0, ch.off = off;
          chunks.push_back(ch);
        }
        segs.push_back(sg);
      }
      if (!segs.empty()) {
        hip_check(hipMemcpyAsync(o->d_segs, segs.data(), segs.size() * sizeof(AdamSeg), hipMemcpyHostToDevice, C.s()),
                  "upload segments");
        hip_check(hipMemcpyAsync(o->d_chunks, chunks.data(), chunks.size() * sizeof(AdamChunk),
                                 hipMemcpyHostToDevice, C.s()),
                  "upload chunks");
        hip_check(hipStreamSynchronize(C.s()), "sync");
      }
      o->nchunks = (int)chunks.size();
      o->uploaded_active = active;
      o->uploaded_shadows = shadows;
    }
    // per element: read p, g, m, v; write p, m, v; and the bf16 copy of p where one is kept
    double bytes = 0.0;
    for (int i : active) {
      TensorRec& t = C.T(o->params[i]);
      t.bf_valid = t.bf != nullptr;
      bytes += (double)t.numel * (28 + (t.bf ? 2 : 0));
    }
    (void)ctx;
    C.timed(TFB_PROF_ADAMW, bytes, [&] {
      hip_check(adamw_step(o->d_segs, o->d_chunks, o->nchunks, o->chunk_elems, o->lr, o->b1, o->b2, o->eps, bc1, bc2,
                           C.s()),
                "adamw");
    });
  });
}

int tfb_adamw_moments(tfb_opt* o, int i, float* host_m, float* host_v, int64_t n) {
  return guarded([&] {
    need(o != nullptr, TFB_ERR_ARG, "null optimizer");
    Ctx C(o->ctx);
    need(i >= 0 && i < (int)o->params.size(), TFB_ERR_ARG, "no such parameter");
    TensorRec& t = C.T(o->params[i]);
    need(n == t.numel, TFB_ERR_SHAPE, "size mismatch");
    if (host_m)
      hip_check(hipMemcpyAsync(host_m, o->m[i], n * sizeof(float), hipMemcpyDeviceToHost, C.s()), "copy m");
    if (host_v)
      hip_check(hipMemcpyAsync(host_v, o->v[i], n * sizeof(float), hipMemcpyDeviceToHost, C.s()), "copy v");
    hip_check(hipStreamSynchronize(C.s()), "sync");
  });
}

int tfb_adamw_destroy(tfb_opt* o) {
  return guarded([&] {
    need(o != nullptr, TFB_ERR_ARG, "null optimizer");
    delete o;
  });
}

int tfb_profile_begin(tfb_ctx* ctx) {
  return guarded([&] {
    Ctx C(ctx);
    ProfileState& pf = ctx->prof;
    pf.on = true;
    pf.used = 0;
    pf.spans.clear();
    for (int k = 0; k < TFB_PROF_KINDS; ++k) pf.ms[k] = pf.work[k] = 0.0, pf.launches[k] = 0;
  });
}

int tfb_profile_end(tfb_ctx* ctx, double* gemm_ms, double* gemm_flops, int* launches) {
  return guarded([&] {
    Ctx C(ctx);
    ProfileState& pf = ctx->prof;
    need(pf.on, TFB_ERR_STATE, "profiling was not started");
    pf.on = false;
    hip_check(hipStreamSynchronize(C.s()), "sync");
    for (const ProfileState::Span& sp : pf.spans) {
      float e = 0.f;
      hip_check(hipEventElapsedTime(&e, pf.pool[sp.ev], pf.pool[sp.ev + 1]), "hipEventElapsedTime");
      pf.ms[sp.kind] += e;
      pf.work[sp.kind] += sp.work;
      pf.launches[sp.kind] += 1;
    }
    pf.spans.clear();
    if (gemm_ms) *gemm_ms = pf.ms[TFB_PROF_GEMM];
    if (gemm_flops) *gemm_flops = pf.work[TFB_PROF_GEMM];
    if (launches) *launches = pf.launches[TFB_PROF_GEMM];
  });
}

int tfb_profile_kind(tfb_ctx* ctx, int kind, double* ms, double* work, int* launches) {
  return guarded([&] {
    need(ctx != nullptr, TFB_ERR_ARG, "null context");
    need(kind >= 0 && kind < TFB_PROF_KINDS, TFB_ERR_ARG, "unknown profile kind");
    const ProfileState& pf = ctx->prof;
    need(!pf.on, TFB_ERR_STATE, "profiling still running: call tfb_profile_end first");
    if (ms) *ms = pf.ms[kind];
    if (work) *work = pf.work[kind];
    if (launches) *launches = pf.launches[kind];
  });
}

// ------------------------------------------------------------------ KV-cached inference
int tfb_kv_create(tfb_ctx* ctx, int layers, int batch, int tmax, int channels, tfb_kv** out) {
  return guarded([&] {
    Ctx C(ctx);
    need(out != nullptr, TFB_ERR_ARG, "null output");
    need(layers > 0 && batch > 0 && tmax > 0 && channels > 0, TFB_ERR_SHAPE, "kv cache sizes must be positive");
    need(tmax <= 16384, TFB_ERR_SHAPE, "kv cache longer than 16384 positions is not supported");
    const size_t n = (size_t)layers * 2 * batch * tmax * channels;
    const bool bf = C.bf16_mode();
    const size_t bytes = Arena::up(n * (bf ? 2 : 4));
    const size_t off = ctx->arena.alloc_persist(bytes);
    float* p = reinterpret_cast<float*>(ctx->arena.base + off);
    hip_check(fill(p, 0.f, (int64_t)(bytes / 4), C.s()), "kv clear");  // zero bits: 0.0 in either form
    tfb_kv* kv = new tfb_kv();
    kv->ctx = ctx, kv->layers = layers, kv->batch = batch, kv->tmax = tmax, kv->channels = channels, kv->data = p;
    kv->bf16 = bf;
    kv->off = off, kv->end = off + bytes;
    *out = kv;
  });
}

int tfb_kv_destroy(tfb_kv* kv) {
  return guarded([&] {
    need(kv != nullptr, TFB_ERR_ARG, "null cache");
    kv->ctx->arena.release_persist(kv->off, kv->end - kv->off);
    delete kv;
  });
}

int tfb_kv_store(tfb_ctx* ctx, tfb_kv* kv, int layer, tfb_tensor qkv, int pos0) {
  return guarded([&] {
    Ctx C(ctx);
    need(kv != nullptr && kv->ctx == ctx, TFB_ERR_ARG, "cache of another context");
    qkv = C.dense_in(qkv);
    TensorRec& Q = C.T(qkv);
    need(Q.ndim == 3 && Q.shape[0] == kv->batch && Q.shape[2] == 3LL * kv->channels, TFB_ERR_SHAPE,
         "kv_store needs qkv [batch, T, 3C], got " + shape_str(Q));
    need(layer >= 0 && layer < kv->layers, TFB_ERR_ARG, "no such layer");
    need(pos0 >= 0 && pos0 + Q.shape[1] <= kv->tmax, TFB_ERR_SHAPE, "positions past the cache length");
    hip_check(kv_store(C.f32(Q), Q.shape[1], kv->channels, kv->data, kv->bf16, layer, kv->batch, kv->tmax, pos0, C.s()),
              "kv_store");
  });
}

int tfb_kv_attend(tfb_ctx* ctx, tfb_kv* kv, int layer, tfb_tensor qkv, int pos, int heads, tfb_tensor* y) {
  return guarded([&] {
    Ctx C(ctx);
    need(kv != nullptr && kv->ctx == ctx && y != nullptr, TFB_ERR_ARG, "bad argument");
    qkv = C.dense_in(qkv);
    TensorRec& Q = C.T(qkv);
    const int Cc = kv->channels;
    need(Q.ndim == 3 && Q.shape[0] == kv->batch && Q.shape[1] == 1 && Q.shape[2] == 3LL * Cc, TFB_ERR_SHAPE,
         "kv_attend needs qkv [batch, 1, 3C], got " + shape_str(Q));
    need(layer >= 0 && layer < kv->layers, TFB_ERR_ARG, "no such layer");
    need(pos >= 0 && pos < kv->tmax, TFB_ERR_SHAPE, "position past the cache length");
    need(heads > 0 && Cc % heads == 0, TFB_ERR_SHAPE, "channels not divisible by heads");
    const float scale = 1.f / std::sqrt((float)(Cc / heads));
    const float* qd = Q.data;
    int h = C.make_output({kv->batch, 1, Cc});
    void* ws = C.scratch(std::max<size_t>(kv_attend_workspace_bytes(kv->batch, Cc, heads, pos), 256));
    // every cached key and value of positions 0..pos, the new one stored, q read, y written
    const double e = kv->bf16 ? 2.0 : 4.0;
    const double bytes = (double)kv->batch * Cc * (2 * e * (pos + 1) + 2 * e + 4.0 + 4.0);
    C.timed(TFB_PROF_KV_ATTEND, bytes, [&] {
      hip_check(kv_attend(qd, kv->data, kv->bf16, ctx->tensors[h].data, layer, kv->batch, kv->tmax, Cc, heads, pos,
                          scale, ws, C.s()),
                "kv_attend");
    });
    *y = h;  // inference only: not recorded on the tape
  });
}

int tfb_sample_topk(tfb_ctx* ctx, tfb_tensor logits, int k, float temperature, const double* dev_uniforms,
                    int32_t* dev_out) {
  return guarded([&] {
    Ctx C(ctx);
    TensorRec& L = C.T(logits);
    need(dev_uniforms != nullptr && dev_out != nullptr, TFB_ERR_ARG, "null argument");
    need(temperature > 0.f, TFB_ERR_ARG, "temperature must be positive");
    need(k >= 0, TFB_ERR_ARG, "k must be >= 0");
    need(L.cols() > 0, TFB_ERR_SHAPE, "logits rows are empty");
    need(L.cols() < (1LL << 31) && L.rows() < 65536, TFB_ERR_SHAPE, "logits too large");
    const float* ld = C.f32(L);
    C.timed(TFB_PROF_SAMPLE, 4.0 * L.rows() * L.cols(), [&] {
      hip_check(sample_topk(ld, L.stride(), (int)L.rows(), (int)L.cols(), k, temperature, dev_uniforms, dev_out,
                            C.s()),
                "sample_topk");
    });
  });
}

int tfb_sgd_step(tfb_ctx* ctx, const tfb_tensor* params, int n, float lr) {
  return guarded([&] {
    Ctx C(ctx);
    need(n == 0 || params != nullptr, TFB_ERR_ARG, "null parameter list");
    for (int i = 0; i < n; ++i) {
      TensorRec& t = C.T(params[i]);
      if (!t.grad) continue;
      C.materialize_zero(t);
      hip_check(sgd_step(t.data, t.grad, lr, t.numel, C.s()), "sgd");
      t.bf_valid = false;
    }
  });
}

}  // extern "C"
