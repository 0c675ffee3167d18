// tfb_softmax_cross_entropy_noalloc: the SoftmaxCrossEntropy forward (mean
// loss over rows) on plain device pointers, for callers that cannot allocate
// device memory.  It runs the kernels of tfb_softmax_cross_entropy's forward
// (per-row log-sum-exp and loss, then the mean accumulated in double); their
// scratch -- the rows' log-sum-exp and per-row losses, 2 * rows floats -- lives
// in a file-scope device array instead of the arena.
//
// The array belongs to the device, one copy per GPU, held until the process
// ends.  Host code never passes the array's name to a kernel (in host code it
// is a host-side stand-in, not a device address): the device address is taken
// once per device with hipGetSymbolAddress, with that device current, and
// kept in `g_scratch_ptr`.  Every call on a GPU uses that GPU's one array, so
// calls that overlap on one GPU (on different streams, or from several
// threads) race; calls queued on one stream run in order.  Nothing in the
// array needs to start at zero: every element a call reads was written by that
// call's first kernel.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "../../include/tfb.h"
#include "kernels.h"

namespace {

constexpr int64_t MAX_ROWS = TFB_NOALLOC_MAX_ROWS;
constexpr size_t SCRATCH_BYTES = 2 * MAX_ROWS * sizeof(float);  // log-sum-exp | per-row loss
constexpr int MAX_DEVICES = 64;

static __device__ __align__(256) char scratch[SCRATCH_BYTES];

std::mutex g_mu;
void* g_scratch_ptr[MAX_DEVICES] = {nullptr};

// The scratch array's device address on the current device (taken once per device).
hipError_t scratch_on(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int tfb_softmax_cross_entropy_noalloc(const float* dev_logits, int64_t ld, const int32_t* dev_targets,
                                                 int64_t rows, int64_t cols, float* dev_loss, void* hip_stream) {
  using tfb::set_last_error;
  if (!dev_logits || !dev_targets || !dev_loss) return set_last_error(TFB_ERR_ARG, "null pointer argument");
  if (rows < 1 || cols < 1 || ld < cols)
    return set_last_error(TFB_ERR_SHAPE, "softmax_cross_entropy_noalloc needs rows >= 1, cols >= 1, ld >= cols");
  if (rows > MAX_ROWS)
    return set_last_error(TFB_ERR_SHAPE, ("softmax_cross_entropy_noalloc takes at most " + std::to_string(MAX_ROWS) +
                                          " rows (its scratch is a fixed device array); got " + std::to_string(rows))
                                             .c_str());
  if (cols >= (int64_t(1) << 31))
    return set_last_error(TFB_ERR_SHAPE, "softmax_cross_entropy_noalloc: rows longer than 2^31 - 1");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_last_error(TFB_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return set_last_error(TFB_ERR_ARG, "device index out of range");
  void* base = nullptr;
  e = scratch_on(dev, &base);
  if (e != hipSuccess) return set_last_error(TFB_ERR_HIP, (std::string("hipGetSymbolAddress: ") + hipGetErrorString(e)).c_str());
  float* lse = static_cast<float*>(base);
  float* loss_rows = lse + MAX_ROWS;
  e = tfb::softmax_ce_fwd(dev_logits, ld, dev_targets, rows, cols, lse, dev_loss, loss_rows,
                          static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return set_last_error(TFB_ERR_HIP, hipGetErrorString(e));
  return TFB_OK;
}
