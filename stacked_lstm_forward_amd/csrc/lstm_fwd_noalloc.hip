// lstm_fwd_noalloc: the forward pass for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).  It is lstm_fwd with the workspace taken from a fixed
// device array inside the library instead of a caller's buffer; the kernels,
// the planner and the launch sequence are lstm_fwd's own.
#include <hip/hip_runtime.h>

#include <mutex>

#include "lstm_fwd.h"  // include/ is on the include path

namespace {

constexpr size_t kScratchBytes = LSTM_FWD_NOALLOC_MAX_WORKSPACE;
constexpr int kMaxDevices = 64;

// The workspace of every lstm_fwd_noalloc call on a device: one copy per
// device, allocated when the library's code object is loaded there and held
// until the process ends.  Host code never passes this name to a kernel (on
// the host it is a stand-in, not a device address); it uses the address
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void* g_ptr[kMaxDevices];
std::mutex g_mu;

// Device address of `scratch` on the current device, looked up once per device.
lstm_status_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LSTM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LSTM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LSTM_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return LSTM_OK;
}

// Copies the call's device error word (the workspace's first int) into the
// caller's status word as an lstm_status_t.
__global__ void __launch_bounds__(64) lstm_status_copy(const int* err, int32_t* out) {
  if (threadIdx.x == 0) *out = *err != 0 ? (int32_t)LSTM_ERR_BARRIER_TIMEOUT : (int32_t)LSTM_OK;
}

}  // namespace

extern "C" lstm_status_t lstm_fwd_noalloc(const lstm_desc_t* d, const void* x, const void* h0, const float* c0,
                                          const void* W, const void* R, const void* b, void* y, void* hT,
                                          float* cT, int32_t* dev_status, hipStream_t stream) {
  // Host-only argument check first (nothing is enqueued on failure).  The
  // check never dereferences the workspace pointer; a 256-aligned stand-in
  // with the scratch size lets it report LSTM_ERR_WORKSPACE for problems that
  // need more than the scratch holds.
  void* const stand_in = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  lstm_status_t st = lstm_fwd_validate(d, x, W, R, b, y, stand_in, kScratchBytes);
  if (st != LSTM_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != LSTM_OK) return st;
  st = lstm_fwd(d, x, h0, c0, W, R, b, y, hT, cT, ws, stream);
  if (st != LSTM_OK || !dev_status) return st;
  hipLaunchKernelGGL(lstm_status_copy, dim3(1), dim3(64), 0, stream, static_cast<const int*>(ws), dev_status);
  return hipGetLastError() == hipSuccess ? LSTM_OK : LSTM_ERR_HIP;
}
