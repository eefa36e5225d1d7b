// mla_verify_run_static: the verify call for callers that cannot allocate
// (code under hipGraph capture, tight serving loops, harnesses that forbid
// device allocation).  It runs the same two launches as mla_verify_run with a
// workspace taken from a file-scope device array instead of the caller.
//
// The array `scratch` is a device symbol: in host code its name is only a
// host-side stand-in, never a device address.  Its address on a device is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and cached; only that pointer is ever passed to the kernels.
// Every call on a device shares that device's array, which keeps the last
// call's contents: the kernels need nothing zeroed (each call writes every
// region before reading it), and calls that overlap on one device race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mla_verify_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MLA_VERIFY_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // per device: the array's device address, once looked up

// The array's address on the current device, looked up on first use.
void* device_scratch(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !ptr) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" mla_verify_status_t mla_verify_run_static(const mla_verify_plan_t* plan, const mla_verify_args_t* args,
                                                     void* stream) {
  size_t need = 0;
  const mla_verify_status_t st = mla_verify_workspace_size(plan, &need);
  if (st != MLA_VERIFY_OK) return st;
  if (need > (size_t)MLA_VERIFY_STATIC_SCRATCH_BYTES) return MLA_VERIFY_ERR_WORKSPACE_TOO_SMALL;
  // argument errors are reported before any HIP call (a 256-byte aligned
  // stand-in for the workspace lets run's own checks run on the host first)
  const mla_verify_status_t ast =
      mlav::check_call(plan, args, reinterpret_cast<void*>(256), (size_t)MLA_VERIFY_STATIC_SCRATCH_BYTES);
  if (ast != MLA_VERIFY_OK) return ast;
  hipError_t err = hipSuccess;
  void* ws = device_scratch(&err);
  if (!ws) return MLA_VERIFY_ERR_LAUNCH;
  return mla_verify_run(plan, args, ws, (size_t)MLA_VERIFY_STATIC_SCRATCH_BYTES, stream);
}
