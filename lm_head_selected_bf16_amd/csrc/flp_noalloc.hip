// Allocation-free forward (flp_forward_noalloc): flp_forward with its workspace in
// a fixed device array that the library holds on every device it runs on.
//
// The array is a file-scope __device__ object, so each device gets its own copy
// when the library's code object is loaded there, and it lives until the process
// ends.  Host code never passes the array's name to a kernel (on the host that
// name is only a stand-in symbol): the device address of each device's copy is
// looked up once per device with hipGetSymbolAddress, with that device current,
// and kept; every later call on that device uses the kept address.
//
// The forward writes every entry of the workspace it reads (the per-tile
// (max, sum of exp) pairs of rows < N, and the target logit of every row whose
// target is in range, the only rows whose target logit is read), so nothing in
// the array needs clearing between calls.  Calls that overlap in time on one
// device share the array and race; calls on different devices do not.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "flp_launch.h"

namespace {

constexpr size_t kScratchBytes = FLP_FORWARD_NOALLOC_MAX_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte blocks");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device.
flp_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FLP_HIP_ERROR;
  if (dev >= kMaxDevices) return FLP_UNSUPPORTED_DEVICE;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lk(g_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
        return FLP_HIP_ERROR;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FLP_OK;
}

}  // namespace

extern "C" flp_status flp_forward_noalloc(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                          const void* hidden, const void* weight,
                                          const float* bias, const void* targets,
                                          flp_dtype t_dtype, const float* temperature,
                                          float* out_logp, float* out_lse, void* stream) {
  flp_status st = flp::validate_forward_noalloc(N, D, V, x_dtype, hidden, weight, bias, targets,
                                                t_dtype, temperature, out_logp, out_lse,
                                                kScratchBytes);
  if (st != FLP_OK || N == 0) return st;
  if ((st = flp::check_device()) != FLP_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws)) != FLP_OK) return st;
  return flp::enqueue_forward(N, D, V, x_dtype, hidden, weight, bias, targets, t_dtype,
                              temperature, out_logp, out_lse, ws,
                              static_cast<hipStream_t>(stream));
}
