// fa_noalloc.hip - the backward without a caller-provided workspace.
//
// fa_backward needs 8 B H N bytes of device scratch between its two launches
// (-D = -rowsum(dO * O) and -LSE log2 e per query row), which the caller
// passes in.  Callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc) use
// fa_backward_noalloc instead, whose scratch is the static device array below:
// every GPU the library runs on holds its own copy, from the first load of the
// library's code on that GPU until the process ends.
//
// On the host the array's name is only a stand-in for its symbol, not a device
// address: the address is looked up once per device with hipGetSymbolAddress
// (with that device current) and only that address is passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa_launch.hpp"

namespace fa {

// 2 floats per query row (the two [B, H, N] arrays of the workspace).
static __device__ __align__(256) float scratch[2 * kNoallocMaxRows];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float* g_ptr[kMaxDevices] = {};

// Device address of `scratch` on device `dev` (looked up on first use).
hipError_t scratch_on(int dev, float** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    g_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_bf16_noalloc(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                   const AttnShape& s, hipStream_t stream) {
  // The scratch of the GPU the stream runs on (the current device for the
  // null stream).
  hipDevice_t dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  float* ws = nullptr;
  if ((e = scratch_on((int)dev, &ws)) != hipSuccess) return e;
  // The preprocess overwrites every word the passes read, so nothing has to
  // be cleared between calls.
  return launch_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, ws, s, stream);
}

}  // namespace fa
