// The library's one static device workspace: a file-scope array that every
// GPU the library runs on holds from module load until the process ends,
// for the entry points that must not allocate (magi_ffa_bwd_noalloc).
//
// In host code the array's name is only a host-side stand-in; the device
// address of each GPU's copy comes from hipGetSymbolAddress, taken once per
// device with that device current and kept here.  Host code passes that
// address, never the array's name, to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace magi {
namespace {

static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_for_stream(void* stream, float** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipSuccess;
  // the stream's own device (the current one for the null stream)
  if (stream != nullptr)
    e = hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dev);
  else
    e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (back != hipSuccess) return back;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace magi
