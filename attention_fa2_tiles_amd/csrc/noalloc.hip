// Device-resident scratch for the entry point that allocates nothing
// (fa_bwd_noalloc): the backward's Delta rows live in a file-scope device
// array instead of a caller-provided workspace.
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it names a stand-in, not device memory): the device address of each
// GPU's copy is looked up once, with that GPU current, and kept per device.
// Every call on a GPU shares that GPU's copy, so calls that overlap on one
// GPU (concurrent streams or threads) race on it; the backward writes every
// Delta row it reads before reading it, so nothing needs clearing.
#include <mutex>

#include "kernels.h"

namespace fa {
namespace {

static __device__ __align__(256) float scratch[kNoAllocDeltaRows];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
float* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_delta_scratch(size_t rows, float** out) {
  *out = nullptr;
  if (rows > (size_t)kNoAllocDeltaRows) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace fa
