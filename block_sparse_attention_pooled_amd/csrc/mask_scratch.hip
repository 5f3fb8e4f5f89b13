// Fixed device scratch for building the mask without a caller workspace
// (spa_build_mask_noalloc): the pooled means of Q and K live in a file-scope device array
// that each GPU holds from the first use of the library on it until the process ends.
//
// The array's name is a host-side stand-in, not a device address: host code uses only the
// pointer that hipGetSymbolAddress returns for the current device, queried once per device
// and kept in a table.  Every call on a GPU shares that GPU's array (calls that overlap on
// one GPU race); nothing in it needs to start at zero: the pooling writes every mean before
// the selection reads it.
#include <mutex>

#include "spa_internal.h"

namespace spa {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices];  // per device: the device address of `scratch`, once known
}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (stream != nullptr) {  // the scratch address is the current device's: so must the stream be
    hipDevice_t sd = -1;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return e;
    if (sd != dev) return hipErrorInvalidDevice;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace spa
