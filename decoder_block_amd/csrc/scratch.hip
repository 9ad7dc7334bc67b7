// Static device scratch for llama_layer_decode_noalloc: the workspace of a
// decode step for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array, so every GPU the library runs on
// holds its own copy (LLAMA_SCRATCH_BYTES bytes) from the moment the code
// object is loaded there until the process ends.  Host code must never pass
// the array's name to a kernel: on the host it is only a stand-in for the
// device symbol.  The device address of each GPU's copy is looked up once per
// device with hipGetSymbolAddress, with that device current, and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/llama_layer.h"
#include "kernels.h"

static __device__ __align__(256) unsigned char scratch[LLAMA_SCRATCH_BYTES];

namespace llk {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_region(void** ptr, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  *bytes = LLAMA_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace llk
