// Library-owned device scratch for callers that cannot allocate.
//
// bsa_forward_split_static runs the key split of the frame-0 rows with its
// partial softmax states in `scratch`, a file-scope device array of
// kStaticScratchBytes: every GPU the library runs on holds its own copy
// until the process ends.  Host code never uses the array's name as an
// address (in host code it names a host-side stand-in); the device address
// of each GPU's copy is looked up once per device with hipGetSymbolAddress,
// with that device current, and kept here.
#include <mutex>

#include "bsa_internal.h"

namespace bsa {
namespace {

__device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices];   // device address of each GPU's copy (null: not looked up yet)

}  // namespace

hipError_t static_scratch(float** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace bsa
