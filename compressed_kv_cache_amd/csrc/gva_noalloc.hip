// Fixed device scratch for the step that allocates nothing
// (gva_decode_step_noalloc).  The array is a file-scope device variable:
// each GPU the library's code is loaded on holds its own copy until the
// process ends.  In host code its name only stands for the symbol; the
// device address of the current GPU's copy comes from hipGetSymbolAddress,
// looked up once per device and kept, and only that address is ever passed
// to kernels.
#include <mutex>

#include "gva_internal.h"

namespace gva {

namespace {

__device__ __align__(256) unsigned char scratch[GVA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** addr) {
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
  *addr = g_addr[dev];
  return hipSuccess;
}

}  // namespace gva
