// noalloc.hip -- device scratch for the entry point that allocates nothing
// (mla_absorbed_attention_noalloc).  The split-KV partial results of that call
// live in one file-scope device array instead of a caller workspace.  Its
// device address is looked up once per device, with that device current, and
// kept; host code never passes the array's own name to a kernel (on the host
// that name is only a stand-in for the symbol, not a device address).

#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace mla {

// Every GPU the library runs on holds one copy of this array until the
// process ends.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices] = {};
}  // namespace

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    scratch_dev[dev] = ptr;
  }
  *out = scratch_dev[dev];
  return hipSuccess;
}

}  // namespace mla
