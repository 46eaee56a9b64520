// Device-resident scratch of the decode entry point that allocates nothing
// (gqa_decode_run_noalloc): the split partials go to a file-scope device
// array instead of a caller workspace.  Each device the library runs on
// holds its own copy from the first such call on that device until the
// process ends.
//
// In host code the array's name is a host-side stand-in, not a device
// address: the device address of the current device's copy is taken once
// per device with hipGetSymbolAddress and kept, and only that address is
// ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <mutex>

#include "gqa_decode.h"

namespace gqa {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[GQA_NOALLOC_SCRATCH_BYTES];

// Device address and size of the current device's scratch array.  The
// first call on a device looks the address up (with that device current)
// and every later call reuses it.
hipError_t scratch_address(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = GQA_NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace gqa
