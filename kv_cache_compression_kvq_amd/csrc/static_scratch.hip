// Scratch of the allocation-free decode entry point
// (kvq_decode_qjl_int8_noalloc): the projected queries and softmax partials
// that kvq_decode_qjl_int8 keeps in a caller workspace live here instead.
//
// The array is a module global, so every device the library runs on holds
// its own copy, at its own address, from module load until the process ends.
// Host code never passes the array's name to a kernel or a copy (its
// host-side symbol is only a stand-in, not a device address): the device
// address is looked up once per device, with that device current, and cached.
#include "kvq_launch.h"

#include <mutex>

namespace kvq {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace kvq
