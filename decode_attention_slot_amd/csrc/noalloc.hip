// The library's own device workspace, for the decode entry point that
// allocates nothing (paged_decode_attention_noalloc): callers under HIP graph
// capture, tight serving loops or harnesses that forbid hipMalloc pass only
// their inputs and outputs, and the split-K partials go here.
//
// `scratch` is a file-scope device array: every device the library runs on
// holds its own copy (kNoallocScratchBytes) from the loading of the code
// object until the process ends. In host code its name is a host-side
// stand-in, not a device address, so it is never passed to a kernel or a
// copy: its address on each device comes from hipGetSymbolAddress, taken
// once per device with that device current and kept here.
#include <atomic>

#include "kvslot_internal.h"

namespace kvs {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<uintptr_t> g_scratch_addr[kMaxScratchDevices];

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  uintptr_t a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (a == 0) {
    // First call on this device (this device is current): look the array up.
    // Two threads racing here both get the same address.
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    a = reinterpret_cast<uintptr_t>(p);
    g_scratch_addr[dev].store(a, std::memory_order_release);
  }
  *ptr = reinterpret_cast<void*>(a);
  return hipSuccess;
}

}  // namespace kvs
