// moe_layer_decode_static: the whole layer with its scratch memory in a
// file-scope device array instead of a caller workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops
// that forbid allocation). Every call on one device shares that device's
// array: calls that may overlap in time on one device race.
#include <atomic>

#include "moe_internal.h"

namespace moe {

// The scratch: one copy per device (each device that runs the call holds it
// until the process ends). Host code never uses this name as an address: the
// device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch[kMaxScratchDevices];

// Zeroes the counter region at the start of the scratch: n16 16-byte words.
__global__ __launch_bounds__(256) void zero_counters(uint4 *__restrict__ p, int n16) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n16; i += gridDim.x * 256) p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t static_scratch_address(char **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void *ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    // First call on this device, which is current: look up this device's
    // copy of the array. Threads racing here store the same address.
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch[dev].store(ptr, std::memory_order_release);
  }
  *out = static_cast<char *>(ptr);
  return hipSuccess;
}

hipError_t clear_scratch_counters(char *ptr, hipStream_t s) {
  static_assert(kCounterBytes % 16 == 0, "counter region in 16-byte words");
  const int n16 = int(kCounterBytes / 16);
  zero_counters<<<64, 256, 0, s>>>(reinterpret_cast<uint4 *>(ptr), n16);
  return hipGetLastError();
}

}  // namespace moe
