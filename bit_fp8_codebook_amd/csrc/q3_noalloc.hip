// Per-device state of the library.
//
// Library-owned scratch memory, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the fused expert MLP's intermediate buffers (the SwiGLU
// activations and the per-pair down outputs) live in one file-scope device
// array instead of a caller workspace.  Each GPU the library runs on holds its
// own copy of the array (allocated with the code object, held until the process
// ends); its device address is looked up once per device with
// hipGetSymbolAddress and kept here.  Host code never passes the array's name
// itself to a kernel or a copy: in host code that name is only a stand-in for
// the symbol, not a device address.
//
// The dynamic-LDS allowances of the kernels, which are per device too.
#include <atomic>
#include <mutex>

#include "q3_internal.h"

namespace q3 {
namespace {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // First call on this device (it is current): resolve the array's address.
    // Two threads racing here both store the same address.
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t allow_dynamic_lds(const void* kernel, size_t bytes, LdsAllowance& seen) {
  if (bytes <= 64 * 1024) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool tracked = dev >= 0 && dev < kMaxDevices;
  if (tracked && bytes <= seen.bytes[dev].load(std::memory_order_acquire)) return hipSuccess;
  // Raising the allowance is serialized, so that the attribute only grows: two
  // threads raising it at once to different sizes could otherwise leave the
  // smaller one set while the larger one is recorded.
  static std::mutex raise;
  std::lock_guard<std::mutex> lock(raise);
  if (tracked && bytes <= seen.bytes[dev].load(std::memory_order_acquire)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess && tracked) seen.bytes[dev].store(bytes, std::memory_order_release);
  return e;
}

}  // namespace q3
