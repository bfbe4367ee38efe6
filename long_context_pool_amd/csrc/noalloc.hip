// Device scratch for callers that cannot allocate (code under graph capture,
// tight serving loops, harnesses that forbid hipMalloc): a file-scope device
// array of fixed size, one copy per GPU, which misa_decode_step_noalloc uses
// in place of the caller's workspace.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address of each GPU's copy comes from hipGetSymbolAddress, looked up
// once per device (with that device current) on the first call there, and
// only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace misa {

namespace {

constexpr int kMaxDevices = 64;

static __device__ __attribute__((aligned(256))) uint8_t scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

}  // namespace

hipError_t static_scratch(void** ptr) {
  *ptr = nullptr;
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
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace misa
