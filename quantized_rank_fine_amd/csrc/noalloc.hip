// Device-resident scratch of the forward entry point that allocates nothing
// (qlora_linear_fwd_noalloc): for callers that cannot allocate device memory
// at the call -- code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc.
//
// The array lives in the library's code object, one copy per GPU the
// library runs on, held until the process ends.  Host code never passes the
// array's name to a kernel or a copy (in host code that name is a host-side
// stand-in, not a device address): the device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and only that
// address is handed out.  Every call on one GPU shares that GPU's copy, so
// calls that overlap on one GPU race; nothing in it needs to start at zero
// (every byte the forward reads from its workspace is written first by the
// same call).
#include <mutex>

#include <hip/hip_runtime.h>

#include "internal.h"

static __device__ __align__(256) unsigned char scratch[qlora::kNoAllocScratchBytes];

namespace qlora {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace qlora
