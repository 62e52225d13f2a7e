// Device scratch of fixed size for moe_layer_forward_noalloc: the decode
// forward's per-call arrays (logits, routing, dispatch, work and fill lists,
// h, fp32 expert outputs) carved out of one file-scope device array, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops).  Each GPU the library runs on holds its own copy of
// the array until the process ends; every call on a GPU shares it.
#include <mutex>

#include "moe_internal.h"

namespace moe {
namespace {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
uint8_t* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch_address(int device, uint8_t** out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[device]) {
    // the array's name is a host-side stand-in; the device address of this
    // device's copy comes from the runtime (the device is current here)
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[device] = static_cast<uint8_t*>(p);
  }
  *out = g_ptr[device];
  return hipSuccess;
}

}  // namespace moe
