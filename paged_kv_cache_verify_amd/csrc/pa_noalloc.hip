// The static scratch of the zero-allocation attention call
// (pa_decode_verify_noalloc): the work list, the reduce lists and the
// partial results of one call live in a file-scope device array instead of
// memory a plan allocates, so a caller that cannot allocate device memory
// can run a host-only plan.
//
// Each device the library runs on holds its own copy of the array, at its
// own address, from the code object's load until the process ends. In host
// code `scratch` names a host-side stand-in, not device memory: its device
// address comes from hipGetSymbolAddress with the device current, looked up
// once per device and kept here; everything on the host side uses that
// address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_internal.h"

namespace pav {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace pav
