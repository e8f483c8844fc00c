// noalloc.hip -- the device-resident scratch of vsa_forward_noalloc.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) get the forward pass
// with its workspace in a fixed array that lives in this library's code
// object: one copy per device, VSA_NOALLOC_SCRATCH_BYTES long, held from the
// first call on that device until the process ends.  The array is alone in
// this translation unit, so a process that never calls the allocation-free
// entry point never loads it.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// kernels must never be given that name.  The device address is obtained once
// per device, with that device current, through hipGetSymbolAddress, and only
// that address is handed to the kernels.
#include <mutex>

#include "vsa.h"
#include "vsa_internal.h"

namespace vsa {

static __device__ __align__(256) unsigned char scratch[VSA_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device
}  // namespace

hipError_t noalloc_scratch(void** out, size_t* bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || ((uintptr_t)p % kAlign) != 0) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    *bytes = sizeof(scratch);
    return hipSuccess;
}

}  // namespace vsa
