// Fixed device scratch for attnqat_fwd_noalloc, the forward entry point for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The buffer is a file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends. In host
// code the array's name is only a stand-in, never a device address, so the
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and that pointer is what the kernels are given.
#include <hip/hip_runtime.h>

#include <mutex>

#include "aq_kernels.h"

namespace aq {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];
}  // namespace

// Device address of `scratch` on device `dev`, which must be the current
// device; looked up on the first call for that device and kept.
hipError_t noalloc_scratch(int dev, void** out) {
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace aq
