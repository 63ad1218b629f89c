// Device scratch behind icp_align_noalloc (kdnn.h): the ICP workspace for
// callers that cannot allocate device memory.  The array is a module global,
// so every device holds its own copy from the moment the library's code is
// loaded onto it until the process ends.  Host code never passes the array's
// name to a kernel or a copy (on the host it is only a stand-in for the
// symbol); it asks the runtime for the current device's address of its copy
// once per device and uses that address from then on.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kdnn_internal.hpp"

namespace kdnn {

static_assert(KDNN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size: a multiple of 256 bytes");

static __device__ __align__(256) unsigned char scratch[KDNN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_setup_mu;            // guards g_ptr
void *g_ptr[kMaxDevices] = {};    // device address of each device's copy
std::mutex g_call_mu[kMaxDevices];  // one call at a time per device

}  // namespace

hipError_t noalloc_scratch(int device, void **ptr, std::mutex **call_mu)
{
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_setup_mu);
    if (!g_ptr[device]) {
        // with `device` current (the caller's current device): its copy
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[device] = p;
    }
    *ptr = g_ptr[device];
    *call_mu = &g_call_mu[device];
    return hipSuccess;
}

}  // namespace kdnn
