// static_scratch.hip -- the workspace of vqkv_decode_step_static: a
// file-scope device array, so that the call needs no allocation by the
// caller or the library.
//
// Each GPU the library runs on holds its own copy of `scratch` for the life
// of the process.  In host code the array's name is only a stand-in, not a
// device address: the device address of this GPU's copy comes from
// hipGetSymbolAddress, taken once per device (with that device current) and
// kept; every use from the host goes through it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace vqkv {

namespace {

__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_addr[kMaxDevices];
hipError_t g_status[kMaxDevices];

}  // namespace

hipError_t static_scratch(void** addr, int* device) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_once[dev], [dev] {
        // The current device is `dev`: this is its copy's address.
        void* p = nullptr;
        g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_addr[dev] = p;
    });
    if (g_status[dev] != hipSuccess) return g_status[dev];
    *addr = g_addr[dev];
    if (device) *device = dev;
    return hipSuccess;
}

}  // namespace vqkv
