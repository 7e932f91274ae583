// scratch.hip -- the library's static device scratch, for the entry points
// that allocate nothing (ssd_chunk_scan_fwd_noalloc): a file-scope device
// array that every GPU the library runs on holds until the process ends.
//
// In host code the array's name stands for a host-side shadow, not a device
// address, so it is never passed to a kernel or a copy: its address on the
// current device is looked up once per device with hipGetSymbolAddress and
// kept, and callers use that address only.
#include <hip/hip_runtime.h>
#include <mutex>

#include "launchers.hpp"

namespace ssm {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_addr[kMaxDevices] = {};   // device address of scratch on each device, once looked up
}  // namespace

hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with this device current
        if (e != hipSuccess) return e;
        g_addr[dev] = p;
    }
    *out = g_addr[dev];
    return hipSuccess;
}

}  // namespace ssm
