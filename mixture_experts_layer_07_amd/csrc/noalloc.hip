// Static device scratch of moe_expert_ffn_noalloc: the FFN's intermediate h
// for callers that cannot allocate device memory.  Each GPU the library runs
// on holds its own copy of the array for the life of the process; host code
// reaches it only through the device address looked up here (the array's
// name is a host-side stand-in, not a device pointer).
#include <mutex>

#include "common.h"

namespace moe {

static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // per device, resolved on first use
}  // namespace

void* noalloc_scratch()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        set_error(MOE_ERR_DEVICE, "noalloc scratch: no current device (or device id >= %d)", kMaxDevices);
        return nullptr;
    }
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            set_error(MOE_ERR_DEVICE, "noalloc scratch: hipGetSymbolAddress failed on device %d: %s", dev,
                      hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace moe
