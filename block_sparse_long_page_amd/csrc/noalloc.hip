// Static device scratch for the entry point that allocates nothing
// (sparse_attn_decode_step_static): the selecting step's workspace and the
// split partials live in one file-scope device array, which every GPU the
// library runs on holds (zero-initialised at load) until the process ends.
//
// In host code the array's name stands for a host-side shadow, not a device
// address: the device address is taken once per device with
// hipGetSymbolAddress (with that device current) and kept, and only that
// address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace sa {

namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once taken

}  // namespace

hipError_t static_scratch(void** ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace sa
