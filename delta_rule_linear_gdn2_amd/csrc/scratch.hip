// Library-owned device scratch for the entry point that allocates nothing
// (gdn2_chunk_bwd_noalloc): a file-scope device array of fixed size.  Each GPU
// the library runs on holds its own copy from the moment the library's code
// is loaded there until the process ends.
//
// In host code the array's name is only a host-side stand-in for the symbol,
// never a device address.  Its device address is looked up once per device
// with hipGetSymbolAddress, with that device current, and kept per device;
// kernels only ever receive that looked-up address.
//
// Every call on one GPU uses the same array, which keeps whatever the last
// call left there.  Calls that overlap on one GPU (two streams, two host
// threads) race on it.  Callers must serialise them.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <mutex>

#include "launch.hpp"

static __device__ __align__(256) unsigned char scratch[gdn2::kScratchBytes];

namespace gdn2 {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t scratch_pointer(void** out)
{
    *out = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            // device `dev` is current here: this is its copy of the array
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace gdn2
