// Static device scratch for callers that cannot allocate: the split partials of
// pkv_paged_decode_attention_noalloc live in a file-scope device array of
// kNoallocScratchBytes, one copy per GPU, held until the process ends.
//
// Host code never uses the array's name as an address (on the host it names a
// stand-in, not device memory): the first call on each device, with that
// device current, asks the runtime for the array's device address and keeps it
// for that device; kernels receive that address as an ordinary argument.

#include "pkv_internal.h"

#include <mutex>

namespace pkv {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || reinterpret_cast<uintptr_t>(p) % 256) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace pkv
