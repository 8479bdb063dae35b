// Fixed device scratch for the entry point that allocates nothing
// (rk_online_softmax_noalloc): a file-scope device array, one copy per GPU,
// held until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol, not a device
// address); it asks the runtime for the array's address on each device once,
// with that device current, and passes that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "rk_internal.h"

static __device__ __align__(256) char scratch[rk::kScratchBytes];

namespace rk {

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mutex;
void *g_address[kMaxDevices];  // per device; null until looked up

}  // namespace

hipError_t scratch_address(int device, void **address)
{
    if (device < 0 || device >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_address[device] == nullptr) {
        void *p = nullptr;
        const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess)
            return err;
        if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0)
            return hipErrorInvalidSymbol;
        g_address[device] = p;
    }
    *address = g_address[device];
    return hipSuccess;
}

}  // namespace rk
