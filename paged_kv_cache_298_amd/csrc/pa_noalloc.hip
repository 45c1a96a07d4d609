// pa_noalloc.hip -- the library-held scratch of pa_decode_noalloc, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).
//
// The scratch is one file-scope device array of kScratchBytes per GPU, loaded with the
// code object and held until the process ends. In host code the array's name is only a
// stand-in, not a device address: the address is looked up once per device, with that
// device current, by hipGetSymbolAddress, and that pointer is what the kernels receive.
// Every call on one GPU shares its array; calls that overlap on one GPU (several streams,
// several host threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[pa_internal::kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace pa_internal {

int scratch_pointer(void** ptr, const char** err) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *err = hipGetErrorString(e);
        return (int)e;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *err = "device index beyond the library's table of scratch addresses";
        return (int)hipErrorInvalidDevice;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *err = e != hipSuccess ? hipGetErrorString(e) : "null scratch address";
            return e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol;
        }
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return 0;
}

}  // namespace pa_internal
