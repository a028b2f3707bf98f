// The library-owned device scratch of the no-allocation entry point
// (sa_decode_attention_append_noalloc): the split-K partials, the balanced
// kernel's unit records and the completion counters a call would otherwise
// keep in a caller's workspace.
//
// One array per GPU, in the code object: the loader creates it, zero-filled,
// on each device the library's kernels are loaded on, and it lives until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the
// host that name is only a stand-in for the symbol); it passes the device
// address hipGetSymbolAddress returns, looked up once per device with that
// device current and kept in `g_ptr`.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sa_internal.h"

static __device__ __align__(256) unsigned char scratch[sa::kScratchBytes];

namespace sa {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];         // device address of `scratch` on each device

}  // namespace

hipError_t scratch_pointer(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace sa
