// noalloc.hip -- the device-resident scratch of lfm2sc_backward_noalloc.
//
// That entry point is lfm2sc_backward with its workspace (the per-window dW /
// dbias partial rows) taken from a fixed array in device memory instead of a
// caller buffer, for callers that cannot allocate.  `scratch` is that array:
// every GPU the library runs on holds one copy of it (at its own address) for
// the life of the process.  In host code its name only stands in for the
// symbol; the device address comes from hipGetSymbolAddress, asked once per
// device with that device current and kept in `g_addr`, and only that address
// is ever handed to a kernel.
//
// The partial rows need no clearing: the backward kernel writes every row and
// column its finishing kernel reads, in the same call.  Calls that overlap on
// one GPU (other streams, other host threads) share the array and race.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "lfm2sc.h"

namespace lfm2sc {

static __device__ __align__(256) unsigned char scratch[LFM2SC_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 256;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};
}  // namespace

size_t noalloc_scratch_bytes() { return sizeof(scratch); }

hipError_t noalloc_scratch(hipStream_t stream, void** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_addr[dev] == nullptr) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (back != hipSuccess) return back;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_addr[dev] = p;
    }
    *out = g_addr[dev];
    return hipSuccess;
}

}  // namespace lfm2sc
