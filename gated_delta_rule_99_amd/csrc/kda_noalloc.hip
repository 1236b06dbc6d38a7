// The library's static device scratch, for kda_prefill_chunked_noalloc: the
// chunked prefill for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
// That entry point runs the same kernels as kda_prefill_chunked with a
// workspace, but the workspace is `scratch`, a file-scope device array of
// SCRATCH_BYTES that every GPU the library runs on holds until the process
// ends.
//
// In host code `scratch` names a host-side stand-in, not the array's device
// address: the address is looked up once per device with hipGetSymbolAddress
// (with that device current) and only that pointer is ever handed to kernels.
// Every call on one GPU shares that GPU's array and leaves the last call's
// contents in it; the prefill writes every byte it later reads (state carry,
// rank table, tiles), so nothing needs clearing.  Calls that overlap on one GPU
// (different streams, no ordering) race on the array.
#include <mutex>

#include "kda_internal.h"

namespace kda {
namespace {

constexpr size_t SCRATCH_BYTES = (size_t)128 << 20;
constexpr int MAX_DEVICES = 64;

__device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];

}  // namespace

size_t static_scratch_bytes() { return SCRATCH_BYTES; }

// The device address of `scratch` on the device that `stream` runs on (the
// current device for the null stream), looked up on the first call there.
hipError_t static_scratch(hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t err = hipSuccess;
    if (stream) {
        hipDevice_t d = 0;
        err = hipStreamGetDevice(stream, &d);
        dev = (int)d;
    } else {
        err = hipGetDevice(&dev);
    }
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        err = hipGetDevice(&cur);
        if (err != hipSuccess) return err;
        if (cur != dev && (err = hipSetDevice(dev)) != hipSuccess) return err;
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (err != hipSuccess) return err;
        if (back != hipSuccess) return back;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace kda
