// Scratch memory of tp_column_linear_noalloc: a static device array, so that the call allocates
// nothing (for callers that cannot allocate: code under HIP graph capture, tight serving loops).
// Every GPU the library runs on holds its own copy of the array until the process ends; all calls
// on one GPU share it, so calls that overlap on one GPU race.
#include <mutex>

#include "tp_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[TP_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

}  // namespace

namespace tpk {

// The host-side name `scratch` is not a device address: the array's address on a device comes
// from hipGetSymbolAddress with that device current, once per device, and only that address is
// handed to kernels.
hipError_t noalloc_scratch(hipStream_t s, void** ptr) {
    int dev = -1;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace tpk
