// noalloc.hip -- the device scratch behind mla_dsa_decode_noalloc, for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops that forbid hipMalloc).
//
// `scratch` is one file-scope device array.  Each GPU that loads this library holds its own copy,
// at its own address, until the process ends.  In host code the array's name is only a host-side
// stand-in, not a device address, so it is never passed to a kernel or a copy: its device
// address on each device comes from hipGetSymbolAddress, looked up once per device (with that
// device current) and kept in g_ptr.  The decode step needs no cleared scratch (its kernels
// write every word they later read), so nothing is cleared; two calls that overlap on one GPU
// share the array and race.
#include <mutex>

#include "common.h"

namespace mla {

static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
static void *g_ptr[NOALLOC_MAX_DEVICES];
static std::mutex g_mu;

mla_status noalloc_scratch(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
        return fail(MLA_ERR_UNSUPPORTED, "static scratch: device index %d beyond %d", dev, NOALLOC_MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return MLA_OK;
}

}  // namespace mla
