// Device scratch of the allocation-free backward (hashgrid_backward_noalloc):
// a fixed array in the library's own device memory, so that callers who
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc) still get the binned table backward.
//
// The array is a file-scope __device__ variable: each GPU that loads the
// library holds its own copy, at its own address, until the process ends.
// Host code never uses the array's name as a device address (in host code it
// names a host-side stand-in); the device address is resolved once per
// device with hipGetSymbolAddress while that device is current, and kept.
// Every call on one GPU shares that GPU's copy: calls that overlap on a GPU
// (two streams, two host threads) race on it.
#include <mutex>

#include "hashgrid_internal.h"

static __device__ __align__(256) unsigned char scratch[hg::kNoallocScratchBytes];

namespace hg {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace hg
