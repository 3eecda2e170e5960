// kla_noalloc.hip -- device scratch of klaFwdNoAlloc, the forward entry point
// for callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The sequence split of the diagonal forward passes its block products,
// carries, local states and q-hat tiles through a workspace (klaFwd takes it
// from the caller).  Here it is one file-scope device array of
// kNoAllocScratchBytes; every GPU the library runs on holds its own copy
// until the process ends.  Its device address is looked up once per device,
// with that device current, and kept: in host code the array's name is only
// a host-side stand-in.  Every call on one GPU shares that GPU's copy, which
// keeps the previous call's contents; the split writes every word it reads
// within the call, so nothing needs clearing.  Calls that overlap on one GPU
// (several streams, several host threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kla_internal.h"

namespace kla {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace kla
