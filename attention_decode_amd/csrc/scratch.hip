// Static device scratch for callers that cannot allocate (code under HIP graph
// capture, serving loops that forbid hipMalloc): the decode workspace of
// tq_attend_decode_noalloc lives in one file-scope device array per GPU.
//
// In host code `scratch` names a host-side stand-in, not device memory, so
// its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to kernels.
#include "tq_internal.h"

#include <mutex>

namespace tq {

constexpr size_t kScratchBytes = static_cast<size_t>(16) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t scratch_capacity() { return kScratchBytes; }

hipError_t scratch_address(void **out)
{
    *out = nullptr;
    int dev = 0;
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

}  // namespace tq
