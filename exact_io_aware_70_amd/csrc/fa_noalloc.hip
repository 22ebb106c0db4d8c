// The backward pass's scratch in a static device array, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): fa_bwd_noalloc takes its workspace (D = rowsum(dout * o) and lse * log2(e))
// from `scratch` instead of a caller-supplied buffer.
//
// `scratch` is a file-scope __device__ array: each GPU the library runs on holds its own
// copy, at its own address, until the process ends.  In host code its name is only a
// stand-in, so the device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and cached; every kernel argument uses the cached address.
// Every call on one GPU shares that GPU's copy: calls that overlap on one GPU race.  The
// contents need no clearing: the backward's first kernel writes every value the later
// kernels read.
#include <mutex>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace fa {

static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_mutex;

}  // namespace

hipError_t scratch_address(hipStream_t stream, void** out) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream) {
        hipDevice_t sd = 0;
        if ((e = hipStreamGetDevice(stream, &sd)) != hipSuccess) return e;
        dev = (int)sd;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        // The symbol's address on `dev` is only defined with `dev` current.
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace fa
