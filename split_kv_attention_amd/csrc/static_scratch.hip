// Library-owned device memory: the scratch of sk_attn_partial_noalloc, the
// variant of sk_attn_partial for callers that cannot allocate device memory,
// and (bounds-checked build only) the record of out-of-range accesses.
//
// The array lives in the code object: every GPU the library is loaded on
// holds its own copy (kStaticScratchBytes) until the process ends.  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol); it looks up the device address once per device
// with hipGetSymbolAddress, with that device current, and hands that
// address to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sk_common.hpp"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[sk::kStaticScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

#if SK_CHECKED
// The bounds-checked build's violation record (zero at load).
static __device__ __align__(256) sk::CheckRecord check_rec;
void* g_check[kMaxDevices] = {};
#endif

}  // namespace

namespace sk {

hipError_t static_scratch(void** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

hipError_t check_record(CheckRecord** out) {
    *out = nullptr;
#if SK_CHECKED
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_check[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(check_rec));
        if (e != hipSuccess) return e;
        g_check[dev] = p;
    }
    *out = static_cast<CheckRecord*>(g_check[dev]);
#endif
    return hipSuccess;
}

}  // namespace sk
