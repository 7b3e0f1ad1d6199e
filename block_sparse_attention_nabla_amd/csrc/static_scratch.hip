// static_scratch.hip -- library-held scratch memory for the allocation-free
// forward entry point (nabla_sparse_attn_fwd_static).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy (kStaticScratchBytes) until the process ends. In host code its
// name is only a host-side stand-in, never a device address: the device
// address is queried once per device with hipGetSymbolAddress (with that device
// current) and cached, and only that pointer is handed to kernels. Calls that
// overlap on one GPU share the array and therefore race.

#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace nabla {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch_ptr(hipStream_t stream, void** out) {
    *out = nullptr;
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream != nullptr) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_ptr[dev] == nullptr) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace nabla
