// static_scratch.hip -- device memory for paged_attention_decode_static, the decode
// entry point that allocates nothing.
//
// The decode kernels keep their partial records (and the balanced split its
// per-sequence start units and merge notes) in a scratch buffer.  For callers that
// cannot allocate, that buffer is the file-scope device array below: every GPU the
// library runs on holds its own copy, at its own address, from the time the
// library's code is loaded on it until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory, so the host never passes it to a
// kernel: the address of each device's copy is looked up once, with that device
// current, and kept.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "internal.h"

namespace pkv {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_lookup;
}  // namespace

hipError_t static_scratch_address(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_lookup);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace pkv
