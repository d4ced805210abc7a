// w4a8_gemm for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// split-K workspace is a static device array of this library instead of a
// caller buffer.
//
// The array lives for the life of the process, one copy per GPU the library
// runs on, each at its own device address.  That address is looked up once
// per device with hipGetSymbolAddress, with the device current; host code
// never passes the array's name to a kernel (on the host the name is only a
// stand-in for the symbol, not a device address).  Every call on a GPU
// shares that GPU's copy: calls that overlap on one GPU (different streams,
// no ordering between them) race on it.  The tile kernels overwrite every
// partial they later read, so no part of it has to start at zero.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "launch.h"
#include "w4a8.h"

#define W4A8_EXPORT extern "C" __attribute__((visibility("default")))

namespace w4a8 {

w4a8_status_t gemm_entry(const int8_t* X, const float* sx, const uint8_t* wq,
                         const uint8_t* s_u8, const uint8_t* a_u8, const float* sw, void* Y,
                         int out_type, int M, int N, int K, int group, int splitk,
                         void* workspace, size_t workspace_bytes, bool use_scratch,
                         hipStream_t stream);

namespace {

static __device__ __align__(256) uint8_t scratch[W4A8_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
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

}  // namespace w4a8

W4A8_EXPORT w4a8_status_t w4a8_gemm_noalloc(const int8_t* X, const float* sx, const uint8_t* wq,
                                            const uint8_t* s_u8, const uint8_t* a_u8,
                                            const float* sw, void* Y, int out_type, int M,
                                            int N, int K, int group, int splitk,
                                            hipStream_t stream) {
    return w4a8::gemm_entry(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K, group, splitk,
                            nullptr, W4A8_NOALLOC_SCRATCH_BYTES, true, stream);
}
