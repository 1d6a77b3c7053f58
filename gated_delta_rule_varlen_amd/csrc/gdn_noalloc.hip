// gdn_noalloc.hip -- gdn_scan_varlen_noalloc: gdn_scan_varlen for callers that cannot allocate device
// memory (code under HIP graph capture, serving loops, harnesses that forbid hipMalloc).
//
// The workspace the chunked path needs lives in `scratch`, a file-scope device array of
// GDN_NOALLOC_SCRATCH_BYTES that the HIP runtime places once on every device the library runs on
// and keeps until the process ends.  In host code the array's name only stands for the symbol (it
// is not a device address), so each device's address is looked up once with hipGetSymbolAddress,
// with that device current, and only that address is handed to kernels.  Nothing here allocates.
//
// Every call on a device shares that device's array and leaves its contents behind; the kernels
// initialise whatever they read (the chunk table header is written before it is read), so nothing
// has to start at zero.  Calls that overlap in time on one device (different streams, or different
// host threads) race on the array and must be serialised by the caller.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "gdn.h"
#include "gdn_launch.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (looked up on the first call on that device).
gdn_status current_scratch(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ERR_HIP;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GDN_ERR_HIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return GDN_OK;
}

}  // namespace

extern "C" gdn_status gdn_scan_varlen_noalloc(const gdn_scan_desc* desc, const void* qkv, const float* qk_prep,
                                              const float* gb_prep, const void* a, const void* b, const float* A_log,
                                              const float* dt_bias, const float* state_in, void* out,
                                              float* state_out, const int32_t* offsets, int32_t* dev_status,
                                              int32_t* path_used, hipStream_t stream) {
    return gdn::scan_varlen_scratch(desc, qkv, qk_prep, gb_prep, a, b, A_log, dt_bias, state_in, out, state_out,
                                    offsets, current_scratch, GDN_NOALLOC_SCRATCH_BYTES, dev_status, path_used,
                                    stream);
}
