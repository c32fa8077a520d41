// ra_ring_forward_noalloc: the ring forward for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops, harnesses that
// forbid hipMalloc).  Its scratch -- the running states, key-range partials
// and tile-queue counters that ra_ring_forward keeps in the caller's
// workspace -- lives in a file-scope device array of kScratchBytes.  The first
// call on a GPU looks its address up (the HIP runtime backs the array with
// device memory then, and the GPU holds it until the process ends); every
// call launches on the caller's stream in order and creates no stream, event
// or device memory of its own.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ra.h"
#include "ra_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(256) << 20;  // 256 MiB

// Device-side scratch.  In host code `scratch` only names the symbol: its
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device (NULL on failure,
// with *err set).
void* scratch_address(hipError_t* err) {
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

thread_local char g_msg[256];

}  // namespace

extern "C" {

size_t ra_ring_noalloc_max_bytes(void) { return kScratchBytes; }

ra_status ra_ring_forward_noalloc(const ra_ring_desc* desc, const void* q, const void* k, const void* v, void* o,
                                  float* lse, void* stream) {
    if (!desc) return ra::ring_forward_on_stream(desc, q, k, v, o, lse, nullptr, 0, stream);
    if (desc->stats || desc->emulate_copy)
        return ra::set_error(RA_ERR_UNSUPPORTED,
                             "ra_ring_forward_noalloc: stats and emulate_copy need library streams and events");
    ra_ring_desc d = *desc;
    d.n_streams = 1;  // one stream: the caller's
    size_t need = 0;
    const ra_status st = ra_ring_workspace_size(&d, &need);
    if (st != RA_OK) return st;
    if (need > kScratchBytes) {
        // report through the library's error message: an oversize call is a
        // workspace error, found before anything is launched
        snprintf(g_msg, sizeof(g_msg), "ra_ring_forward_noalloc: %zu bytes of scratch needed, at most %zu held",
                 need, kScratchBytes);
        return ra::set_error(RA_ERR_WORKSPACE, g_msg);
    }
    hipError_t e = hipSuccess;
    void* ws = scratch_address(&e);
    if (!ws) return ra::set_error(RA_ERR_HIP, hipGetErrorString(e));
    return ra::ring_forward_on_stream(&d, q, k, v, o, lse, ws, kScratchBytes, stream);
}

}  // extern "C"
