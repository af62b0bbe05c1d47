// ffn_noalloc.hip -- ffn_forward for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The workspace of ffn_forward_ex comes from a file-scope
// device array instead of the caller; inputs and outputs are still the
// caller's.
//
// The array is a device symbol: its host-side name is only a stand-in, so the
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that address is ever handed to the kernels.
// Each device holds its own copy until the process ends.  Every call on one
// device shares that copy and it keeps the last call's contents: the dense
// paths read only workspace bytes they wrote earlier in the same call, so
// nothing needs clearing, but calls that overlap on one device (different
// streams, threads or processes sharing a context) race on it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>

#include "ffn.h"
#include "ffn_internal.h"

namespace {

constexpr size_t kScratchBytes = FFN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

std::atomic<void*> g_scratch[ffn::kMaxDevices] = {};

thread_local char g_err_noalloc[256] = "";

// Device address of this device's copy of `scratch` (looked up on the first
// call on the device), or nullptr with the reason in g_err_noalloc.
void* scratch_ptr() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        snprintf(g_err_noalloc, sizeof g_err_noalloc, "hipGetDevice: %s", hipGetErrorString(e));
        return nullptr;
    }
    if (dev < 0 || dev >= ffn::kMaxDevices) {
        snprintf(g_err_noalloc, sizeof g_err_noalloc, "device %d beyond the supported %d", dev,
                 ffn::kMaxDevices);
        return nullptr;
    }
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
        snprintf(g_err_noalloc, sizeof g_err_noalloc, "hipGetSymbolAddress(scratch): %s",
                 hipGetErrorString(e));
        return nullptr;
    }
    g_scratch[dev].store(p, std::memory_order_release);   // concurrent first calls store the same value
    return p;
}

}  // namespace

extern "C" {

int ffn_forward_noalloc(const void* X, const void* W1, const void* b1, const void* W2,
                        const void* b2, void* Y, int64_t M, int64_t N, int64_t O, int64_t P,
                        int dtype, int act1, int act2, int variant, void* stream) {
    // the size check needs no device, so an oversized call is refused first
    const size_t need = ffn_workspace_size_ex(M, N, O, P, dtype, variant);
    if (need > kScratchBytes)
        return ffn::set_error(FFN_EWORKSPACE,
                              "this shape needs %zu bytes of workspace; the static scratch of "
                              "ffn_forward_noalloc holds %zu",
                              need, kScratchBytes);
    void* ws = scratch_ptr();
    if (!ws) return ffn::set_error(FFN_ELAUNCH, "%s", g_err_noalloc);
    return ffn_forward_ex(X, W1, b1, W2, b2, Y, M, N, O, P, dtype, act1, act2, variant, ws,
                          kScratchBytes, stream);
}

}  // extern "C"
