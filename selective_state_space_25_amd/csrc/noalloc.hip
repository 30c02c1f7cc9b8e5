// noalloc.hip -- the Mamba-1 forward scan for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): selscan_fwd_noalloc runs the kernels of selscan_fwd_h0 with
// their scratch (the fp32 B/C records and the chunk summaries) in a
// file-scope device array of fixed size instead of a workspace.
//
// The array is a per-device object: every GPU the library runs on holds its
// own copy until the process ends.  Its device address is looked up once per
// device (hipGetSymbolAddress with that device current) and cached; host code
// passes that address, never the array's name, to the kernels.  Calls that
// overlap on one device share the array and race; they must be ordered (one
// stream, or events between streams).  Nothing in the scratch needs to start
// at zero: every word a call reads it has written earlier in the same call.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "kernels.hpp"
#include "selscan.h"

namespace {

constexpr size_t kScratchBytes = SELSCAN_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size must keep 256-byte alignment");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {nullptr};

// Device address of this device's scratch array (looked up on the first call
// on the device, with the device current).
selscan_status_t scratch_ptr(int dev, void** out) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return selscan::set_error(SELSCAN_ERR_LAUNCH, std::string("hipGetSymbolAddress of the scratch array failed: ") +
                                                              hipGetErrorString(e));
        }
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return SELSCAN_OK;
}

}  // namespace

extern "C" selscan_status_t selscan_fwd_noalloc(const selscan_shape_t* shape, const void* u, const void* delta,
                                                const float* A, const void* B, const void* C, const float* D,
                                                const void* z, const float* delta_bias, int softplus,
                                                const float* h0, void* y, float* last_state, void* stream) {
    try {
        if (!shape) return selscan::set_error(SELSCAN_ERR_INVALID_ARG, "shape is NULL");
        selscan_shape_t s = *shape;
        s.workspace = nullptr;
        s.workspace_bytes = 0;
        // 0 for a shape selscan_fwd_h0 rejects; it reports why below
        const size_t need = selscan_workspace_bytes(&s);
        if (need > kScratchBytes)
            return selscan::set_error(SELSCAN_ERR_WORKSPACE,
                                      "selscan_fwd_noalloc: this shape needs " + std::to_string(need) +
                                          " scratch bytes, more than its fixed maximum of " +
                                          std::to_string(kScratchBytes) + " (use selscan_fwd with a workspace)");
        if (need > 0) {
            int dev = -1;
            if (hipGetDevice(&dev) != hipSuccess || dev < 0)
                return selscan::set_error(SELSCAN_ERR_NO_DEVICE, "no HIP device available");
            if (dev >= kMaxDevices)
                return selscan::set_error(SELSCAN_ERR_UNSUPPORTED, "selscan_fwd_noalloc supports device ids below 64");
            void* p = nullptr;
            const selscan_status_t st = scratch_ptr(dev, &p);
            if (st != SELSCAN_OK) return st;
            s.workspace = p;
            s.workspace_bytes = kScratchBytes;
        }
        // with a workspace of the required size the call allocates nothing
        return selscan_fwd_h0(&s, u, delta, A, B, C, D, z, delta_bias, softplus, h0, y, last_state, stream);
    } catch (...) {
        return selscan::set_error(SELSCAN_ERR_LAUNCH, "unexpected host exception");
    }
}
