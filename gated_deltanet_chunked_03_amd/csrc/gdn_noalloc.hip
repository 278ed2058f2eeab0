// gdn_fwd_noalloc: gdn_fwd with its workspace in a file-scope device array,
// for callers that cannot allocate device memory. See include/gdn.h.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn_internal.h"

namespace {

// The scratch array. In host code its name is only a host-side stand-in for
// the symbol: every host use goes through the device address that
// hipGetSymbolAddress returns for the current device (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// This device's copy of the array: looked up once per device, with that
// device current (each device holds its own copy at its own address).
gdn_status scratch_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return (gdn_status)gdn::record_error(GDN_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return (gdn_status)gdn::record_error(GDN_ERR_HIP, "device %d is beyond the %d devices served", dev,
                                             kMaxDevices);
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev])
        return (gdn_status)gdn::record_error(GDN_ERR_HIP, "hipGetSymbolAddress of the scratch array failed: %s",
                                             hipGetErrorString(g_scratch_err[dev]));
    *out = g_scratch_ptr[dev];
    return GDN_OK;
}

}  // namespace

extern "C" gdn_status gdn_fwd_noalloc(const gdn_desc* desc, const void* q, const void* k, const void* v,
                                      const float* g, const float* beta, float scale, const float* initial_state,
                                      const int32_t* cu_seqlens, void* out, float* final_state, void* stream) {
    // the workspace this descriptor needs (0 with a message on an invalid one)
    const size_t need = gdn_fwd_workspace_bytes(desc);
    if (need == 0) {
        gdn_plan_info info;
        const gdn_status st = gdn_plan(desc, &info);   // the planner's own status and message
        if (st != GDN_OK) return st;
    }
    if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
        return (gdn_status)gdn::record_error(
            GDN_ERR_WORKSPACE_TOO_SMALL,
            "gdn_fwd_noalloc: this descriptor needs %zu workspace bytes, above the %zu-byte scratch array "
            "(use gdn_fwd with a caller workspace)",
            need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    const gdn_status st = scratch_ptr(&ws);
    if (st != GDN_OK) return st;
    // gdn_fwd writes every workspace byte it reads: the array needs no clearing
    return gdn_fwd(desc, q, k, v, g, beta, scale, initial_state, cu_seqlens, out, final_state, ws,
                   (size_t)GDN_NOALLOC_SCRATCH_BYTES, stream);
}
