// libgdn: the allocation-free forward entry point (gdn_fwd_noalloc), whose
// workspace is a static device array of this file; everything else of the C
// ABI is in gdn_plan.cpp.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace {

int err(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int err(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    return gdn::set_error(status, buf);
}

// ---- the allocation-free forward's workspace: one static device array per
// GPU (each device holds its own copy, at its own address, from the time the
// library's code object is loaded on it until the process ends).  Host code
// never passes `scratch` itself (its host-side name is a stand-in, not a
// device address): the address is looked up once per device with that device
// current and kept in g_scratch_dev.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

// This thread's current device, the stream's device (they must agree), and the
// device address of that device's scratch array.
int scratch_for_stream(void *stream, void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return err(GDN_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return err(GDN_EHIP, "device index %d out of range", dev);
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e != hipSuccess) return err(GDN_EHIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    if ((int)sdev != dev)
        return err(GDN_EINVAL, "the stream belongs to device %d but device %d is current", (int)sdev, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return err(GDN_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_fwd_noalloc(const gdn_fwd_desc *d, const gdn_fwd_ptrs *p, void *stream) {
    size_t need = 0;
    const int rc = gdn::fwd_workspace_bytes(d, &need);
    if (rc != GDN_OK) return rc;
    if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
        return err(GDN_EWORKSPACE,
                   "this call needs %zu bytes of workspace; the allocation-free entry point has %zu (use gdn_fwd "
                   "with a caller workspace, or a longer segment length)",
                   need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if (need > 0) {
        const int rs = scratch_for_stream(stream, &ws);
        if (rs != GDN_OK) return rs;
    }
    return gdn_fwd(d, p, ws, need, stream);
}

}  // extern "C"
