// moe_forward_packed_noalloc: moe_forward_packed with its workspace in a
// fixed device array of this library instead of a caller buffer, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ variable: every GPU the library's code
// object is loaded on holds its own copy (MOE_NOALLOC_WORKSPACE_BYTES) until
// the process ends. In host code the name `scratch` is only a host-side
// stand-in for that variable; its device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and kept, and
// only that address is ever handed to kernels.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/moe_routed.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device ordinal
std::mutex g_mu;

// Address of this device's copy of `scratch`, where `dev` is the current
// device. Resolved on the first call for that device, then reused.
int scratch_of(int dev, void **out)
{
    if (dev < 0 || dev >= kMaxDevices) return MOE_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" int moe_forward_packed_noalloc(const void *x, const int32_t *ids, const float *w,
                                          const void *pw_gate, const void *pw_up,
                                          const void *pw_down, int dtype, int T, int K, int E,
                                          int d, int f, int tm, float *out, moe_stream_t stream)
{
    // size checks first: nothing below runs for a request that cannot fit
    size_t need = 0;
    const int rc = moe_forward_workspace(T, K, E, d, f, tm, dtype, &need);
    if (rc != MOE_OK) return rc;
    if (need > (size_t)MOE_NOALLOC_WORKSPACE_BYTES) return MOE_ENOSPACE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
    if (stream) {
        // kernels run on the stream's device: it must be the one whose array
        // address is used
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
            return MOE_EHIP;
        if (sdev != dev) return MOE_EINVAL;
    }
    void *ws = nullptr;
    const int rs = scratch_of(dev, &ws);
    if (rs != MOE_OK) return rs;
    return moe_forward_packed(x, ids, w, pw_gate, pw_up, pw_down, dtype, T, K, E, d, f, tm, ws,
                              (size_t)MOE_NOALLOC_WORKSPACE_BYTES, out, stream);
}
