// gdn2_noalloc.hip -- gdn2_chunk_fwd for callers that cannot allocate device memory.
//
// The workspace of the chunked forward comes from `scratch`, a static device array that the
// HIP runtime places on every GPU the library runs on when it loads the code object, and
// that each GPU keeps until the process ends. The host never passes the array's name to a
// kernel: in host code that name is only a host-side stand-in. The device address is looked
// up once per device with hipGetSymbolAddress (that device current) and cached; every use
// goes through the cached pointer.
//
// The kernels of the chunked forward write every workspace byte they read within one call
// (the chunk map, the per-chunk records, the segment states and transitions), so nothing
// in the array has to start at zero and the previous call's contents are harmless. All
// calls on one GPU share its array: calls that may overlap in time on one GPU (different
// streams without ordering between them) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn2.h"
#include "gdn2_internal.h"

namespace {

static_assert(GDN2_STATIC_WORKSPACE_BYTES % 256 == 0, "whole 256-byte blocks");

__device__ __align__(256) unsigned char scratch[GDN2_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// Device address of `scratch` on device `dev` (looked up with that device current once,
// then cached). Returns the HIP error of the lookup, if any.
hipError_t scratch_ptr(int dev, void **out) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_ptr[dev] == nullptr) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" gdn2_status gdn2_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                              const void *log_alpha, const void *b,
                                              const void *w, const float *S0,
                                              const int32_t *cu_seqlens, int32_t chunk_size,
                                              void *o, float *S_T, const gdn2_dims *dims,
                                              const gdn2_fusion *fusion, void *stream) {
    if (!dims) return gdn2::report(GDN2_ERR_NULL_ARG, "dims is NULL");
    // the size the regular call would need (0: invalid dims, which it reports itself)
    const size_t need = gdn2_chunk_fwd_workspace_bytes(dims, chunk_size);
    if (need > GDN2_STATIC_WORKSPACE_BYTES)
        return gdn2::report(GDN2_ERR_WORKSPACE,
                            "these dims need more workspace than the static array "
                            "(GDN2_STATIC_WORKSPACE_BYTES); use gdn2_chunk_fwd with a workspace");
    int dev = -1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return gdn2::report_hip(e, "gdn2_chunk_fwd_noalloc: device of the stream");
    if (dev < 0 || dev >= kMaxDevices)
        return gdn2::report(GDN2_ERR_UNSUPPORTED, "device index beyond the static array table");
    void *ws = nullptr;
    e = scratch_ptr(dev, &ws);
    if (e != hipSuccess) return gdn2::report_hip(e, "gdn2_chunk_fwd_noalloc: static workspace address");
    return gdn2_chunk_fwd(q, k, v, log_alpha, b, w, S0, cu_seqlens, chunk_size, o, S_T, dims, ws,
                          GDN2_STATIC_WORKSPACE_BYTES, fusion, stream);
}
