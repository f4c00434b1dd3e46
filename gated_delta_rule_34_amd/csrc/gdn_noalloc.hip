// gdn_noalloc.hip -- gdn2_chunk_fwd without a caller-supplied workspace, for
// callers that cannot allocate device memory at all (code under stream
// capture, tight serving loops, harnesses that forbid allocation).
//
// The workspace lives in a file-scope device array of a fixed size.  In host
// code the array's name is only a stand-in: its device address is obtained
// once per device with hipGetSymbolAddress (with that device current) and
// that address is what the kernels receive.  Every call on one GPU shares
// that GPU's copy of the array, so calls that overlap on one GPU (several
// streams, several host threads) race and must be serialised by the caller.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/gdn.h"

namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[GDN2_NOALLOC_SCRATCH_BYTES];

// device address of `scratch` on device d, filled on the first call there
std::atomic<void *> g_scratch_ptr[kMaxDevices];

gdn_status scratch_on_current_device(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GDN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        // idempotent: concurrent first calls on one device store the same address
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN_ERR_HIP;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return GDN_OK;
}

}  // namespace

extern "C" {

size_t gdn2_chunk_fwd_noalloc_max_bytes(void) { return (size_t)GDN2_NOALLOC_SCRATCH_BYTES; }

gdn_status gdn2_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *log_alpha,
                                  const void *b, const void *w, const float *h0, float *o, float *ht, int B,
                                  int T, int H, int Dk, int Dv, gdn_dtype dtype, float scale, void *stream) {
    const size_t need = gdn2_chunk_fwd_workspace(B, T, H, Dk, Dv, dtype);
    if (need == 0) {
        // invalid sizes, head size or dtype: the same status the workspace form returns
        return gdn2_chunk_fwd(q, k, v, log_alpha, b, w, h0, o, ht, B, T, H, Dk, Dv, dtype, scale, nullptr, 0,
                              stream);
    }
    if (need > (size_t)GDN2_NOALLOC_SCRATCH_BYTES) return GDN_ERR_WORKSPACE;
    void *ws = nullptr;
    const gdn_status s = scratch_on_current_device(&ws);
    if (s != GDN_OK) return s;
    return gdn2_chunk_fwd(q, k, v, log_alpha, b, w, h0, o, ht, B, T, H, Dk, Dv, dtype, scale, ws,
                          (size_t)GDN2_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
