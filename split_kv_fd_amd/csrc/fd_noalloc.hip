// fd_decode_noalloc: fd_decode for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Its workspace -- the split partials and the in-launch
// merge's arrival counters -- is a static device array of this library,
// FD_NOALLOC_SCRATCH_BYTES long, one copy per GPU, held until the process
// ends.  Nothing in it has to start at zero: the counters carry a per-call
// tag (a word with any other tag is recounted from zero) and every partial
// is written before it is read.  Calls on one GPU share the array, so calls
// that overlap in time on one GPU race.
#include <mutex>

#include "fd_kernels.h"

// The scratch itself.  In host code this name is only a handle for
// hipGetSymbolAddress: the kernels get the device address it returns.
static __device__ __align__(256) unsigned char scratch[FD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device
// (with that device current) and kept.
fd_status_t scratch_address(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fdk::hip_error(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fdk::error(FD_ERR_UNSUPPORTED, "device id beyond 63");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return fdk::hip_error(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fdk::error(FD_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return FD_OK;
}

}  // namespace

extern "C" fd_status_t fd_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                         const int32_t *page_table, const int32_t *seq_lens, float *out,
                                         float *lse, int B, int Hq, int Hkv, int T, int D, float scale,
                                         int n_splits, const fd_options_t *opt) {
    // every argument and the plan's scratch size first (host only), then the device
    fd_status_t st = fdk::scratch_plan(q, k_cache, v_cache, page_table, seq_lens, out, lse, B, Hq, Hkv, T, D, scale,
                                       n_splits, opt, FD_NOALLOC_SCRATCH_BYTES);
    if (st != FD_OK) return st;
    void *ptr = nullptr;
    st = scratch_address(&ptr);
    if (st != FD_OK) return st;
    return fdk::decode_with_scratch(q, k_cache, v_cache, page_table, seq_lens, out, lse, B, Hq, Hkv, T, D, scale,
                                    n_splits, opt, ptr, FD_NOALLOC_SCRATCH_BYTES);
}
