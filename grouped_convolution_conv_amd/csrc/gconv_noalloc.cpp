// gconv_noalloc.cpp -- the fused chain for callers that cannot allocate:
// its workspace is a static device array of the library instead of a
// caller-provided buffer.
//
// The chain's only scratch memory is the per-tile GroupNorm partials (and,
// for the recompute organisation, the merged (mean, rstd) per group).  Here
// it lives in `scratch`, a file-scope __device__ array: every GPU the
// library runs on holds its own copy of kScratchBytes from module load until
// the process ends.  The host never passes the array's name to a kernel (on
// the host that name is only a stand-in for the device symbol): its device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and that address is what the kernels receive.
//
// Nothing in the array has to start at zero: every partial slot and every
// merged statistic is written by the call before it is read.  Calls that
// overlap on one GPU (two streams, two host threads) share the array and
// race; the caller serializes them.
#include <atomic>
#include <mutex>

#include "internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB per device
constexpr int kMaxScratchDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void *> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch` in *out (looked
// up on the first call on that device); the HIP error of a failed lookup.
hipError_t scratch_for_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t conv_fused_gn_noalloc_limit(void) { return kScratchBytes; }

int conv_fused_gn_fwd_noalloc(gconv_desc_t d, const float *x, const float *w, const float *bias,
                              const float *scale, const float *gamma, const float *beta, int gn_groups, float eps,
                              float *y, void *stream) {
    if (!d) return GCONV_ERR_INVALID_ARG;
    size_t need = 0;
    const int rc = gconv::fused_workspace_bytes(d, gn_groups, &need);
    if (rc != GCONV_OK) return rc;
    if (need > kScratchBytes) return GCONV_ERR_SCRATCH_LIMIT;
    void *ws = nullptr;
    const int st = gconv::launch_status(scratch_for_current_device(&ws));
    if (st != GCONV_OK) return st;
    return gconv::fused_gn_run(d, x, w, bias, scale, gamma, beta, gn_groups, eps, y, ws, kScratchBytes, stream);
}

}  // extern "C"
