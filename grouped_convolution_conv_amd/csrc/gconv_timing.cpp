// gconv_timing.cpp -- graph-boundary timing helper of the C ABI.
//
// The GroupConv Atlas page ("Method" and "Results": device events around
// launches captured in a CUDA graph, 10 batches of 30 samples) times every
// kernel under two boundaries; this file is the graph one, in native code so
// that what lies between the two events is nothing but the captured kernels.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "gconv.h"

namespace {

struct Call {
    gconv_desc_t desc;
    int fused;
    const float *const *xs;
    float *const *ys;
    int nsets;
    const float *w, *bias, *scale, *gamma, *beta;
    int gn_groups;
    float eps;
    void *ws;
    size_t ws_bytes;
    void *stream;

    int operator()(int i) const {
        const int s = i % nsets;
        if (fused)
            return conv_fused_gn_fwd(desc, xs[s], w, bias, scale, gamma, beta, gn_groups, eps, ys[s], ws, ws_bytes,
                                     stream);
        return conv_fwd(desc, xs[s], w, bias, ys[s], stream);
    }
};

// Destroys whatever was created, in reverse order, whatever the exit path.
struct GraphState {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    std::vector<hipEvent_t> events;
    ~GraphState() {
        for (hipEvent_t e : events) (void)hipEventDestroy(e);
        if (exec) (void)hipGraphExecDestroy(exec);
        if (graph) (void)hipGraphDestroy(graph);
    }
};

}  // namespace

extern "C" int gconv_time_graph(gconv_desc_t desc, int fused, const float *const *xs, float *const *ys, int nsets,
                                const float *w, const float *bias, const float *scale, const float *gamma,
                                const float *beta, int gn_groups, float eps, void *workspace,
                                size_t workspace_bytes, int launches, int replays, float *ms_per_launch,
                                void *stream) {
    if (!desc || !xs || !ys || nsets < 1 || launches < 1 || replays < 1 || !ms_per_launch || !stream)
        return GCONV_ERR_INVALID_ARG;
    if (fused != 0 && fused != 1) return GCONV_ERR_INVALID_ARG;
    for (int i = 0; i < nsets; ++i)
        if (!xs[i] || !ys[i]) return GCONV_ERR_INVALID_ARG;
    const Call call{desc, fused, xs, ys, nsets, w, bias, scale, gamma, beta, gn_groups, eps, workspace,
                    workspace_bytes, stream};
    hipStream_t st = static_cast<hipStream_t>(stream);

    // one eager call: argument validation and code-object loading happen
    // before the capture, so a bad argument never leaves a capture open
    int rc = call(0);
    if (rc != GCONV_OK) return rc;

    GraphState g;
    if (hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal) != hipSuccess) return GCONV_ERR_LAUNCH;
    for (int i = 0; i < launches && rc == GCONV_OK; ++i) rc = call(i);
    const hipError_t end = hipStreamEndCapture(st, &g.graph);
    if (rc != GCONV_OK) return rc;
    if (end != hipSuccess || !g.graph) return GCONV_ERR_LAUNCH;
    if (hipGraphInstantiate(&g.exec, g.graph, nullptr, nullptr, 0) != hipSuccess) return GCONV_ERR_LAUNCH;

    g.events.assign(2 * (size_t)replays, nullptr);
    for (hipEvent_t &e : g.events)
        if (hipEventCreate(&e) != hipSuccess) return GCONV_ERR_LAUNCH;
    for (int i = 0; i < 3; ++i)  // warm-up replays
        if (hipGraphLaunch(g.exec, st) != hipSuccess) return GCONV_ERR_LAUNCH;
    for (int r = 0; r < replays; ++r) {
        if (hipEventRecord(g.events[2 * r], st) != hipSuccess) return GCONV_ERR_LAUNCH;
        if (hipGraphLaunch(g.exec, st) != hipSuccess) return GCONV_ERR_LAUNCH;
        if (hipEventRecord(g.events[2 * r + 1], st) != hipSuccess) return GCONV_ERR_LAUNCH;
    }
    if (hipEventSynchronize(g.events.back()) != hipSuccess) return GCONV_ERR_LAUNCH;
    for (int r = 0; r < replays; ++r) {
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, g.events[2 * r], g.events[2 * r + 1]) != hipSuccess) return GCONV_ERR_LAUNCH;
        ms_per_launch[r] = ms / (float)launches;
    }
    return GCONV_OK;
}

// ---------------------------------------------------------------------------
// Measured compute peaks.  Fractions of the published peaks say how far a
// kernel is from the datasheet; fractions of what the chip sustains under
// load (clocks drop under a full MFMA load) say how far it is from what is
// reachable.  Two register-only probes, each one timed launch after one
// warm-up launch on every CU: chains of v_mfma_f32_32x32x2f32 (four
// independent accumulators per wave) and chains of non-packed FP32 FMAs
// (eight independent per lane).  No memory is touched but one store that
// only a value the arithmetic cannot produce would trigger, which keeps the
// loops from being optimized away.

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
constexpr int kProbeBlock = 256;
constexpr int kMfmaChains = 4;
constexpr int kFmaChains = 8;
constexpr float kNever = -3.0e38f;  // below anything the probes compute

__global__ __launch_bounds__(kProbeBlock) void mfma_peak_kernel(float *sink, int iters) {
    floatx16 acc[kMfmaChains];
    for (int i = 0; i < kMfmaChains; ++i)
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
    const float a = 1.0f + (float)threadIdx.x * 1e-7f, b = 0.5f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kMfmaChains; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[i], 0, 0, 0);
    }
    float s = 0.0f;
    for (int i = 0; i < kMfmaChains; ++i)
        for (int v = 0; v < 16; ++v) s += acc[i][v];
    if (s == kNever) sink[0] = s;
}

__global__ __launch_bounds__(kProbeBlock) void fma_peak_kernel(float *sink, int iters) {
    float v[kFmaChains];
    for (int i = 0; i < kFmaChains; ++i) v[i] = (float)threadIdx.x * 1e-3f + (float)i;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kFmaChains; ++i) v[i] = fmaf(v[i], 0.999f, 0.001f);
    }
    float s = 0.0f;
    for (int i = 0; i < kFmaChains; ++i) s += v[i];
    if (s == kNever) sink[0] = s;
}

// Vector-ALU peaks: kVecChains independent FMA chains per lane, eight
// workgroups (32 waves) per CU, in FP32 and in FP64.  The FP64 probe is the
// control: its datasheet peak (256 CUs x 4 SIMDs x 16 lanes x 2 flop x
// 2.4 GHz = 78.6 TFLOP/s) is what the same loop shape reaches when each lane
// retires one FMA per clock.
constexpr int kVecChains = 16;

template <typename T>
__global__ __launch_bounds__(kProbeBlock) void vec_fma_peak_kernel(float *sink, int iters) {
    T v[kVecChains];
    for (int i = 0; i < kVecChains; ++i) v[i] = (T)threadIdx.x * (T)1e-3 + (T)i;
    const T a = (T)0.999, b = (T)0.001;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kVecChains; ++i) v[i] = fma(v[i], a, b);
    }
    T s = 0;
    for (int i = 0; i < kVecChains; ++i) s += v[i];
    if (s == (T)kNever) sink[0] = (float)s;
}

// Streaming copy for the measured HBM rate: each lane moves kCopyUnroll
// 16-byte pieces per round (all loads issued before the stores), rounds
// grid-strided over the buffer.
constexpr int kCopyUnroll = 4;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeBlock) void copy_probe_kernel(f32x4 *__restrict__ dst,
                                                                 const f32x4 *__restrict__ src, size_t n4) {
    const size_t stride = (size_t)gridDim.x * kProbeBlock * kCopyUnroll;
    for (size_t base = (size_t)blockIdx.x * kProbeBlock * kCopyUnroll + threadIdx.x; base < n4; base += stride) {
        f32x4 v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const size_t i = base + (size_t)u * kProbeBlock;
            if (i < n4) v[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const size_t i = base + (size_t)u * kProbeBlock;
            if (i < n4) __builtin_nontemporal_store(v[u], dst + i);
        }
    }
}

struct EventPair {
    hipEvent_t a = nullptr, b = nullptr;
    ~EventPair() {
        if (a) (void)hipEventDestroy(a);
        if (b) (void)hipEventDestroy(b);
    }
};

// Milliseconds of one launch of `kern` (after one warm-up launch).
template <typename K>
int time_probe(K kern, int blocks, float *sink, int iters, hipStream_t st, float *ms) {
    EventPair ev;
    if (hipEventCreate(&ev.a) != hipSuccess || hipEventCreate(&ev.b) != hipSuccess) return GCONV_ERR_LAUNCH;
    (void)hipGetLastError();
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(kProbeBlock), 0, st, sink, iters);
    if (hipEventRecord(ev.a, st) != hipSuccess) return GCONV_ERR_LAUNCH;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(kProbeBlock), 0, st, sink, iters);
    if (hipEventRecord(ev.b, st) != hipSuccess) return GCONV_ERR_LAUNCH;
    if (hipGetLastError() != hipSuccess) return GCONV_ERR_LAUNCH;
    if (hipEventSynchronize(ev.b) != hipSuccess) return GCONV_ERR_LAUNCH;
    if (hipEventElapsedTime(ms, ev.a, ev.b) != hipSuccess || !(*ms > 0.0f)) return GCONV_ERR_LAUNCH;
    return GCONV_OK;
}

}  // namespace

extern "C" int gconv_probe_vector_peaks(float *fp32_tflops, float *fp64_tflops, float *sink, void *stream) {
    if (!fp32_tflops || !fp64_tflops || !sink) return GCONV_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return GCONV_ERR_LAUNCH;
    const int blocks = 8 * cus;  // eight workgroups (32 waves) per CU
    const int iters = 4096;      // a few ms per probe
    const double flops = (double)blocks * kProbeBlock * iters * kVecChains * 2.0;
    float ms = 0.0f;
    int rc = time_probe(vec_fma_peak_kernel<float>, blocks, sink, iters, st, &ms);
    if (rc != GCONV_OK) return rc;
    *fp32_tflops = (float)(flops / (ms * 1e-3) / 1e12);
    rc = time_probe(vec_fma_peak_kernel<double>, blocks, sink, iters, st, &ms);
    if (rc != GCONV_OK) return rc;
    *fp64_tflops = (float)(flops / (ms * 1e-3) / 1e12);
    return GCONV_OK;
}

extern "C" int gconv_probe_copy(float *gbs, float *dst, const float *src, size_t bytes, void *stream) {
    if (!gbs || !dst || !src || bytes < 16 || (bytes & 15u) || (((uintptr_t)dst | (uintptr_t)src) & 15u))
        return GCONV_ERR_INVALID_ARG;
    const uintptr_t d0 = (uintptr_t)dst, s0 = (uintptr_t)src;
    if (d0 < s0 + bytes && s0 < d0 + bytes) return GCONV_ERR_INVALID_ARG;  // overlapping buffers
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return GCONV_ERR_LAUNCH;
    const size_t n4 = bytes / 16;
    const size_t per_block = (size_t)kProbeBlock * kCopyUnroll;
    const size_t want = (n4 + per_block - 1) / per_block;
    // at most 16 workgroups per CU: enough loads in flight, few rounds per lane
    const int blocks = (int)(want < (size_t)16 * cus ? want : (size_t)16 * cus);
    EventPair ev;
    if (hipEventCreate(&ev.a) != hipSuccess || hipEventCreate(&ev.b) != hipSuccess) return GCONV_ERR_LAUNCH;
    (void)hipGetLastError();
    float best = 0.0f;
    for (int rep = 0; rep < 6; ++rep) {  // one warm-up, then the fastest of five
        if (hipEventRecord(ev.a, st) != hipSuccess) return GCONV_ERR_LAUNCH;
        hipLaunchKernelGGL(copy_probe_kernel, dim3(blocks), dim3(kProbeBlock), 0, st, (f32x4 *)dst,
                           (const f32x4 *)src, n4);
        if (hipEventRecord(ev.b, st) != hipSuccess) return GCONV_ERR_LAUNCH;
        if (hipGetLastError() != hipSuccess) return GCONV_ERR_LAUNCH;
        if (hipEventSynchronize(ev.b) != hipSuccess) return GCONV_ERR_LAUNCH;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, ev.a, ev.b) != hipSuccess || !(ms > 0.0f)) return GCONV_ERR_LAUNCH;
        const float rate = (float)(2.0 * (double)bytes / (ms * 1e-3) / 1e9);
        if (rep > 0 && rate > best) best = rate;
    }
    *gbs = best;
    return GCONV_OK;
}

extern "C" int gconv_probe_peaks(float *mfma_tflops, float *fma_tflops, float *sink, void *stream) {
    if (!mfma_tflops || !fma_tflops || !sink) return GCONV_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return GCONV_ERR_LAUNCH;
    const int blocks = 4 * cus;  // four workgroups (16 waves) per CU
    // about 2 ms per probe at the published peaks
    const int mfma_iters = 4096, fma_iters = 32768;
    float ms = 0.0f;
    int rc = time_probe(mfma_peak_kernel, blocks, sink, mfma_iters, st, &ms);
    if (rc != GCONV_OK) return rc;
    const double mfma_flops = (double)blocks * (kProbeBlock / 64) * mfma_iters * kMfmaChains * (32.0 * 32.0 * 2.0 * 2.0);
    *mfma_tflops = (float)(mfma_flops / (ms * 1e-3) / 1e12);
    rc = time_probe(fma_peak_kernel, blocks, sink, fma_iters, st, &ms);
    if (rc != GCONV_OK) return rc;
    const double fma_flops = (double)blocks * kProbeBlock * fma_iters * kFmaChains * 2.0;
    *fma_tflops = (float)(fma_flops / (ms * 1e-3) / 1e12);
    return GCONV_OK;
}
