// gconv_timing.cpp -- graph-boundary timing helper of the C ABI.
//
// The GroupConv Atlas page ("Method" and "Results": device events around
// launches captured in a CUDA graph, 10 batches of 30 samples) times every
// kernel under two boundaries; this file is the graph one, in native code so
// that what lies between the two events is nothing but the captured kernels.
#include <hip/hip_runtime.h>

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
