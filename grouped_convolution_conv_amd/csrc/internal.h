// internal.h -- shared host-side declarations of the gconv library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "gconv.h"

// Descriptor: geometry fixed at creation plus the derived quantities every
// launcher needs.
struct gconv_desc {
    int N, C, H, W, K, R, S;
    // per-axis geometry (h: along H and R, w: along W and S)
    int stride_h, stride_w, pad_h, pad_w, dil_h, dil_w;
    // the common value when both axes agree, else -1: the fast paths, which
    // take one value for both axes, test these and so refuse asymmetric
    // geometry (the direct kernel takes the per-axis fields)
    int stride, pad, dil;
    int groups;
    int Ho, Wo;
    int cin;   // input channels per group  (C / groups)
    int cout;  // output channels per group (K / groups)
    int algo;           // GCONV_ALGO_* requested by the caller (AUTO by default)
    int fused_variant;  // GCONV_FUSED_* requested by the caller (AUTO by default)
    int fused_wait_us;  // one-pass variant: bounded wait for an image's statistics, microseconds
};

namespace gconv {

// hipLaunchKernelGGL reports through the runtime's per-thread last error,
// which an unrelated earlier call (a stream or event query that found work
// pending, say) may have left set.  Launchers drop that stale value first so
// the error they return belongs to their own launch.
inline void clear_stale_launch_error() { (void)hipGetLastError(); }

// GCONV_OK for hipSuccess; otherwise records `e` for gconv_last_launch_error
// and returns GCONV_ERR_LAUNCH.
int launch_status(hipError_t e);

// Per-tile GroupNorm statistics written by a fused stage-A kernel and read by
// the normalize kernel: element count, mean and sum of squared deviations
// from that mean (the fourth slot is padding).
struct alignas(16) Partial {
    float count, mean, m2, pad;
};

// Epilogue parameters of the fused chain.
struct FusedEpilogue {
    const float *bias;   // [K]
    const float *scale;  // [K]
    Partial *parts;      // [N][gn_groups][parts_per_group]
    int gn_groups;
    int gn_cpg;          // channels per GroupNorm group (K / gn_groups)
    int parts_per_group;
};

// ---- applicability tests -------------------------------------------------
bool grouped3x3_supported(const gconv_desc *d);
bool igemm_supported(const gconv_desc *d);
bool depthwise_supported(const gconv_desc *d);
bool depthwise_small_3x3(const gconv_desc *d);            // small depthwise 3x3 planes (packed kernel)
bool depthwise_small_3x3_preferred(const gconv_desc *d);  // ... and enough of them to prefer it
bool igemm_fused_supported(const gconv_desc *d, int gn_groups);

// grouped 3x3 with 16 input and 16 output channels per group on the FP32
// matrix cores (taken inside launch_grouped3x3 when it applies)
bool grouped16_mfma_applies(const gconv_desc *d);
hipError_t launch_grouped16_mfma(const gconv_desc *d, const float *x, const float *w,
                                 const float *bias, float *y, hipStream_t st);

// ---- plain convolution launchers (y = conv(x, w) [+ bias]) ---------------
hipError_t launch_direct(const gconv_desc *d, const float *x, const float *w,
                         const float *bias, float *y, hipStream_t st);
hipError_t launch_grouped3x3(const gconv_desc *d, const float *x, const float *w,
                             const float *bias, float *y, hipStream_t st);
hipError_t launch_igemm(const gconv_desc *d, const float *x, const float *w,
                        const float *bias, float *y, hipStream_t st);
hipError_t launch_depthwise(const gconv_desc *d, const float *x, const float *w,
                            const float *bias, float *y, hipStream_t st);

// ---- fused chain, stage A: conv + bias/scale/sigmoid + per-tile stats ----
int direct_fused_parts_per_group(const gconv_desc *d, int gn_groups);
int igemm_fused_parts_per_group(const gconv_desc *d, int gn_groups);
hipError_t launch_direct_fused(const gconv_desc *d, const float *x, const float *w,
                               float *y, const FusedEpilogue &ep, hipStream_t st);
hipError_t launch_igemm_fused(const gconv_desc *d, const float *x, const float *w,
                              float *y, const FusedEpilogue &ep, hipStream_t st);

// ---- persistent MFMA kernel with LDS-resident weights (few input channels)
bool igemm_res_supported(const gconv_desc *d);
bool igemm_res_fused_supported(const gconv_desc *d, int gn_groups);
int igemm_res_parts_per_group(const gconv_desc *d);
hipError_t launch_igemm_res(const gconv_desc *d, const float *x, const float *w, const float *bias,
                            float *y, hipStream_t st);
// conv + bias/scale/sigmoid + per-tile statistics; stores v when `store`
hipError_t launch_igemm_res_stats(const gconv_desc *d, const float *x, const float *w, float *y,
                                  bool store, const FusedEpilogue &ep, hipStream_t st);
// merged (mean, rstd) per (n, group) from the partials
hipError_t launch_gn_merge(const gconv_desc *d, const Partial *parts, int gn_groups,
                           int parts_per_group, float eps, float2 *gstat, hipStream_t st);
// conv + bias/scale/sigmoid + normalization with merged statistics, stored to y
// The whole fused chain in one conv pass (variant GCONV_FUSED_ONEPASS): gstat
// [N][gn_groups] (mean, rstd) and sync [igemm_res_onepass_sync_ints] ints are
// workspace the call clears and fills itself.
bool igemm_res_onepass_supported(const gconv_desc *d, int gn_groups);
size_t igemm_res_onepass_sync_ints(const gconv_desc *d);
hipError_t launch_igemm_res_onepass(const gconv_desc *d, const float *x, const float *w, float *y,
                                    const FusedEpilogue &fe, float2 *gstat, int *sync, const float *gamma,
                                    const float *beta, float eps, int wait_us, hipStream_t st);
hipError_t launch_igemm_res_normalize(const gconv_desc *d, const float *x, const float *w, float *y,
                                      const FusedEpilogue &ep, const float2 *gstat,
                                      const float *gamma, const float *beta, hipStream_t st);

// ---- the fused chain as a whole (both compute entry points of the chain) -
// Device workspace bytes of the fused chain for gn_groups groups.
int fused_workspace_bytes(const gconv_desc *d, int gn_groups, size_t *bytes);
// Validates the arguments and enqueues the fused chain on `stream` with the
// given workspace; returns a GCONV_* status.
int fused_gn_run(const gconv_desc *d, const float *x, const float *w, const float *bias, const float *scale,
                 const float *gamma, const float *beta, int gn_groups, float eps, float *y, void *workspace,
                 size_t workspace_bytes, void *stream);

// ---- fused chain, stage B: merge statistics, normalize y in place -------
hipError_t launch_gn_normalize(const gconv_desc *d, float *y, const Partial *parts,
                               int gn_groups, int parts_per_group, const float *gamma,
                               const float *beta, float eps, hipStream_t st);

}  // namespace gconv
