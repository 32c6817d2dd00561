// gconv_api.cpp -- the C ABI: descriptor validation, dispatch and the two
// compute entry points.  No allocation, free, memset or synchronization
// happens inside conv_fwd / conv_fused_gn_fwd.
#include <climits>
#include <cstdint>
#include <new>

#include "internal.h"

namespace {

int out_dim(int in, int k, int stride, int pad, int dil) {
    const long long num = (long long)in + 2LL * pad - (long long)dil * (k - 1) - 1;
    if (num < 0) return 0;
    return (int)(num / stride) + 1;
}

bool fits_int32(long long a, long long b, long long c, long long d) {
    const long long lim = (long long)INT_MAX;
    long long p = a;
    for (long long f : {b, c, d}) {
        if (f > 0 && p > lim / f) return false;
        p *= f;
    }
    return p <= lim;
}

int resolve_algo(const gconv_desc *d) {
    if (d->algo != GCONV_ALGO_AUTO) return d->algo;
    if (gconv::depthwise_small_3x3_preferred(d)) return GCONV_ALGO_DEPTHWISE;
    if (gconv::grouped3x3_supported(d)) return GCONV_ALGO_GROUPED3X3;
    if (gconv::depthwise_supported(d)) return GCONV_ALGO_DEPTHWISE;
    if (gconv::igemm_supported(d)) return GCONV_ALGO_IGEMM;
    return GCONV_ALGO_DIRECT;
}

bool algo_supported(const gconv_desc *d, int algo) {
    switch (algo) {
        case GCONV_ALGO_AUTO:
        case GCONV_ALGO_DIRECT: return true;
        case GCONV_ALGO_GROUPED3X3: return gconv::grouped3x3_supported(d);
        case GCONV_ALGO_IGEMM: return gconv::igemm_supported(d);
        case GCONV_ALGO_DEPTHWISE: return gconv::depthwise_supported(d);
        default: return false;
    }
}

// Kernel that runs the conv of the fused chain: the persistent MFMA kernel
// with LDS-resident weights, the chunked MFMA kernel, or the direct kernel.
enum StageA { kStageDirect, kStageIgemm, kStageResident };

// The recompute variant measured fastest on MI355X for the shapes the
// resident kernel takes: it trades re-reading and re-writing v for a second
// MFMA pass, where the store and one-pass variants move v through memory
// (measured at the fused 8 -> 32 chain on 64 images of 256 x 256: recompute
// 450-472 us, one-pass 493-514 us, store over batch slices 454-464 us).
constexpr int kDefaultResidentVariant = GCONV_FUSED_RECOMPUTE;
constexpr int kDefaultWaitUs = 200;
constexpr int kMaxWaitUs = 10000000;

// Bytes of v per slice of the store variant (the Infinity Cache holds 256 MB;
// measured at the fused 8 -> 32 chain: 32 MB 667 us, 64 MB 519 us, 128 MB
// 464 us, one slice 527 us).
constexpr size_t kStoreSliceBytes = size_t(128) << 20;

StageA fused_stage_a(const gconv_desc *d, int gn_groups) {
    if (resolve_algo(d) == GCONV_ALGO_IGEMM) {
        if (gconv::igemm_res_fused_supported(d, gn_groups)) return kStageResident;
        if (gconv::igemm_fused_supported(d, gn_groups)) return kStageIgemm;
    }
    return kStageDirect;
}

int resolve_fused_variant(const gconv_desc *d, int gn_groups) {
    if (d->fused_variant != GCONV_FUSED_AUTO) return d->fused_variant;
    return fused_stage_a(d, gn_groups) == kStageResident ? kDefaultResidentVariant : GCONV_FUSED_STORE;
}

size_t align16(size_t b) { return (b + 15) & ~(size_t)15; }

int fused_parts_per_group(const gconv_desc *d, int gn_groups) {
    switch (fused_stage_a(d, gn_groups)) {
        case kStageResident: return gconv::igemm_res_parts_per_group(d);
        case kStageIgemm: return gconv::igemm_fused_parts_per_group(d, gn_groups);
        default: return gconv::direct_fused_parts_per_group(d, gn_groups);
    }
}

size_t partials_bytes(const gconv_desc *d, int gn_groups) {
    return sizeof(gconv::Partial) * (size_t)d->N * (size_t)gn_groups * (size_t)fused_parts_per_group(d, gn_groups);
}

// HIP error behind the most recent GCONV_ERR_LAUNCH of the calling thread.
thread_local hipError_t g_last_hip_error = hipSuccess;

}  // namespace

namespace gconv {

int launch_status(hipError_t e) {
    if (e == hipSuccess) return GCONV_OK;
    g_last_hip_error = e;
    return GCONV_ERR_LAUNCH;
}

}  // namespace gconv

namespace {
using gconv::launch_status;
}  // namespace

namespace gconv {

int fused_workspace_bytes(const gconv_desc *d, int gn_groups, size_t *bytes) {
    if (!d || !bytes) return GCONV_ERR_INVALID_ARG;
    if (gn_groups < 1 || d->K % gn_groups != 0) return GCONV_ERR_INVALID_ARG;
    size_t b = partials_bytes(d, gn_groups);
    const int variant = resolve_fused_variant(d, gn_groups);
    if (variant == GCONV_FUSED_RECOMPUTE || variant == GCONV_FUSED_ONEPASS)
        b += align16(sizeof(float2) * (size_t)d->N * (size_t)gn_groups);
    if (variant == GCONV_FUSED_ONEPASS && fused_stage_a(d, gn_groups) == kStageResident &&
        gconv::igemm_res_onepass_supported(d, gn_groups))
        b += align16(sizeof(int) * gconv::igemm_res_onepass_sync_ints(d));
    *bytes = b;
    return GCONV_OK;
}

int fused_gn_run(const gconv_desc *d, const float *x, const float *w, const float *bias,
                 const float *scale, const float *gamma, const float *beta, int gn_groups, float eps, float *y,
                 void *workspace, size_t workspace_bytes, void *stream) {
    if (!d || !x || !w || !bias || !scale || !y) return GCONV_ERR_INVALID_ARG;
    if (gn_groups < 1 || d->K % gn_groups != 0 || !(eps > 0.0f)) return GCONV_ERR_INVALID_ARG;
    if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y | (uintptr_t)bias | (uintptr_t)scale |
         (uintptr_t)gamma | (uintptr_t)beta) & 3u)
        return GCONV_ERR_INVALID_ARG;
    size_t need = 0;
    fused_workspace_bytes(d, gn_groups, &need);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15u)) return GCONV_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const StageA stage = fused_stage_a(d, gn_groups);
    const int variant = resolve_fused_variant(d, gn_groups);
    if (variant == GCONV_FUSED_RECOMPUTE && stage != kStageResident) return GCONV_ERR_UNSUPPORTED;
    if (variant == GCONV_FUSED_ONEPASS && (stage != kStageResident || !gconv::igemm_res_onepass_supported(d, gn_groups)))
        return GCONV_ERR_UNSUPPORTED;
    gconv::FusedEpilogue ep;
    ep.bias = bias;
    ep.scale = scale;
    ep.parts = (gconv::Partial *)workspace;
    ep.gn_groups = gn_groups;
    ep.gn_cpg = d->K / gn_groups;
    ep.parts_per_group = fused_parts_per_group(d, gn_groups);
    int rc;
    if (variant == GCONV_FUSED_ONEPASS) {
        char *base = (char *)workspace + partials_bytes(d, gn_groups);
        float2 *gstat = (float2 *)base;
        int *sync = (int *)(base + align16(sizeof(float2) * (size_t)d->N * (size_t)gn_groups));
        return launch_status(gconv::launch_igemm_res_onepass(d, x, w, y, ep, gstat, sync, gamma, beta, eps,
                                                             d->fused_wait_us, st));
    }
    if (variant == GCONV_FUSED_RECOMPUTE) {
        float2 *gstat = (float2 *)((char *)workspace + partials_bytes(d, gn_groups));
        rc = launch_status(gconv::launch_igemm_res_stats(d, x, w, nullptr, false, ep, st));
        if (rc != GCONV_OK) return rc;
        rc = launch_status(gconv::launch_gn_merge(d, ep.parts, gn_groups, ep.parts_per_group, eps, gstat, st));
        if (rc != GCONV_OK) return rc;
        return launch_status(gconv::launch_igemm_res_normalize(d, x, w, y, ep, gstat, gamma, beta, st));
    }
    // The store variant writes v and then normalizes it in place.  It runs
    // over slices of the batch whose v fits the GPU's last-level (Infinity)
    // cache with room to spare, so the normalize pass finds v there and HBM
    // sees x read once and the output written once.  A GroupNorm group never
    // spans two images, so slicing the batch changes no arithmetic.
    const size_t x_img = (size_t)d->C * d->H * d->W;
    const size_t y_img = (size_t)d->K * d->Ho * d->Wo;
    long long per = (long long)(kStoreSliceBytes / (y_img * sizeof(float)));
    if (per < 1) per = 1;
    const int slice = per < d->N ? (int)per : d->N;
    for (int n0 = 0; n0 < d->N; n0 += slice) {
        gconv_desc ds = *d;
        ds.N = d->N - n0 < slice ? d->N - n0 : slice;
        const float *xs = x + (size_t)n0 * x_img;
        float *ys = y + (size_t)n0 * y_img;
        gconv::FusedEpilogue es = ep;
        es.parts = ep.parts + (size_t)n0 * gn_groups * ep.parts_per_group;
        hipError_t e;
        switch (stage) {
            case kStageResident: e = gconv::launch_igemm_res_stats(&ds, xs, w, ys, true, es, st); break;
            case kStageIgemm: e = gconv::launch_igemm_fused(&ds, xs, w, ys, es, st); break;
            default: e = gconv::launch_direct_fused(&ds, xs, w, ys, es, st); break;
        }
        rc = launch_status(e);
        if (rc != GCONV_OK) return rc;
        rc = launch_status(gconv::launch_gn_normalize(&ds, ys, es.parts, gn_groups, es.parts_per_group, gamma,
                                                      beta, eps, st));
        if (rc != GCONV_OK) return rc;
    }
    return GCONV_OK;
}

}  // namespace gconv

extern "C" {

int conv_desc_create_2d(gconv_desc_t *out, int N, int C, int H, int W, int K, int R, int S, int stride_h,
                        int stride_w, int pad_h, int pad_w, int dil_h, int dil_w, int groups) {
    if (!out) return GCONV_ERR_INVALID_ARG;
    *out = nullptr;
    if (N < 1 || C < 1 || H < 1 || W < 1 || K < 1 || R < 1 || S < 1) return GCONV_ERR_INVALID_ARG;
    if (stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1 || pad_h < 0 || pad_w < 0 || groups < 1)
        return GCONV_ERR_INVALID_ARG;
    if (C % groups != 0 || K % groups != 0) return GCONV_ERR_INVALID_ARG;
    const int Ho = out_dim(H, R, stride_h, pad_h, dil_h);
    const int Wo = out_dim(W, S, stride_w, pad_w, dil_w);
    if (Ho < 1 || Wo < 1) return GCONV_ERR_INVALID_ARG;
    if (!fits_int32(N, C, H, W) || !fits_int32(N, K, Ho, Wo) || !fits_int32(K, C / groups, R, S))
        return GCONV_ERR_INVALID_ARG;
    // padded extents used by the tiled kernels must stay in int range too
    if ((long long)H + 2LL * pad_h > INT_MAX / 2 || (long long)W + 2LL * pad_w > INT_MAX / 2)
        return GCONV_ERR_INVALID_ARG;
    gconv_desc *d = new (std::nothrow) gconv_desc;
    if (!d) return GCONV_ERR_INVALID_ARG;
    d->N = N; d->C = C; d->H = H; d->W = W; d->K = K; d->R = R; d->S = S;
    d->stride_h = stride_h; d->stride_w = stride_w;
    d->pad_h = pad_h; d->pad_w = pad_w;
    d->dil_h = dil_h; d->dil_w = dil_w;
    d->stride = stride_h == stride_w ? stride_h : -1;
    d->pad = pad_h == pad_w ? pad_h : -1;
    d->dil = dil_h == dil_w ? dil_h : -1;
    d->groups = groups;
    d->Ho = Ho; d->Wo = Wo; d->cin = C / groups; d->cout = K / groups;
    d->algo = GCONV_ALGO_AUTO;
    d->fused_variant = GCONV_FUSED_AUTO;
    d->fused_wait_us = kDefaultWaitUs;
    *out = d;
    return GCONV_OK;
}

int conv_desc_create(gconv_desc_t *out, int N, int C, int H, int W, int K, int R, int S,
                     int stride, int pad, int dilation, int groups) {
    return conv_desc_create_2d(out, N, C, H, W, K, R, S, stride, stride, pad, pad, dilation, dilation, groups);
}

int conv_desc_destroy(gconv_desc_t desc) {
    delete desc;
    return GCONV_OK;
}

int conv_desc_get_output_dims(gconv_desc_t d, int *Ho, int *Wo) {
    if (!d || !Ho || !Wo) return GCONV_ERR_INVALID_ARG;
    *Ho = d->Ho;
    *Wo = d->Wo;
    return GCONV_OK;
}

int conv_desc_set_algo(gconv_desc_t d, int algo) {
    if (!d) return GCONV_ERR_INVALID_ARG;
    if (algo < GCONV_ALGO_AUTO || algo > GCONV_ALGO_DEPTHWISE) return GCONV_ERR_INVALID_ARG;
    if (!algo_supported(d, algo)) return GCONV_ERR_UNSUPPORTED;
    d->algo = algo;
    return GCONV_OK;
}

int conv_desc_get_algo(gconv_desc_t d, int *algo) {
    if (!d || !algo) return GCONV_ERR_INVALID_ARG;
    *algo = resolve_algo(d);
    return GCONV_OK;
}

int conv_desc_set_fused_variant(gconv_desc_t d, int variant) {
    if (!d) return GCONV_ERR_INVALID_ARG;
    if (variant < GCONV_FUSED_AUTO || variant > GCONV_FUSED_ONEPASS) return GCONV_ERR_INVALID_ARG;
    d->fused_variant = variant;
    return GCONV_OK;
}

int conv_desc_set_fused_wait(gconv_desc_t d, int wait_us) {
    if (!d || wait_us < -1 || wait_us > kMaxWaitUs) return GCONV_ERR_INVALID_ARG;
    d->fused_wait_us = wait_us;
    return GCONV_OK;
}

int conv_desc_get_fused_variant(gconv_desc_t d, int gn_groups, int *variant) {
    if (!d || !variant) return GCONV_ERR_INVALID_ARG;
    if (gn_groups < 1 || d->K % gn_groups != 0) return GCONV_ERR_INVALID_ARG;
    *variant = resolve_fused_variant(d, gn_groups);
    return GCONV_OK;
}

int conv_fwd(gconv_desc_t d, const float *x, const float *w, const float *bias, float *y,
             void *stream) {
    if (!d || !x || !w || !y) return GCONV_ERR_INVALID_ARG;
    if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y | (uintptr_t)bias) & 3u) return GCONV_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    switch (resolve_algo(d)) {
        case GCONV_ALGO_GROUPED3X3: return launch_status(gconv::launch_grouped3x3(d, x, w, bias, y, st));
        case GCONV_ALGO_DEPTHWISE: return launch_status(gconv::launch_depthwise(d, x, w, bias, y, st));
        case GCONV_ALGO_IGEMM:
            if (gconv::igemm_res_supported(d)) return launch_status(gconv::launch_igemm_res(d, x, w, bias, y, st));
            return launch_status(gconv::launch_igemm(d, x, w, bias, y, st));
        default: return launch_status(gconv::launch_direct(d, x, w, bias, y, st));
    }
}

int conv_fused_gn_workspace_size(gconv_desc_t d, int gn_groups, size_t *bytes) {
    return gconv::fused_workspace_bytes(d, gn_groups, bytes);
}

int conv_fused_gn_fwd(gconv_desc_t d, const float *x, const float *w, const float *bias,
                      const float *scale, const float *gamma, const float *beta, int gn_groups,
                      float eps, float *y, void *workspace, size_t workspace_bytes, void *stream) {
    return gconv::fused_gn_run(d, x, w, bias, scale, gamma, beta, gn_groups, eps, y, workspace, workspace_bytes,
                               stream);
}

const char *gconv_last_launch_error(void) {
    return g_last_hip_error == hipSuccess ? "none" : hipGetErrorString(g_last_hip_error);
}

const char *gconv_status_string(int status) {
    switch (status) {
        case GCONV_OK: return "ok";
        case GCONV_ERR_INVALID_ARG: return "invalid argument";
        case GCONV_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case GCONV_ERR_UNSUPPORTED: return "algorithm does not support this geometry";
        case GCONV_ERR_LAUNCH: return "kernel launch failed";
        case GCONV_ERR_SCRATCH_LIMIT:
            return "problem needs more scratch than the allocation-free entry point's static buffer holds";
        default: return "unknown status";
    }
}

}  // extern "C"
