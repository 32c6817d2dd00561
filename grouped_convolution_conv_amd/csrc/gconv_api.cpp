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
    if (gconv::grouped3x3_supported(d)) return GCONV_ALGO_GROUPED3X3;
    if (gconv::igemm_supported(d)) return GCONV_ALGO_IGEMM;
    return GCONV_ALGO_DIRECT;
}

bool algo_supported(const gconv_desc *d, int algo) {
    switch (algo) {
        case GCONV_ALGO_AUTO:
        case GCONV_ALGO_DIRECT: return true;
        case GCONV_ALGO_GROUPED3X3: return gconv::grouped3x3_supported(d);
        case GCONV_ALGO_IGEMM: return gconv::igemm_supported(d);
        default: return false;
    }
}

// Stage-A flavour for the fused chain: the MFMA kernel when it covers the
// geometry and the GroupNorm grouping, otherwise the direct kernel.
bool fused_uses_igemm(const gconv_desc *d, int gn_groups) {
    return resolve_algo(d) == GCONV_ALGO_IGEMM && gconv::igemm_fused_supported(d, gn_groups);
}

int fused_parts_per_group(const gconv_desc *d, int gn_groups) {
    return fused_uses_igemm(d, gn_groups) ? gconv::igemm_fused_parts_per_group(d, gn_groups)
                                          : gconv::direct_fused_parts_per_group(d, gn_groups);
}

// HIP error behind the most recent GCONV_ERR_LAUNCH of the calling thread.
thread_local hipError_t g_last_hip_error = hipSuccess;

int launch_status(hipError_t e) {
    if (e == hipSuccess) return GCONV_OK;
    g_last_hip_error = e;
    return GCONV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int conv_desc_create(gconv_desc_t *out, int N, int C, int H, int W, int K, int R, int S,
                     int stride, int pad, int dilation, int groups) {
    if (!out) return GCONV_ERR_INVALID_ARG;
    *out = nullptr;
    if (N < 1 || C < 1 || H < 1 || W < 1 || K < 1 || R < 1 || S < 1) return GCONV_ERR_INVALID_ARG;
    if (stride < 1 || dilation < 1 || pad < 0 || groups < 1) return GCONV_ERR_INVALID_ARG;
    if (C % groups != 0 || K % groups != 0) return GCONV_ERR_INVALID_ARG;
    const int Ho = out_dim(H, R, stride, pad, dilation);
    const int Wo = out_dim(W, S, stride, pad, dilation);
    if (Ho < 1 || Wo < 1) return GCONV_ERR_INVALID_ARG;
    if (!fits_int32(N, C, H, W) || !fits_int32(N, K, Ho, Wo) || !fits_int32(K, C / groups, R, S))
        return GCONV_ERR_INVALID_ARG;
    // padded extents used by the tiled kernels must stay in int range too
    if ((long long)H + 2LL * pad > INT_MAX / 2 || (long long)W + 2LL * pad > INT_MAX / 2)
        return GCONV_ERR_INVALID_ARG;
    gconv_desc *d = new (std::nothrow) gconv_desc;
    if (!d) return GCONV_ERR_INVALID_ARG;
    d->N = N; d->C = C; d->H = H; d->W = W; d->K = K; d->R = R; d->S = S;
    d->stride = stride; d->pad = pad; d->dil = dilation; d->groups = groups;
    d->Ho = Ho; d->Wo = Wo; d->cin = C / groups; d->cout = K / groups;
    d->algo = GCONV_ALGO_AUTO;
    *out = d;
    return GCONV_OK;
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
    if (algo < GCONV_ALGO_AUTO || algo > GCONV_ALGO_IGEMM) return GCONV_ERR_INVALID_ARG;
    if (!algo_supported(d, algo)) return GCONV_ERR_UNSUPPORTED;
    d->algo = algo;
    return GCONV_OK;
}

int conv_desc_get_algo(gconv_desc_t d, int *algo) {
    if (!d || !algo) return GCONV_ERR_INVALID_ARG;
    *algo = resolve_algo(d);
    return GCONV_OK;
}

int conv_fwd(gconv_desc_t d, const float *x, const float *w, const float *bias, float *y,
             void *stream) {
    if (!d || !x || !w || !y) return GCONV_ERR_INVALID_ARG;
    if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y | (uintptr_t)bias) & 3u) return GCONV_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    switch (resolve_algo(d)) {
        case GCONV_ALGO_GROUPED3X3: return launch_status(gconv::launch_grouped3x3(d, x, w, bias, y, st));
        case GCONV_ALGO_IGEMM: return launch_status(gconv::launch_igemm(d, x, w, bias, y, st));
        default: return launch_status(gconv::launch_direct(d, x, w, bias, y, st));
    }
}

int conv_fused_gn_workspace_size(gconv_desc_t d, int gn_groups, size_t *bytes) {
    if (!d || !bytes) return GCONV_ERR_INVALID_ARG;
    if (gn_groups < 1 || d->K % gn_groups != 0) return GCONV_ERR_INVALID_ARG;
    *bytes = sizeof(gconv::Partial) * (size_t)d->N * (size_t)gn_groups *
             (size_t)fused_parts_per_group(d, gn_groups);
    return GCONV_OK;
}

int conv_fused_gn_fwd(gconv_desc_t d, const float *x, const float *w, const float *bias,
                      const float *scale, const float *gamma, const float *beta, int gn_groups,
                      float eps, float *y, void *workspace, size_t workspace_bytes, void *stream) {
    if (!d || !x || !w || !bias || !scale || !y) return GCONV_ERR_INVALID_ARG;
    if (gn_groups < 1 || d->K % gn_groups != 0 || !(eps > 0.0f)) return GCONV_ERR_INVALID_ARG;
    if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y | (uintptr_t)bias | (uintptr_t)scale |
         (uintptr_t)gamma | (uintptr_t)beta) & 3u)
        return GCONV_ERR_INVALID_ARG;
    size_t need = 0;
    conv_fused_gn_workspace_size(d, gn_groups, &need);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15u)) return GCONV_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    gconv::FusedEpilogue ep;
    ep.bias = bias;
    ep.scale = scale;
    ep.parts = (gconv::Partial *)workspace;
    ep.gn_groups = gn_groups;
    ep.gn_cpg = d->K / gn_groups;
    ep.parts_per_group = fused_parts_per_group(d, gn_groups);
    hipError_t e = fused_uses_igemm(d, gn_groups) ? gconv::launch_igemm_fused(d, x, w, y, ep, st)
                                                  : gconv::launch_direct_fused(d, x, w, y, ep, st);
    int rc = launch_status(e);
    if (rc != GCONV_OK) return rc;
    return launch_status(gconv::launch_gn_normalize(d, y, ep.parts, gn_groups, ep.parts_per_group,
                                                    gamma, beta, eps, st));
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
        default: return "unknown status";
    }
}

}  // extern "C"
