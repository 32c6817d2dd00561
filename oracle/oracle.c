/*
 * oracle.c -- plain CPU oracle for FP32 NCHW 2-D convolution and for the
 * conv -> +bias -> *scale -> sigmoid -> GroupNorm chain.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke entry and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant with the HIP
 * path.
 *
 * Everything is the written-out definition, accumulated in double precision
 * from the FP32 inputs promoted to double.  There is no tiling, no fusion
 * and no reordering beyond the loop nest that the definition states; the
 * only concession to speed is an OpenMP "parallel for" over independent
 * (n, k) output planes, which does not change any sum.
 *
 * Sources (the pages):
 *  - POPCORNBENCH trace "Kimi-K2.6 l2_p21" (fused conv + bias + scale +
 *    sigmoid + GroupNorm): the direct-convolution sum over input channels and
 *    the 3x3 window (design discussion of the tiled direct conv), zero
 *    padding at the borders (tile loader of the fused conv kernel), the
 *    module order conv -> +bias -> *scale -> sigmoid -> GroupNorm (parameter
 *    discussion), sigmoid = 1/(1+exp(-t)), GroupNorm over contiguous channel
 *    groups with the population variance and eps inside the square root.
 *  - POPCORNBENCH trace "Kimi-K2.6 l1_p62" (dense 5x9 conv): weight layout
 *    [K][C/groups][KH][KW], output size (H + 2p - d(KH-1) - 1)/s + 1, and
 *    the input coordinate out*stride - pad + tap*dilation.
 *  - GroupConv Atlas project page, "Source / Method / Records": complete
 *    output checks with separate FP64 reference points.
 *
 * Readings where the pages are silent: output channel k belongs to group
 * k / (K/groups) and reads input channels [g*C/groups, (g+1)*C/groups)
 * (contiguous groups); the conv carries no bias of its own in the fused
 * chain, a single per-channel bias is added after it; gamma == NULL means
 * 1 and beta == NULL means 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD 1
#define ORACLE_NOMEM 2

/* Output extent along one axis: floor((in + 2p - d(k-1) - 1)/s) + 1, or 0
 * when the dilated window does not fit (dense 5x9 trace, output-size
 * formula). */
int oracle_out_dim(int in, int k, int stride, int pad, int dil)
{
    long long num = (long long)in + 2LL * pad - (long long)dil * (k - 1) - 1;
    if (num < 0 || stride < 1) return 0;
    return (int)(num / stride) + 1;
}

static int geometry_ok(int N, int C, int H, int W, int K, int R, int S,
                       int sh, int sw, int ph, int pw, int dh, int dw, int groups)
{
    if (N < 1 || C < 1 || H < 1 || W < 1 || K < 1 || R < 1 || S < 1) return 0;
    if (sh < 1 || sw < 1 || dh < 1 || dw < 1 || ph < 0 || pw < 0 || groups < 1) return 0;
    if (C % groups != 0 || K % groups != 0) return 0;
    if (oracle_out_dim(H, R, sh, ph, dh) < 1) return 0;
    if (oracle_out_dim(W, S, sw, pw, dw) < 1) return 0;
    return 1;
}

/* One output element of the convolution, y[n,k,oh,ow], and its bound
 * A = sum |x * w| over the same receptive field (plus |bias[k]|). */
static void conv_one(int C, int H, int W, int K, int R, int S,
                     int sh, int sw, int ph, int pw, int dh, int dw, int groups,
                     const float *x, const float *w, const float *bias,
                     int n, int k, int oh, int ow, double *yv, double *av)
{
    const int cin = C / groups;          /* input channels per group  */
    const int cout = K / groups;         /* output channels per group */
    const int g = k / cout;              /* group of output channel k */
    double acc = 0.0, ab = 0.0;
    for (int c = 0; c < cin; ++c) {
        const int ic = g * cin + c;
        for (int r = 0; r < R; ++r) {
            const int ih = oh * sh - ph + r * dh;
            if (ih < 0 || ih >= H) continue;            /* zero padding */
            for (int s = 0; s < S; ++s) {
                const int iw = ow * sw - pw + s * dw;
                if (iw < 0 || iw >= W) continue;        /* zero padding */
                const double xv =
                    (double)x[(((int64_t)n * C + ic) * H + ih) * W + iw];
                const double wv =
                    (double)w[(((int64_t)k * cin + c) * R + r) * S + s];
                acc += xv * wv;
                ab += fabs(xv * wv);
            }
        }
    }
    if (bias) {
        acc += (double)bias[k];
        ab += fabs((double)bias[k]);
    }
    *yv = acc;
    if (av) *av = ab;
}

/* Full convolution: y[N][K][Ho][Wo] (double), optional bound absb of the
 * same shape.  bias may be NULL.  Stride, padding and dilation are given
 * per axis (h: along H and R, w: along W and S). */
int oracle_conv2d_2d(int N, int C, int H, int W, int K, int R, int S,
                     int sh, int sw, int ph, int pw, int dh, int dw, int groups,
                     const float *x, const float *w, const float *bias,
                     double *y, double *absb, int nthreads)
{
    if (!geometry_ok(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, groups)) return ORACLE_BAD;
    if (!x || !w || !y) return ORACLE_BAD;
    const int Ho = oracle_out_dim(H, R, sh, ph, dh);
    const int Wo = oracle_out_dim(W, S, sw, pw, dw);
    if (nthreads < 1) nthreads = 1;
    const int64_t planes = (int64_t)N * K;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t p = 0; p < planes; ++p) {
        const int n = (int)(p / K), k = (int)(p % K);
        for (int oh = 0; oh < Ho; ++oh)
            for (int ow = 0; ow < Wo; ++ow) {
                const int64_t o = ((p * Ho) + oh) * Wo + ow;
                conv_one(C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, groups, x, w, bias,
                         n, k, oh, ow, &y[o], absb ? &absb[o] : NULL);
            }
    }
    return ORACLE_OK;
}

/* The same with one stride, padding and dilation for both axes. */
int oracle_conv2d(int N, int C, int H, int W, int K, int R, int S,
                  int stride, int pad, int dil, int groups,
                  const float *x, const float *w, const float *bias,
                  double *y, double *absb, int nthreads)
{
    return oracle_conv2d_2d(N, C, H, W, K, R, S, stride, stride, pad, pad, dil, dil, groups,
                            x, w, bias, y, absb, nthreads);
}

/* The same definition evaluated only at the given flat NCHW output indices
 * (for sampled checks of outputs too large to compute whole). */
int oracle_conv2d_points_2d(int N, int C, int H, int W, int K, int R, int S,
                            int sh, int sw, int ph, int pw, int dh, int dw, int groups,
                            const float *x, const float *w, const float *bias,
                            int64_t npts, const int64_t *idx,
                            double *y, double *absb, int nthreads)
{
    if (!geometry_ok(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, groups)) return ORACLE_BAD;
    if (!x || !w || !y || (npts > 0 && !idx)) return ORACLE_BAD;
    const int Ho = oracle_out_dim(H, R, sh, ph, dh);
    const int Wo = oracle_out_dim(W, S, sw, pw, dw);
    const int64_t total = (int64_t)N * K * Ho * Wo;
    for (int64_t i = 0; i < npts; ++i)
        if (idx[i] < 0 || idx[i] >= total) return ORACLE_BAD;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t i = 0; i < npts; ++i) {
        int64_t t = idx[i];
        const int ow = (int)(t % Wo); t /= Wo;
        const int oh = (int)(t % Ho); t /= Ho;
        const int k = (int)(t % K);
        const int n = (int)(t / K);
        conv_one(C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, groups, x, w, bias,
                 n, k, oh, ow, &y[i], absb ? &absb[i] : NULL);
    }
    return ORACLE_OK;
}

int oracle_conv2d_points(int N, int C, int H, int W, int K, int R, int S,
                         int stride, int pad, int dil, int groups,
                         const float *x, const float *w, const float *bias,
                         int64_t npts, const int64_t *idx,
                         double *y, double *absb, int nthreads)
{
    return oracle_conv2d_points_2d(N, C, H, W, K, R, S, stride, stride, pad, pad, dil, dil, groups,
                                   x, w, bias, npts, idx, y, absb, nthreads);
}

/* Fused chain of the l2_p21 trace, per sample n:
 *   t = (conv(x, w)[n,k,.,.] + bias[k]) * scale[k]
 *   v = 1 / (1 + exp(-t))
 *   for each GroupNorm group gg (channels [gg*K/G, (gg+1)*K/G)) of sample n:
 *       mu  = mean(v)                       (first pass)
 *       var = mean((v - mu)^2)              (second pass, population)
 *       out = (v - mu) / sqrt(var + eps) * gamma[k] + beta[k]
 * v_out (may be NULL) receives v; out receives the normalized result. */
int oracle_fused_gn_2d(int N, int C, int H, int W, int K, int R, int S,
                       int sh, int sw, int ph, int pw, int dh, int dw, int groups,
                       const float *x, const float *w, const float *bias,
                       const float *scale, const float *gamma, const float *beta,
                       int gn_groups, double eps,
                       double *v_out, double *out, int nthreads)
{
    if (!geometry_ok(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, groups)) return ORACLE_BAD;
    if (!x || !w || !bias || !scale || !out) return ORACLE_BAD;
    if (gn_groups < 1 || K % gn_groups != 0 || !(eps > 0.0)) return ORACLE_BAD;
    const int Ho = oracle_out_dim(H, R, sh, ph, dh);
    const int Wo = oracle_out_dim(W, S, sw, pw, dw);
    const int64_t plane = (int64_t)Ho * Wo;
    const int cpg = K / gn_groups;
    if (nthreads < 1) nthreads = 1;

    double *v = (double *)malloc(sizeof(double) * (size_t)K * (size_t)plane);
    if (!v) return ORACLE_NOMEM;

    for (int n = 0; n < N; ++n) {
        /* conv, then the elementwise epilogue in module order */
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
        for (int k = 0; k < K; ++k)
            for (int oh = 0; oh < Ho; ++oh)
                for (int ow = 0; ow < Wo; ++ow) {
                    double yv;
                    conv_one(C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, groups, x, w,
                             NULL, n, k, oh, ow, &yv, NULL);
                    const double t = (yv + (double)bias[k]) * (double)scale[k];
                    v[(int64_t)k * plane + (int64_t)oh * Wo + ow] = 1.0 / (1.0 + exp(-t));
                }
        if (v_out)
            memcpy(v_out + (int64_t)n * K * plane, v, sizeof(double) * (size_t)K * (size_t)plane);

        /* GroupNorm, two passes per group */
#pragma omp parallel for schedule(static) num_threads(nthreads)
        for (int gg = 0; gg < gn_groups; ++gg) {
            const double *vg = v + (int64_t)gg * cpg * plane;
            const int64_t m = (int64_t)cpg * plane;
            double sum = 0.0;
            for (int64_t i = 0; i < m; ++i) sum += vg[i];
            const double mu = sum / (double)m;
            double sq = 0.0;
            for (int64_t i = 0; i < m; ++i) sq += (vg[i] - mu) * (vg[i] - mu);
            const double var = sq / (double)m;
            const double inv = 1.0 / sqrt(var + eps);
            for (int cl = 0; cl < cpg; ++cl) {
                const int k = gg * cpg + cl;
                const double ga = gamma ? (double)gamma[k] : 1.0;
                const double be = beta ? (double)beta[k] : 0.0;
                double *o = out + ((int64_t)n * K + k) * plane;
                const double *vk = vg + (int64_t)cl * plane;
                for (int64_t i = 0; i < plane; ++i) o[i] = (vk[i] - mu) * inv * ga + be;
            }
        }
    }
    free(v);
    return ORACLE_OK;
}

int oracle_fused_gn(int N, int C, int H, int W, int K, int R, int S,
                    int stride, int pad, int dil, int groups,
                    const float *x, const float *w, const float *bias,
                    const float *scale, const float *gamma, const float *beta,
                    int gn_groups, double eps,
                    double *v_out, double *out, int nthreads)
{
    return oracle_fused_gn_2d(N, C, H, W, K, R, S, stride, stride, pad, pad, dil, dil, groups,
                              x, w, bias, scale, gamma, beta, gn_groups, eps, v_out, out, nthreads);
}
