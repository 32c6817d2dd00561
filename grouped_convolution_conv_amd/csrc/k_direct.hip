// k_direct.hip -- direct convolution for any geometry: one output per lane.
//
// This is the always-available path (the "direct mapping" kernel of the
// GroupConv Atlas page, "CUDA / Mapping / Data reuse": recover the output
// coordinates from the thread index and support general geometry).  A
// workgroup covers 256 consecutive pixels of one (n, k) output plane, so
// the weight reads of a workgroup are uniform and go through the scalar
// cache.  The fused variant also applies the bias/scale/sigmoid epilogue and
// writes one GroupNorm partial (count, mean, M2) per workgroup.
#include "dev_common.h"
#include "internal.h"

namespace gconv {
namespace {

constexpr int kBlock = 256;

struct DirectGeom {
    int C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, cin, cout, Ho, Wo;
    int pblocks;  // 256-pixel blocks per output plane
};

// The grid is one-dimensional: block b covers pixel block b % pblocks of
// output plane (n, k) = (b / pblocks / K, b / pblocks % K).  N * K * pblocks
// stays below 2^31 for every descriptor (each block holds at least one of
// the fewer than 2^31 outputs), so any N and K fit.
struct BlockCoord {
    int n, k, pb;
};

__device__ __forceinline__ BlockCoord block_coord(const DirectGeom &g) {
    const int b = blockIdx.x;
    const int nk = b / g.pblocks;
    BlockCoord c;
    c.pb = b - nk * g.pblocks;
    c.n = nk / g.K;
    c.k = nk - c.n * g.K;
    return c;
}

__device__ __forceinline__ float direct_point(const float *__restrict__ x,
                                              const float *__restrict__ w, const DirectGeom &g,
                                              int n, int k, int oh, int ow) {
    const int grp = k / g.cout;
    const float *xb = x + ((size_t)n * g.C + (size_t)grp * g.cin) * g.H * g.W;
    const float *wk = w + (size_t)k * g.cin * g.R * g.S;
    const int ih0 = oh * g.sh - g.ph;
    const int iw0 = ow * g.sw - g.pw;
    float acc = 0.0f;
    for (int c = 0; c < g.cin; ++c) {
        const float *xc = xb + (size_t)c * g.H * g.W;
        const float *wc = wk + c * g.R * g.S;
        for (int r = 0; r < g.R; ++r) {
            const int ih = ih0 + r * g.dh;
            if (ih < 0 || ih >= g.H) continue;
            const float *xr = xc + (size_t)ih * g.W;
            const float *wr = wc + r * g.S;
            for (int s = 0; s < g.S; ++s) {
                const int iw = iw0 + s * g.dw;
                if (iw < 0 || iw >= g.W) continue;
                acc = fmaf(xr[iw], wr[s], acc);
            }
        }
    }
    return acc;
}

__global__ __launch_bounds__(kBlock) void direct_conv_kernel(const float *__restrict__ x,
                                                             const float *__restrict__ w,
                                                             const float *__restrict__ bias,
                                                             float *__restrict__ y, DirectGeom g) {
    const int plane = g.Ho * g.Wo;
    const BlockCoord bc = block_coord(g);
    const int p = bc.pb * kBlock + threadIdx.x;
    if (p >= plane) return;
    const int k = bc.k, n = bc.n;
    const int oh = p / g.Wo, ow = p - oh * g.Wo;
    float acc = direct_point(x, w, g, n, k, oh, ow);
    if (bias) acc += bias[k];
    y[((size_t)n * g.K + k) * plane + p] = acc;
}

__global__ __launch_bounds__(kBlock) void direct_fused_kernel(const float *__restrict__ x,
                                                              const float *__restrict__ w,
                                                              float *__restrict__ y, DirectGeom g,
                                                              FusedEpilogue ep) {
    __shared__ float scratch[4];
    const int plane = g.Ho * g.Wo;
    const BlockCoord bc = block_coord(g);
    const int p = bc.pb * kBlock + threadIdx.x;
    const int k = bc.k, n = bc.n;
    const bool valid = p < plane;
    float v = 0.0f;
    if (valid) {
        const int oh = p / g.Wo, ow = p - oh * g.Wo;
        const float acc = direct_point(x, w, g, n, k, oh, ow);
        v = sigmoidf((acc + ep.bias[k]) * ep.scale[k]);
        y[((size_t)n * g.K + k) * plane + p] = v;
    }
    // two-pass statistics of this block's values
    const int cnt = min(kBlock, plane - bc.pb * kBlock);
    const float mean = block256_sum(valid ? v : 0.0f, scratch) / (float)cnt;
    const float d = valid ? v - mean : 0.0f;
    const float m2 = block256_sum(d * d, scratch);
    if (threadIdx.x == 0) {
        const int gg = k / ep.gn_cpg, kl = k - gg * ep.gn_cpg;
        const size_t idx = ((size_t)n * ep.gn_groups + gg) * ep.parts_per_group +
                           (size_t)kl * g.pblocks + bc.pb;
        Partial pt;
        pt.count = (float)cnt;
        pt.mean = mean;
        pt.m2 = m2;
        pt.pad = 0.0f;
        ep.parts[idx] = pt;
    }
}

DirectGeom make_geom(const gconv_desc *d) {
    DirectGeom g;
    g.C = d->C; g.H = d->H; g.W = d->W; g.K = d->K; g.R = d->R; g.S = d->S;
    g.sh = d->stride_h; g.sw = d->stride_w; g.ph = d->pad_h; g.pw = d->pad_w; g.dh = d->dil_h; g.dw = d->dil_w;
    g.cin = d->cin; g.cout = d->cout; g.Ho = d->Ho; g.Wo = d->Wo;
    g.pblocks = (d->Ho * d->Wo + kBlock - 1) / kBlock;
    return g;
}

// N * K * pblocks blocks; below 2^31 for every valid descriptor (checked
// anyway: the caller gets hipErrorInvalidConfiguration, never a wrapped grid)
bool direct_blocks(const gconv_desc *d, unsigned *blocks) {
    const long long pb = ((long long)d->Ho * d->Wo + kBlock - 1) / kBlock;
    const long long b = (long long)d->N * d->K * pb;
    if (b > 0x7fffffffLL) return false;
    *blocks = (unsigned)b;
    return true;
}

}  // namespace

int direct_fused_parts_per_group(const gconv_desc *d, int gn_groups) {
    const int plane = d->Ho * d->Wo;
    return (d->K / gn_groups) * ((plane + kBlock - 1) / kBlock);
}

hipError_t launch_direct(const gconv_desc *d, const float *x, const float *w, const float *bias,
                         float *y, hipStream_t st) {
    unsigned blocks = 0;
    if (!direct_blocks(d, &blocks)) return hipErrorInvalidConfiguration;
    clear_stale_launch_error();
    hipLaunchKernelGGL(direct_conv_kernel, dim3(blocks), dim3(kBlock), 0, st, x, w, bias, y, make_geom(d));
    return hipGetLastError();
}

hipError_t launch_direct_fused(const gconv_desc *d, const float *x, const float *w, float *y,
                               const FusedEpilogue &ep, hipStream_t st) {
    unsigned blocks = 0;
    if (!direct_blocks(d, &blocks)) return hipErrorInvalidConfiguration;
    clear_stale_launch_error();
    hipLaunchKernelGGL(direct_fused_kernel, dim3(blocks), dim3(kBlock), 0, st, x, w, y, make_geom(d), ep);
    return hipGetLastError();
}

}  // namespace gconv
