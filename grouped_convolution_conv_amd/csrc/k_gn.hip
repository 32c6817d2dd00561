// k_gn.hip -- GroupNorm stage B: merge the per-tile statistics of each
// (sample, group) and normalize y in place.
//
// GroupNorm as in the POPCORNBENCH trace "Kimi-K2.6 l2_p21" (group_norm
// kernel and the parameter discussion): contiguous channel groups, the
// population variance, eps inside the square root, then the per-channel
// affine gamma, beta.  Instead of that trace's single-pass sum of squares,
// the statistics arrive as per-tile (count, mean, M2) triples computed in
// two passes by the conv kernel; here they are combined with the pairwise
// update of Chan, Golub and LeVeque in double precision, in a fixed order,
// so the result is bitwise repeatable.
#include "dev_common.h"
#include "internal.h"

namespace gconv {
namespace {

constexpr int kBlock = 256;
constexpr int kUnroll = 4;

struct Moments {
    double n, mean, m2;
};

__device__ __forceinline__ Moments merge(Moments a, Moments b) {
    if (b.n == 0.0) return a;
    if (a.n == 0.0) return b;
    Moments r;
    r.n = a.n + b.n;
    const double delta = b.mean - a.mean;
    r.mean = a.mean + delta * (b.n / r.n);
    r.m2 = a.m2 + b.m2 + delta * delta * (a.n * b.n / r.n);
    return r;
}

// one-dimensional grid: block b = (n * G + gg) * (cpg * nsplit) + channel-in-group * nsplit + split
__global__ __launch_bounds__(kBlock) void gn_normalize_kernel(float *__restrict__ y,
                                                              const Partial *__restrict__ parts,
                                                              int P, const float *__restrict__ gamma,
                                                              const float *__restrict__ beta, int K,
                                                              int G, int cpg, int plane, int nsplit,
                                                              float eps, int vec4) {
    __shared__ double sn[kBlock], smean[kBlock], sm2[kBlock];
    const int per_group = cpg * nsplit;
    const int ng = (int)blockIdx.x / per_group;
    const int within = (int)blockIdx.x - ng * per_group;
    const int tid = threadIdx.x;

    Moments acc = {0.0, 0.0, 0.0};
    const Partial *pp = parts + (size_t)ng * P;
    for (int i = tid; i < P; i += kBlock) {
        const Partial pt = pp[i];
        acc = merge(acc, Moments{(double)pt.count, (double)pt.mean, (double)pt.m2});
    }
    sn[tid] = acc.n;
    smean[tid] = acc.mean;
    sm2[tid] = acc.m2;
    __syncthreads();
    for (int off = kBlock / 2; off > 0; off >>= 1) {
        if (tid < off) {
            const Moments m = merge(Moments{sn[tid], smean[tid], sm2[tid]},
                                    Moments{sn[tid + off], smean[tid + off], sm2[tid + off]});
            sn[tid] = m.n;
            smean[tid] = m.mean;
            sm2[tid] = m.m2;
        }
        __syncthreads();
    }
    const double var = sm2[0] / sn[0];
    const float mean = (float)smean[0];
    const float rstd = (float)(1.0 / sqrt(var + (double)eps));

    const int gg = ng % G, n = ng / G;
    const int cl = within / nsplit, part = within - cl * nsplit;
    const int k = gg * cpg + cl;
    const float a = gamma ? rstd * gamma[k] : rstd;
    const float b = beta ? beta[k] : 0.0f;
    float *yk = y + ((size_t)n * K + k) * plane;

    if (vec4) {
        const int nv = plane >> 2;
        const int per = (nv + nsplit - 1) / nsplit;
        const int beg = part * per, end = min(nv, beg + per);
        float4 *yv = reinterpret_cast<float4 *>(yk);
        // kUnroll independent 128-bit loads in flight per lane
        for (int i0 = beg + tid; i0 < end; i0 += kUnroll * kBlock) {
            float4 v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int i = i0 + u * kBlock;
                if (i < end) v[u] = yv[i];
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int i = i0 + u * kBlock;
                if (i < end) {
                    float4 o;
                    o.x = fmaf(v[u].x - mean, a, b);
                    o.y = fmaf(v[u].y - mean, a, b);
                    o.z = fmaf(v[u].z - mean, a, b);
                    o.w = fmaf(v[u].w - mean, a, b);
                    yv[i] = o;
                }
            }
        }
    } else {
        const int per = (plane + nsplit - 1) / nsplit;
        const int beg = part * per, end = min(plane, beg + per);
        for (int i = beg + tid; i < end; i += kBlock) yk[i] = fmaf(yk[i] - mean, a, b);
    }
}

}  // namespace

hipError_t launch_gn_normalize(const gconv_desc *d, float *y, const Partial *parts, int gn_groups,
                               int parts_per_group, const float *gamma, const float *beta, float eps,
                               hipStream_t st) {
    const int cpg = d->K / gn_groups;
    const int plane = d->Ho * d->Wo;
    // about 32K elements per workgroup
    int nsplit = (plane + 32767) / 32768;
    if (nsplit < 1) nsplit = 1;
    // N * K * nsplit blocks: below 2^31 for every valid descriptor (each
    // block normalizes at least one of the fewer than 2^31 outputs)
    const long long blocks = (long long)d->N * gn_groups * cpg * nsplit;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int vec4 = (plane % 4 == 0) && (((uintptr_t)y & 15u) == 0);
    clear_stale_launch_error();
    hipLaunchKernelGGL(gn_normalize_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, y,
                       parts, parts_per_group, gamma, beta, d->K, gn_groups, cpg, plane, nsplit, eps,
                       vec4);
    return hipGetLastError();
}

}  // namespace gconv
