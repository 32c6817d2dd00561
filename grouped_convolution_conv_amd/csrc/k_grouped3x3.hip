// k_grouped3x3.hip -- grouped / depthwise 3x3, stride 1, pad 1, dilation 1,
// with 1, 2 or 4 input channels per group (the workload of the GroupConv
// Atlas page).
//
// Design for gfx950 (VALU, HBM-bound):
//  - One workgroup (256 lanes = 4 wave64) owns one (n, group, block of up
//    to 4 output channels, band of BH rows x TW columns).  It stages the
//    band's input rows for the group's channels, with a one-pixel zero halo,
//    in LDS: every input byte comes from HBM once per output-channel block
//    (the cooperative shared halo of the Atlas page's third kernel).
//  - Each lane computes Q adjacent outputs along W for every output channel
//    of the block (the Atlas page's fourth kernel computes four adjacent
//    outputs per thread; here Q is 4 or 8 and the lane also covers up to four
//    output channels).  Per input channel and kernel row it reads Q+2
//    inputs with 128-bit LDS loads and issues CO*3*Q FMAs, with the weights
//    held in scalar registers (uniform over the workgroup).
//  - Results leave as 128-bit stores; the W tail is masked.
#include "dev_common.h"
#include "internal.h"

namespace gconv {
namespace {

constexpr int kBlock = 256;

struct G3Params {
    int C, H, W, K;
    int cout;       // output channels per group
    int n_cob;      // output-channel blocks per group (cout / CO)
    int BH, TW;     // band height (rows) and width (columns, multiple of Q)
    int n_cb;       // column bands
    int pitch;      // LDS row pitch in floats (multiple of 4, >= TW + 2)
    int vec_store;  // W % 4 == 0 and y 16-byte aligned
};

template <int CI, int CO, int Q>
__global__ __launch_bounds__(kBlock) void grouped3x3_kernel(const float *__restrict__ x,
                                                            const float *__restrict__ w,
                                                            const float *__restrict__ bias,
                                                            float *__restrict__ y, G3Params p) {
    extern __shared__ float4 lds4[];
    float *lds = reinterpret_cast<float *>(lds4);
    const int tid = threadIdx.x;
    const int rb = blockIdx.x / p.n_cb, cb = blockIdx.x - rb * p.n_cb;
    const int g = blockIdx.y / p.n_cob, cob = blockIdx.y - g * p.n_cob;
    const int n = blockIdx.z;
    const int oh0 = rb * p.BH, c0 = cb * p.TW;
    const int rows = p.BH + 2, cols = p.TW + 2;
    const size_t HW = (size_t)p.H * p.W;

    // ---- stage input rows [oh0-1, oh0+BH] x cols [c0-1, c0+TW] of the
    //      group's CI channels; LDS column j holds input column c0 - 1 + j.
    const float *xg = x + ((size_t)n * p.C + (size_t)g * CI) * HW;
    const int total = CI * rows * cols;
    for (int e = tid; e < total; e += kBlock) {
        const int row = e / cols;           // ci * rows + lr
        const int lc = e - row * cols;
        const int ci = row / rows;
        const int lr = row - ci * rows;
        const int ih = oh0 - 1 + lr, iw = c0 - 1 + lc;
        float v = 0.0f;
        if (ih >= 0 && ih < p.H && iw >= 0 && iw < p.W) v = xg[ci * HW + (size_t)ih * p.W + iw];
        lds[row * p.pitch + lc] = v;
    }
    __syncthreads();

    const int k0 = g * p.cout + cob * CO;
    const float *wb = w + (size_t)k0 * CI * 9;  // uniform over the workgroup

    const int tasks_per_row = p.TW / Q;
    const int ntask = p.BH * tasks_per_row;
    for (int task = tid; task < ntask; task += kBlock) {
        const int lr = task / tasks_per_row;
        const int jq = (task - lr * tasks_per_row) * Q;
        const int oh = oh0 + lr, ow = c0 + jq;
        if (oh >= p.H || ow >= p.W) continue;

        float acc[CO][Q];
#pragma unroll
        for (int co = 0; co < CO; ++co)
#pragma unroll
            for (int q = 0; q < Q; ++q) acc[co][q] = 0.0f;

#pragma unroll
        for (int ci = 0; ci < CI; ++ci) {
            // this input channel's weights for the block (scalar loads)
            float wr[CO][9];
#pragma unroll
            for (int co = 0; co < CO; ++co)
#pragma unroll
                for (int t = 0; t < 9; ++t) wr[co][t] = wb[(co * CI + ci) * 9 + t];
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                const float *src = lds + (ci * rows + lr + r) * p.pitch + jq;
                float win[Q + 2];
#pragma unroll
                for (int q = 0; q < Q; q += 4) {
                    const float4 v = *reinterpret_cast<const float4 *>(src + q);
                    win[q] = v.x; win[q + 1] = v.y; win[q + 2] = v.z; win[q + 3] = v.w;
                }
                const float2 t2 = *reinterpret_cast<const float2 *>(src + Q);
                win[Q] = t2.x;
                win[Q + 1] = t2.y;
#pragma unroll
                for (int co = 0; co < CO; ++co)
#pragma unroll
                    for (int s = 0; s < 3; ++s)
#pragma unroll
                        for (int q = 0; q < Q; ++q)
                            acc[co][q] = fmaf(win[q + s], wr[co][r * 3 + s], acc[co][q]);
            }
        }

#pragma unroll
        for (int co = 0; co < CO; ++co) {
            const float b = bias ? bias[k0 + co] : 0.0f;
            float *dst = y + ((size_t)n * p.K + k0 + co) * HW + (size_t)oh * p.W + ow;
            if (p.vec_store && ow + Q <= p.W) {
#pragma unroll
                for (int q = 0; q < Q; q += 4)
                    *reinterpret_cast<float4 *>(dst + q) =
                        make_float4(acc[co][q] + b, acc[co][q + 1] + b, acc[co][q + 2] + b, acc[co][q + 3] + b);
            } else {
#pragma unroll
                for (int q = 0; q < Q; ++q)
                    if (ow + q < p.W) dst[q] = acc[co][q] + b;
            }
        }
    }
}

template <int CI, int CO, int Q>
hipError_t launch_t(const G3Params &p, dim3 grid, size_t lds, const float *x, const float *w,
                    const float *bias, float *y, hipStream_t st) {
    clear_stale_launch_error();
    hipLaunchKernelGGL((grouped3x3_kernel<CI, CO, Q>), grid, dim3(kBlock), lds, st, x, w, bias, y, p);
    return hipGetLastError();
}

template <int CI, int Q>
hipError_t launch_co(int CO, const G3Params &p, dim3 grid, size_t lds, const float *x,
                     const float *w, const float *bias, float *y, hipStream_t st) {
    switch (CO) {
        case 4: return launch_t<CI, 4, Q>(p, grid, lds, x, w, bias, y, st);
        case 2: return launch_t<CI, 2, Q>(p, grid, lds, x, w, bias, y, st);
        default: return launch_t<CI, 1, Q>(p, grid, lds, x, w, bias, y, st);
    }
}

template <int Q>
hipError_t launch_ci(int CI, int CO, const G3Params &p, dim3 grid, size_t lds, const float *x,
                     const float *w, const float *bias, float *y, hipStream_t st) {
    switch (CI) {
        case 4: return launch_co<4, Q>(CO, p, grid, lds, x, w, bias, y, st);
        case 2: return launch_co<2, Q>(CO, p, grid, lds, x, w, bias, y, st);
        default: return launch_co<1, Q>(CO, p, grid, lds, x, w, bias, y, st);
    }
}

}  // namespace

bool grouped3x3_supported(const gconv_desc *d) {
    return d->R == 3 && d->S == 3 && d->stride == 1 && d->pad == 1 && d->dil == 1 &&
           (d->cin == 1 || d->cin == 2 || d->cin == 4);
}

hipError_t launch_grouped3x3(const gconv_desc *d, const float *x, const float *w, const float *bias,
                             float *y, hipStream_t st) {
    if (!grouped3x3_supported(d)) return hipErrorInvalidValue;
    const int Q = d->W >= 32 ? 8 : 4;
    const int CO = d->cout % 4 == 0 ? 4 : (d->cout % 2 == 0 ? 2 : 1);
    G3Params p;
    p.C = d->C; p.H = d->H; p.W = d->W; p.K = d->K;
    p.cout = d->cout;
    p.n_cob = d->cout / CO;
    // band width: the whole row when it fits 32 lanes, else 32*Q columns
    const int wq = (d->W + Q - 1) / Q;
    const int tasks_per_row = wq < 32 ? wq : 32;
    p.TW = tasks_per_row * Q;
    p.n_cb = (d->W + p.TW - 1) / p.TW;
    // band height: fill 256 lanes, then even out the bands over H
    int bh = kBlock / tasks_per_row;
    if (bh > d->H) bh = d->H;
    const int n_rb = (d->H + bh - 1) / bh;
    p.BH = (d->H + n_rb - 1) / n_rb;
    p.pitch = ((p.TW + 2) + 3) & ~3;
    p.vec_store = (d->W % 4 == 0) && (((uintptr_t)y & 15u) == 0);
    const long long gx = (long long)n_rb * p.n_cb;
    const long long gy = (long long)d->groups * p.n_cob;
    if (gx > 0x7fffffffLL || gy > 65535 || d->N > 65535) return hipErrorInvalidConfiguration;
    const size_t lds = sizeof(float) * (size_t)d->cin * (p.BH + 2) * p.pitch;
    dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)d->N);
    if (Q == 8) return launch_ci<8>(d->cin, CO, p, grid, lds, x, w, bias, y, st);
    return launch_ci<4>(d->cin, CO, p, grid, lds, x, w, bias, y, st);
}

}  // namespace gconv
