// k_depthwise.hip -- depthwise K x K convolution with zero padding
// dilation * (K/2) ("same" padding): K = 5 or 7 at stride 1, K = 3 or 5 at
// stride 2, K = 3 at dilation 2 (stride 1), and K = 3 at stride 1 on small
// depthwise planes packed several to a wave.  The GroupConv Atlas
// project page's direct kernel (k0, "Direct mapping") takes any geometry;
// its k3 card computes four adjacent outputs per thread.  This kernel is the
// four-outputs-per-lane form for these depthwise geometries.  VALU
// arithmetic, HBM-bound for K = 3 and 5.
//
// The same register-streaming design as grouped3x3_rows_kernel, for one
// input channel per group (depthwise, with any channel multiplier) or groups
// of 2, 4, 8 or 16 input channels, with CO output channels per lane:
//  - a wave owns whole output rows of one (n, group, block of CO output
//    channels) plane; a lane owns RB output rows x 4 output columns of each
//    of the CO channels, and walks the group's input channels one by one;
//  - per input row it needs, a lane reads its own ST*4 input columns (one or
//    two 16-byte buffer loads, zero outside the image) and takes the padding
//    columns to its left and the columns past its right edge from the
//    neighbouring lanes with cross-lane moves;
//  - ragged rows (an output width that is not a multiple of 4, an input row
//    not 16-byte aligned, or an odd input width at stride 2) take the same
//    kernel with one 4-byte load per column, each zero past the row's end,
//    and masked 4-byte stores; small depthwise planes are packed several to
//    a wave;
//  - no LDS, no barriers; rows shared by neighbouring lanes and waves come
//    from the L2.
#include "dev_common.h"
#include "internal.h"

namespace gconv {
namespace {

constexpr int kBlock = 256;
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer access, gfx9 family
constexpr int kOutOfPlane = 0x7fffffff;

struct DwParams {
    int C, H, W, Ho, Wo, K;
    int G;        // groups
    int cout;     // output channels per group
    int n_cob;    // blocks of CO output channels per group
    int cg;       // 4-column output groups per row: ceil(Wo / 4)
    int rpw;      // lane strips (of RB output rows) per wave: 64 / cg
    int strips;   // strips per plane: ceil(Ho / RB)
    int wpp;      // waves per plane: ceil(strips / rpw)
    int waves;    // N * G * n_cob * wpp (packed planes: ceil(planes / ppw))
    // packed planes only
    int lpp;      // lanes per plane: cg * strips (at most 32)
    int ppw;      // planes per wave: 64 / lpp
    int planes;   // N * G * n_cob
    int x_bytes;  // size of x (below 2^31)
    int rb;       // output rows per lane (the kernel's RB)
};

// Row forms.  kAligned: every row holds exactly 4 * ST input columns and 4
// output columns per lane, 16-byte aligned.  kRagged: one 4-byte load per
// column, zero past the row's end, masked stores.  kPacked: ragged rows of
// small planes, several (n, group, channel block) planes per wave, each lane
// with its own plane (per-lane weights and offsets); for planes that would
// leave most of a wave's lanes idle (7x7 or 14x14 outputs).
constexpr int kAligned = 0, kRagged = 1, kPacked = 2;

// RB: output rows per lane.
template <int KS, int ST, int DL, int CI, int CO, int RM, int RB>
__global__ __launch_bounds__(kBlock) void depthwise_rows_kernel(const float *__restrict__ x,
                                                                const float *__restrict__ w,
                                                                const float *__restrict__ bias,
                                                                float *__restrict__ y, DwParams p) {
    constexpr int PAD = DL * (KS / 2);
    constexpr int SPAN = DL * (KS - 1) + 1;          // input rows (columns) one output sees
    constexpr int NIR = ST * (RB - 1) + SPAN;        // input rows a lane reads
    constexpr int OWN = 4 * ST;                      // input columns a lane loads itself
    constexpr int RIGHT = SPAN - PAD - ST;           // columns needed past the lane's own ones
    constexpr int WL = PAD + OWN + RIGHT;            // window: input columns ST*oc0 - PAD ...
    static_assert(PAD <= OWN && RIGHT >= 0 && RIGHT <= OWN, "neighbour exchange reaches one lane");

    constexpr bool RAG = RM != kAligned;

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)blockIdx.x * (kBlock / 64) + (int)(threadIdx.x >> 6));
    if (wv >= p.waves) return;  // whole waves only
    const int HW = p.H * p.W;
    int cob, g, n, strip, cgi;
    bool active;
    __amdgpu_buffer_rsrc_t rs;
    int base = 0;  // byte offset of the group's first input plane in rs
    if constexpr (RM == kPacked) {
        // lane -> (plane slot, strip, column group); plane -> (n, group,
        // output-channel block), block fastest
        const int pl = lane / p.lpp, r = lane - pl * p.lpp;
        const int sl = r / p.cg;
        cgi = r - sl * p.cg;
        strip = sl;
        const int plane = wv * p.ppw + pl;
        active = pl < p.ppw && plane < p.planes;
        const int pc = active ? plane : 0;
        cob = pc % p.n_cob;
        const int t1 = pc / p.n_cob;
        g = t1 % p.G;
        n = t1 / p.G;
        // one resource over all of x (below 2^31 bytes)
        rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(x), (short)0, p.x_bytes, kBufferWord3);
        base = (n * p.C + g * CI) * HW * (int)sizeof(float);
    } else {
        // wave -> (n, group, wave in plane, output-channel block), block
        // fastest: blocks that read the same input rows are neighbouring waves
        cob = wv % p.n_cob;
        const int t0 = wv / p.n_cob;
        const int wip = t0 % p.wpp;
        const int t1 = t0 / p.wpp;
        g = t1 % p.G;
        n = t1 / p.G;
        const int sl = lane / p.cg;
        cgi = lane - sl * p.cg;
        strip = wip * p.rpw + sl;
        active = sl < p.rpw && strip < p.strips;
        // one resource over the group's CI input planes
        rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(x + ((size_t)n * p.C + (size_t)g * CI) * HW),
                                               (short)0, CI * HW * (int)sizeof(float), kBufferWord3);
    }
    const int k0 = g * p.cout + cob * CO;
    const int oh0 = strip * RB, oc0 = cgi * 4;
    const int ih0 = ST * oh0 - PAD, ic0 = ST * oc0;
    const bool has_left = cgi > 0, has_right = cgi < p.cg - 1;

    float acc[CO][RB][4];
#pragma unroll
    for (int co = 0; co < CO; ++co) {
        const float b = bias ? bias[k0 + co] : 0.0f;
#pragma unroll
        for (int rr = 0; rr < RB; ++rr)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[co][rr][q] = b;
    }

    // two input channels per iteration: the second channel's loads can be
    // issued before the first one's FMAs
#pragma unroll 2
    for (int ci = 0; ci < CI; ++ci) {
        // weights of the block's output channels for input channel ci
        // (wave-uniform: scalar loads)
        float wk[CO][KS * KS];
#pragma unroll
        for (int co = 0; co < CO; ++co)
#pragma unroll
            for (int t = 0; t < KS * KS; ++t) wk[co][t] = w[((size_t)(k0 + co) * CI + ci) * KS * KS + t];

        // the lane's own columns of every input row it needs: buffer loads
        // with out-of-range offsets (rows above/below the image, idle lanes)
        // reading 0
        float own[NIR][OWN];
#pragma unroll
        for (int i = 0; i < NIR; ++i) {
            const int ih = ih0 + i;
            const int rowb = base + ((ci * p.H + ih) * p.W + ic0) * (int)sizeof(float);
            const bool row_in = active && ih >= 0 && ih < p.H;
            if constexpr (RAG) {
#pragma unroll
                for (int t = 0; t < OWN; ++t) {
                    const int off = row_in && ic0 + t < p.W ? rowb + 4 * t : kOutOfPlane;
                    own[i][t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
                }
            } else {
#pragma unroll
                for (int v = 0; v < ST; ++v) {
                    const int off = row_in ? rowb + 16 * v : kOutOfPlane;
                    const float4 f =
                        __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
                    own[i][4 * v + 0] = f.x; own[i][4 * v + 1] = f.y;
                    own[i][4 * v + 2] = f.z; own[i][4 * v + 3] = f.w;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NIR; ++i) {
            float win[WL];
#pragma unroll
            for (int t = 0; t < PAD; ++t) {  // columns ic0 - PAD + t: the left lane's last ones
                const float v = __shfl_up(own[i][OWN - PAD + t], 1, 64);
                win[t] = has_left ? v : 0.0f;
            }
#pragma unroll
            for (int t = 0; t < OWN; ++t) win[PAD + t] = own[i][t];
#pragma unroll
            for (int t = 0; t < RIGHT; ++t) {  // columns ic0 + OWN + t: the right lane's first ones
                const float v = __shfl_down(own[i][t], 1, 64);
                win[PAD + OWN + t] = has_right ? v : 0.0f;
            }
#pragma unroll
            for (int kr = 0; kr < KS; ++kr) {
                // input row i feeds output row rr through kernel row kr when
                // i = ST*rr + DL*kr
                const int di = i - DL * kr;
                if (di < 0 || di % ST != 0 || di / ST >= RB) continue;
                const int rr = di / ST;
#pragma unroll
                for (int co = 0; co < CO; ++co)
#pragma unroll
                    for (int s = 0; s < KS; ++s)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[co][rr][q] = fmaf(win[ST * q + DL * s], wk[co][kr * KS + s], acc[co][rr][q]);
            }
        }
    }
    if (!active) return;
    const size_t plane_out = (size_t)p.Ho * p.Wo;
    float *yb = y + ((size_t)n * p.K + k0) * plane_out + oc0;
#pragma unroll
    for (int co = 0; co < CO; ++co)
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
            const int oh = oh0 + rr;
            if (oh >= p.Ho) continue;
            float *yr = yb + co * plane_out + (size_t)oh * p.Wo;
            if constexpr (RAG) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (oc0 + q < p.Wo) yr[q] = acc[co][rr][q];
            } else {
                *reinterpret_cast<float4 *>(yr) =
                    make_float4(acc[co][rr][0], acc[co][rr][1], acc[co][rr][2], acc[co][rr][3]);
            }
        }
}

template <int KS, int ST, int DL, int CI, int CO>
hipError_t launch_t(int rm, const DwParams &p, const float *x, const float *w, const float *bias, float *y,
                    hipStream_t st) {
    const int grid = (p.waves + kBlock / 64 - 1) / (kBlock / 64);
    clear_stale_launch_error();
    if (rm == kPacked) {
        // packed planes are instantiated for one input channel per group;
        // one output row per lane at stride 2 only
        if constexpr (CI == 1 && ST == 2) {
            if (p.rb == 1) {
                hipLaunchKernelGGL((depthwise_rows_kernel<KS, ST, DL, CI, CO, kPacked, 1>), dim3(grid), dim3(kBlock),
                                   0, st, x, w, bias, y, p);
                return hipGetLastError();
            }
        }
        if constexpr (CI == 1)
            hipLaunchKernelGGL((depthwise_rows_kernel<KS, ST, DL, CI, CO, kPacked, 2>), dim3(grid), dim3(kBlock), 0,
                               st, x, w, bias, y, p);
        else
            return hipErrorInvalidValue;
    } else if (rm == kRagged) {
        if constexpr (ST == 2) {
            if (p.rb == 1) {
                hipLaunchKernelGGL((depthwise_rows_kernel<KS, ST, DL, CI, CO, kRagged, 1>), dim3(grid), dim3(kBlock),
                                   0, st, x, w, bias, y, p);
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((depthwise_rows_kernel<KS, ST, DL, CI, CO, kRagged, 2>), dim3(grid), dim3(kBlock), 0, st,
                           x, w, bias, y, p);
    } else {
        if constexpr (ST == 2) {
            if (p.rb == 1) {
                hipLaunchKernelGGL((depthwise_rows_kernel<KS, ST, DL, CI, CO, kAligned, 1>), dim3(grid), dim3(kBlock),
                                   0, st, x, w, bias, y, p);
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((depthwise_rows_kernel<KS, ST, DL, CI, CO, kAligned, 2>), dim3(grid), dim3(kBlock), 0, st,
                           x, w, bias, y, p);
    }
    return hipGetLastError();
}

// channels per group (CI) and output channels per lane (CO) for one geometry
template <int KS, int ST, int DL>
hipError_t launch_geom(int rm, int CI, int CO, const DwParams &p, const float *x, const float *w, const float *bias,
                       float *y, hipStream_t st) {
    if (CI == 1) {
        if (CO == 4) return launch_t<KS, ST, DL, 1, 4>(rm, p, x, w, bias, y, st);
        if (CO == 2) return launch_t<KS, ST, DL, 1, 2>(rm, p, x, w, bias, y, st);
        return launch_t<KS, ST, DL, 1, 1>(rm, p, x, w, bias, y, st);
    }
    if (CI == 16) {
        if (CO == 4) return launch_t<KS, ST, DL, 16, 4>(rm, p, x, w, bias, y, st);
        if (CO == 2) return launch_t<KS, ST, DL, 16, 2>(rm, p, x, w, bias, y, st);
        return launch_t<KS, ST, DL, 16, 1>(rm, p, x, w, bias, y, st);
    }
    if (CI == 8) {
        if (CO == 4) return launch_t<KS, ST, DL, 8, 4>(rm, p, x, w, bias, y, st);
        if (CO == 2) return launch_t<KS, ST, DL, 8, 2>(rm, p, x, w, bias, y, st);
        return launch_t<KS, ST, DL, 8, 1>(rm, p, x, w, bias, y, st);
    }
    if (CI == 2) {
        if (CO == 2) return launch_t<KS, ST, DL, 2, 2>(rm, p, x, w, bias, y, st);
        return launch_t<KS, ST, DL, 2, 1>(rm, p, x, w, bias, y, st);
    }
    if (CO == 4) return launch_t<KS, ST, DL, 4, 4>(rm, p, x, w, bias, y, st);
    if (CO == 2) return launch_t<KS, ST, DL, 4, 2>(rm, p, x, w, bias, y, st);
    return launch_t<KS, ST, DL, 4, 1>(rm, p, x, w, bias, y, st);
}

}  // namespace

namespace {

// The instantiated (K, stride, dilation) triples: 0 if none.
int variant_of(int ks, int st, int dl) {
    if (ks == 5 && st == 1 && dl == 1) return 1;
    if (ks == 7 && st == 1 && dl == 1) return 2;
    if (ks == 3 && st == 2 && dl == 1) return 3;
    if (ks == 5 && st == 2 && dl == 1) return 4;
    if (ks == 3 && st == 1 && dl == 2) return 5;
    if (ks == 3 && st == 1 && dl == 1) return 6;  // small depthwise planes only
    return 0;
}

}  // namespace

// Output channels per lane: as many as the group has input channels, up to 4;
// with one input channel per group (a depthwise channel multiplier) up to 4
// as well, since each loaded input window then feeds only KS * KS FMAs per
// output channel.  Always a divisor of the group's output channels.
int dw_co(const gconv_desc *d) {
    const int lim = d->cin == 1 || d->cin >= 4 ? 4 : d->cin;
    return d->cout % lim == 0 ? lim : (d->cout % 2 == 0 ? 2 : 1);
}

// 3x3, stride 1, padding 1, one input channel per group, on planes small
// enough that the packed form puts at least two of them in a wave (outputs of
// about 16 x 16 or less): there the grouped 3x3 kernels would give each plane
// a wave or a workgroup of its own and leave most lanes idle.
bool depthwise_small_3x3(const gconv_desc *d) {
    if (!(d->R == 3 && d->S == 3 && d->stride_h == 1 && d->stride_w == 1 && d->dil_h == 1 && d->dil_w == 1 &&
          d->pad_h == 1 && d->pad_w == 1 && d->cin == 1))
        return false;
    // the launcher's packing rule at two output rows per lane
    const long long lpp = (long long)((d->Wo + 3) / 4) * ((d->Ho + 1) / 2);
    const long long x_bytes = (long long)d->N * d->C * d->H * d->W * (long long)sizeof(float);
    const long long planes = (long long)d->N * d->groups * (d->cout / dw_co(d));
    return lpp <= 32 && x_bytes < 0x7fffffffLL && planes < 0x7fffffffLL - 64 * 64;
}

// The dispatcher's choice among the small-plane 3x3 layers: the packed kernel
// once it has a wave per SIMD (1024 waves); below that the grouped 3x3
// register kernel, which gives each plane its own wave, measured faster
// (about 2.8-3.1 against 3.4-3.5 us on 64-512 planes of 14 x 14).
bool depthwise_small_3x3_preferred(const gconv_desc *d) {
    if (!depthwise_small_3x3(d)) return false;
    const long long lpp = (long long)((d->Wo + 3) / 4) * ((d->Ho + 1) / 2);
    const long long planes = (long long)d->N * d->groups * (d->cout / dw_co(d));
    const long long ppw = 64 / lpp;
    return (planes + ppw - 1) / ppw >= 1024;
}

bool depthwise_supported(const gconv_desc *d) {
    // one input channel per group (depthwise, with any channel multiplier),
    // or groups of 2, 4, 8 or 16 input channels; any output channels per group
    const bool dw = d->cin == 1;
    const bool small_groups = (d->cin == 2 || d->cin == 4 || d->cin == 8 || d->cin == 16) && d->groups > 1;
    if (!(dw || small_groups) || d->R != d->S) return false;
    if (d->stride_h != d->stride_w || d->dil_h != d->dil_w) return false;
    const int ks = d->R, st = d->stride_h, dl = d->dil_h;
    if (d->pad_h != dl * (ks / 2) || d->pad_w != dl * (ks / 2)) return false;
    const int var = variant_of(ks, st, dl);
    if (!var || (var == 6 && !depthwise_small_3x3(d))) return false;
    // an output row within one wave (64 lanes of 4 columns); the input row
    // no wider than stride * output width, which this padding implies, so
    // the last lane of a row needs no columns from a lane it does not have;
    // buffer offsets in 32 bits
    if (d->Wo < 1 || d->Wo > 256 || d->Ho < 1) return false;
    if (d->W > st * d->Wo) return false;
    return (long long)d->cin * (d->H + 16) * d->W * 4 < 0x7fffffffLL;
}

// Whole rows of 4 * stride input and 4 output columns per lane, 16-byte
// aligned; anything else takes the ragged form of the kernel.
static bool depthwise_aligned(const gconv_desc *d, const float *x, const float *y) {
    return d->Wo % 4 == 0 && d->W == d->stride_h * d->Wo && ((((uintptr_t)x) | ((uintptr_t)y)) & 15u) == 0;
}

hipError_t launch_depthwise(const gconv_desc *d, const float *x, const float *w, const float *bias, float *y,
                            hipStream_t st) {
    if (!depthwise_supported(d)) return hipErrorInvalidValue;
    int rm = depthwise_aligned(d, x, y) ? kAligned : kRagged;
    const int CO = dw_co(d);
    DwParams p;
    p.C = d->C; p.H = d->H; p.W = d->W; p.Ho = d->Ho; p.Wo = d->Wo; p.K = d->K;
    p.G = d->groups;
    p.cout = d->cout;
    p.n_cob = d->cout / CO;
    p.cg = (d->Wo + 3) / 4;
    p.rpw = 64 / p.cg;
    // output rows per lane: 2, or 1 at stride 2, where a second output row
    // costs 2 more input rows of 2 + K - 1 and shorter lanes hide more
    // latency (depthwise 3x3 from 144 x 112: 31.9 -> 30.6 us, 5x5 from
    // 144 x 56: 11.1 -> 10.0 us, 14 -> 7 columns: 8.7 -> 7.4 us; grouped 3x3
    // with 4 and 8 channels per group: 18.7 -> 16.9 and 22.9 -> 20.9 us; at
    // stride 1 one row per lane measured slower)
    p.rb = d->stride_h == 2 ? 1 : 2;
    p.strips = (d->Ho + p.rb - 1) / p.rb;
    p.wpp = (p.strips + p.rpw - 1) / p.rpw;
    const long long waves = (long long)d->N * d->groups * p.n_cob * p.wpp;
    if (waves > 0x7fffffffLL - 64) return hipErrorInvalidConfiguration;
    p.waves = (int)waves;
    // small planes with one input channel per group: several planes per
    // wave when one plane fills at most half of it
    const long long x_bytes = (long long)d->N * d->C * d->H * d->W * (long long)sizeof(float);
    const long long planes = (long long)d->N * d->groups * p.n_cob;
    p.lpp = p.cg * p.strips;
    if (d->cin == 1 && p.lpp <= 32 && x_bytes < 0x7fffffffLL && planes < 0x7fffffffLL - 64 * 64) {
        rm = kPacked;
        p.ppw = 64 / p.lpp;
        p.planes = (int)planes;
        p.x_bytes = (int)x_bytes;
        p.waves = (int)((planes + p.ppw - 1) / p.ppw);
    }
    switch (variant_of(d->R, d->stride_h, d->dil_h)) {
        case 1: return launch_geom<5, 1, 1>(rm, d->cin, CO, p, x, w, bias, y, st);
        case 2: return launch_geom<7, 1, 1>(rm, d->cin, CO, p, x, w, bias, y, st);
        case 3: return launch_geom<3, 2, 1>(rm, d->cin, CO, p, x, w, bias, y, st);
        case 4: return launch_geom<5, 2, 1>(rm, d->cin, CO, p, x, w, bias, y, st);
        case 5: return launch_geom<3, 1, 2>(rm, d->cin, CO, p, x, w, bias, y, st);
        default:  // 3x3 stride 1: packed depthwise planes (one input channel per group)
            if (CO == 4) return launch_t<3, 1, 1, 1, 4>(rm, p, x, w, bias, y, st);
            if (CO == 2) return launch_t<3, 1, 1, 1, 2>(rm, p, x, w, bias, y, st);
            return launch_t<3, 1, 1, 1, 1>(rm, p, x, w, bias, y, st);
    }
}

}  // namespace gconv
