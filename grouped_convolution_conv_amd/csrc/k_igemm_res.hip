// k_igemm_res.hip -- persistent FP32 MFMA implicit GEMM for convolutions
// whose whole weight tensor fits in LDS (few input channels: the Conv2d
// 8 -> 32, 3x3 of the POPCORNBENCH trace "Kimi-K2.6 l2_p21" is the case it is
// shaped for), with the fused epilogues of that trace's chain.
//
// The arithmetic is the implicit GEMM of k_igemm.hip (same MFMA, same
// operand and accumulator layout): D[k][p] = sum_q W[k][q] X[q][p] with
// q = (c, r, s) split between the two 32-lane halves by input channel.
// What differs is the data movement, designed for gfx950:
//  - a workgroup loads the weights once into LDS ([32*MB][CP*R*S], odd row
//    pitch so 32 lanes reading 32 output channels hit 32 banks) and then
//    walks output tiles (n, 8 rows, 64 columns) in a grid-stride loop;
//  - a tile's input band [CP][8+R-1][64+S-1] (rows padded to whole 16-byte
//    pieces) is prefetched into registers two tiles ahead (one 16-byte load
//    per piece when W and the padding are multiples of 4, else four 4-byte
//    loads) and written to one of two LDS band buffers after the current
//    tile's MFMAs, so the global loads of tile u+2 are in flight during the
//    epilogue of tile u and the MFMAs of tile u+1;
//  - the barriers between tiles order LDS only, so no wave waits for its own
//    output stores before starting the next tile.
// Epilogue modes:
//  kPlain      y = acc (+ bias)
//  kStats      v = sigmoid((acc + bias) * scale), optional store of v, and
//              per wave (two rows of the tile) the (count, mean, M2) of each
//              GroupNorm group of 4 channels, two passes over the registers
//              and no cross-wave reduction (no barrier in the epilogue)
//  kNormalize  v as above, then out = (v - mean) * rstd * gamma + beta with
//              the group statistics already merged, stored to y
#include "dev_common.h"
#include "internal.h"

namespace gconv {
namespace {

constexpr int kBlock = 256;
constexpr int kNBR = 2;  // output rows per wave
constexpr int kNBC = 2;  // 32-column blocks per wave row
constexpr int kTH = 4 * kNBR;
constexpr int kTW = 32 * kNBC;

constexpr int kPlain = 0, kStats = 1, kNormalize = 2;

typedef float floatx16 __attribute__((ext_vector_type(16)));

struct ResParams {
    int C, H, W, K, Ho, Wo, pad;
    int cin, cout;
    int n_tw, n_tiles, units;   // tiles per image row band, per image, in total
    int store;                  // kStats: also store v
    int vec;                    // W, pad multiples of 4 and x 16-byte aligned: 16-byte DMA pieces
};

struct ResEpilogue {
    const float *bias;      // kPlain: nullable conv bias; kStats/kNormalize: required
    const float *scale;     // kStats/kNormalize
    Partial *parts;         // kStats: [N][gn_groups][n_tiles * 4 waves]
    const float2 *gstat;    // kNormalize: (mean, rstd) per (n, gn group)
    const float *gamma;     // kNormalize, nullable
    const float *beta;      // kNormalize, nullable
    int gn_groups;
};

// Workgroup barrier that orders LDS only: unlike __syncthreads() it does not
// wait for the wave's outstanding global stores.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int R, int S, int MB, int CP, int MODE>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(MB == 1 ? 3 : 2))) void igemm_res_kernel(const float *__restrict__ x,
                                                           const float *__restrict__ w,
                                                           float *__restrict__ y, ResParams p,
                                                           ResEpilogue ep) {
    constexpr int RS = R * S;
    constexpr int KW = 32 * MB;
    constexpr int TIH = kTH + R - 1;
    constexpr int TIW = kTW + S - 1;
    constexpr int PITCH = (TIW + 3) & ~3;     // LDS row pitch: whole 16-byte pieces
    constexpr int P4 = PITCH / 4;
    constexpr int XE = CP * TIH * PITCH;      // band elements
    constexpr int XE4 = XE / 4;
    constexpr int NSLOT4 = (XE4 + kBlock - 1) / kBlock;
    constexpr int WP = (CP * RS) | 1;         // weight row pitch (odd)
    constexpr int NB = kNBR * kNBC;
    constexpr int HALF = CP / 2;

    __shared__ float wl[KW * WP];
    // per-channel constants, staged once: LDS reads in the epilogue count on
    // lgkmcnt, whereas per-lane global loads would count on vmcnt and make
    // the epilogue wait for the next tile's DMA
    __shared__ float2 chan_bs[KW];   // (bias, scale); kPlain: (bias or 0, unused)
    __shared__ float2 chan_gb[KW];   // kNormalize: (gamma or 1, beta or 0)
    __shared__ float4 bufA4[XE4 + 1];
    __shared__ float4 bufB4[XE4 + 1];
    float *bufA = reinterpret_cast<float *>(bufA4);
    float *bufB = reinterpret_cast<float *>(bufB4);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, j = lane & 31;
    const size_t HW = (size_t)p.H * p.W;
    const size_t plane = (size_t)p.Ho * p.Wo;

    // ---- weights, once: w[k][c][r][s] for k < cout, c < cin, zero elsewhere
    for (int e = tid; e < KW * CP * RS; e += kBlock) {
        const int k = e / (CP * RS), q = e - k * (CP * RS);
        const int c = q / RS;
        float v = 0.0f;
        if (k < p.cout && c < p.cin) v = w[((size_t)k * p.cin + c) * RS + (q - c * RS)];
        wl[k * WP + q] = v;
    }

    for (int k = tid; k < KW; k += kBlock) {
        float b = 0.0f, sc = 1.0f, ga = 1.0f, be = 0.0f;
        if (k < p.cout) {
            if (ep.bias) b = ep.bias[k];
            if constexpr (MODE != kPlain) sc = ep.scale[k];
            if constexpr (MODE == kNormalize) {
                if (ep.gamma) ga = ep.gamma[k];
                if (ep.beta) be = ep.beta[k];
            }
        }
        chan_bs[k] = make_float2(b, sc);
        chan_gb[k] = make_float2(ga, be);
    }

    // ---- band prefetch through registers: pf holds this lane's pieces of a
    //      tile's band (16-byte pieces when p.vec, else 4-byte elements),
    //      zero outside the image; commit() writes them to an LDS buffer
    float4 pf[NSLOT4];
    auto load = [&](int u) __attribute__((always_inline)) {
        const int t = u % p.n_tiles, n = u / p.n_tiles;
        const int th = t / p.n_tw, tw = t - th * p.n_tw;
        const int ih0 = th * kTH - p.pad, iw0 = tw * kTW - p.pad;
        const float *xb = x + (size_t)n * p.C * HW;
        // an opaque copy of the thread id: the per-slot offsets are the same
        // for every tile, and hoisting them out of the tile loop would keep
        // them live across the MFMA loop
        int tid_o = threadIdx.x;
        asm volatile("" : "+v"(tid_o));
#pragma unroll
        for (int i = 0; i < NSLOT4; ++i) {
            // piece f = (cl*TIH + lr)*P4 + c4: input columns iw0 + 4*c4 .. +3
            // of row ih0 + lr, channel cl
            const int f = i * kBlock + tid_o;
            const int cl = f / (TIH * P4), rem = f - cl * (TIH * P4);
            const int lr = rem / P4, c4 = rem - lr * P4;
            const int ih = ih0 + lr, iw = iw0 + 4 * c4;
            const bool row_ok = f < XE4 && cl < p.cin && ih >= 0 && ih < p.H;
            const float *src = xb + (size_t)cl * HW + (size_t)ih * p.W + iw;
            if (p.vec) {
                // W and iw0 multiples of 4: the piece is wholly in or out
                pf[i] = (row_ok && iw >= 0 && iw < p.W) ? *reinterpret_cast<const float4 *>(src)
                                                        : make_float4(0.f, 0.f, 0.f, 0.f);
            } else {
                pf[i].x = (row_ok && iw + 0 >= 0 && iw + 0 < p.W) ? src[0] : 0.0f;
                pf[i].y = (row_ok && iw + 1 >= 0 && iw + 1 < p.W) ? src[1] : 0.0f;
                pf[i].z = (row_ok && iw + 2 >= 0 && iw + 2 < p.W) ? src[2] : 0.0f;
                pf[i].w = (row_ok && iw + 3 >= 0 && iw + 3 < p.W) ? src[3] : 0.0f;
            }
        }
    };
    auto commit = [&](float *buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NSLOT4; ++i) {
            const int f = i * kBlock + tid;
            if (f < XE4) reinterpret_cast<float4 *>(buf)[f] = pf[i];
        }
    };

    auto compute = [&](int u, const float *buf, auto &&between) __attribute__((always_inline)) {
        const int t = u % p.n_tiles, n = u / p.n_tiles;
        const int th = t / p.n_tw, tw = t - th * p.n_tw;
        const int oh0 = th * kTH, ow0 = tw * kTW;

        floatx16 acc[MB][NB];
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[m][b][v] = 0.0f;
#pragma unroll
        for (int ci = 0; ci < HALF; ++ci) {
            const int cl = h * HALF + ci;
            const float *xq = buf + (cl * TIH + wave * kNBR) * PITCH + j;
            const float *wq = wl + j * WP + cl * RS;
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    float a[MB], b[NB];
#pragma unroll
                    for (int m = 0; m < MB; ++m) a[m] = wq[m * 32 * WP + r * S + s];
#pragma unroll
                    for (int br = 0; br < kNBR; ++br)
#pragma unroll
                        for (int bc = 0; bc < kNBC; ++bc) b[br * kNBC + bc] = xq[(br + r) * PITCH + bc * 32 + s];
#pragma unroll
                    for (int m = 0; m < MB; ++m)
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[m][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[m], b[nb], acc[m][nb], 0, 0, 0);
                }
        }

        between();  // next tiles' data movement, after this tile's LDS reads
        float *yb = y + (size_t)n * p.K * plane;
        if constexpr (MODE == kPlain) {
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int br = 0; br < kNBR; ++br) {
                    const int oh = oh0 + wave * kNBR + br;
#pragma unroll
                    for (int bc = 0; bc < kNBC; ++bc) {
                        const int ow = ow0 + bc * 32 + j;
                        if (oh >= p.Ho || ow >= p.Wo) continue;
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int k = m * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                            if (k < p.cout) yb[(size_t)k * plane + (size_t)oh * p.Wo + ow] = acc[m][br * kNBC + bc][v] + chan_bs[k].x;
                        }
                    }
                }
        } else {
            // local GroupNorm group of accumulator v in block m: rows
            // 8q + 4h + (0..3) -> lg = 8m + 2q + h (4 channels per group)
            float gm[MB][4], ga[MB][4];  // kNormalize: mean and rstd of the lane's groups
            if constexpr (MODE == kNormalize) {
                // uniform addresses: scalar loads for both halves, then a select
                const float2 *gs = ep.gstat + (size_t)n * ep.gn_groups;
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float2 s0 = gs[8 * m + 2 * q], s1v = gs[8 * m + 2 * q + 1];
                        // readfirstlane pins the loaded values as uniform, so
                        // the select is not turned into a per-lane load
                        const float m0 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s0.x)));
                        const float r0 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s0.y)));
                        const float m1 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s1v.x)));
                        const float r1 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s1v.y)));
                        gm[m][q] = h ? m1 : m0;
                        ga[m][q] = h ? r1 : r0;
                    }
            }
            float s1[MB][4];
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int q = 0; q < 4; ++q) s1[m][q] = 0.0f;
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int k = m * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                    const float2 bs = chan_bs[k];
                    const float bk = bs.x, sk = bs.y;
                    float gk = 1.0f, ck = 0.0f;
                    if constexpr (MODE == kNormalize) {
                        const float2 gb = chan_gb[k];
                        gk = ga[m][v >> 2] * gb.x;
                        ck = gb.y;
                    }
#pragma unroll
                    for (int br = 0; br < kNBR; ++br)
#pragma unroll
                        for (int bc = 0; bc < kNBC; ++bc) {
                            const int oh = oh0 + wave * kNBR + br, ow = ow0 + bc * 32 + j;
                            const bool ok = oh < p.Ho && ow < p.Wo;
                            const float val = sigmoidf((acc[m][br * kNBC + bc][v] + bk) * sk);
                            float *dst = yb + (size_t)k * plane + (size_t)oh * p.Wo + ow;
                            if constexpr (MODE == kStats) {
                                acc[m][br * kNBC + bc][v] = val;
                                if (ok) {
                                    if (p.store) *dst = val;
                                    s1[m][v >> 2] += val;
                                }
                            } else {
                                if (ok) *dst = fmaf(val - gm[m][v >> 2], gk, ck);
                            }
                        }
                }
            if constexpr (MODE == kStats) {
                // statistics of this wave's part of the tile (its kNBR rows),
                // two passes over the registers, no cross-wave reduction: one
                // partial per (tile, wave, group)
                const int rows_ok = max(0, min(kNBR, p.Ho - (oh0 + wave * kNBR)));
                const int cols_ok = min(kTW, p.Wo - ow0);
                const float count = 4.0f * (float)(rows_ok * cols_ok);
                const float inv = count > 0.0f ? 1.0f / count : 0.0f;
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float mu = half_wave_sum(s1[m][q]) * inv;
                        float tq = 0.0f;
#pragma unroll
                        for (int br = 0; br < kNBR; ++br)
#pragma unroll
                            for (int bc = 0; bc < kNBC; ++bc) {
                                const int oh = oh0 + wave * kNBR + br, ow = ow0 + bc * 32 + j;
                                if (oh < p.Ho && ow < p.Wo) {
#pragma unroll
                                    for (int uu = 0; uu < 4; ++uu) {
                                        const float dv = acc[m][br * kNBC + bc][4 * q + uu] - mu;
                                        tq = fmaf(dv, dv, tq);
                                    }
                                }
                            }
                        const float m2 = half_wave_sum(tq);
                        if (j == 0) {
                            Partial pt;
                            pt.count = count;
                            pt.mean = mu;
                            pt.m2 = m2;
                            pt.pad = 0.0f;
                            ep.parts[((size_t)n * ep.gn_groups + 8 * m + 2 * q + h) * (4 * p.n_tiles) + t * 4 + wave] = pt;
                        }
                    }
            }
        }
    };

    // Tile loop: barrier (LDS only) -> MFMAs of tile u -> commit tile u+G
    // (loaded one iteration earlier) to the other buffer -> load tile u+2G
    // into registers -> epilogue of tile u.  The loads have an epilogue and a
    // whole MFMA phase to land; the barriers fence LDS only, so no wave ever
    // waits for its output stores.  Two static buffers keep the LDS objects
    // of the reads and the writes of an iteration distinct.
    int u = blockIdx.x;
    const int G = gridDim.x;
    if (u < p.units) {
        load(u);
        commit(bufA);
        if (u + G < p.units) load(u + G);
    }
    while (u < p.units) {
        lds_barrier();
        compute(u, bufA, [&]() __attribute__((always_inline)) {
            if (u + G < p.units) commit(bufB);
            if (u + 2 * G < p.units) load(u + 2 * G);
        });
        u += G;
        if (u >= p.units) break;
        lds_barrier();
        compute(u, bufB, [&]() __attribute__((always_inline)) {
            if (u + G < p.units) commit(bufA);
            if (u + 2 * G < p.units) load(u + 2 * G);
        });
        u += G;
    }
}

// Merged (mean, rstd) of every (n, GroupNorm group) from the per-tile
// partials, Chan-Golub-LeVeque pairwise updates in double, fixed order.
struct Moments {
    double n, mean, m2;
};

__device__ __forceinline__ Moments merge_m(Moments a, Moments b) {
    if (b.n == 0.0) return a;
    if (a.n == 0.0) return b;
    Moments r;
    r.n = a.n + b.n;
    const double delta = b.mean - a.mean;
    r.mean = a.mean + delta * (b.n / r.n);
    r.m2 = a.m2 + b.m2 + delta * delta * (a.n * b.n / r.n);
    return r;
}

__global__ __launch_bounds__(kBlock) void gn_merge_kernel(const Partial *__restrict__ parts, int P,
                                                          float eps, float2 *__restrict__ gstat) {
    __shared__ double sn[kBlock], smean[kBlock], sm2[kBlock];
    const int ng = blockIdx.x, tid = threadIdx.x;
    Moments acc = {0.0, 0.0, 0.0};
    const Partial *pp = parts + (size_t)ng * P;
    for (int i = tid; i < P; i += kBlock) {
        const Partial pt = pp[i];
        acc = merge_m(acc, Moments{(double)pt.count, (double)pt.mean, (double)pt.m2});
    }
    sn[tid] = acc.n;
    smean[tid] = acc.mean;
    sm2[tid] = acc.m2;
    __syncthreads();
    for (int off = kBlock / 2; off > 0; off >>= 1) {
        if (tid < off) {
            const Moments m = merge_m(Moments{sn[tid], smean[tid], sm2[tid]},
                                      Moments{sn[tid + off], smean[tid + off], sm2[tid + off]});
            sn[tid] = m.n;
            smean[tid] = m.mean;
            sm2[tid] = m.m2;
        }
        __syncthreads();
    }
    if (tid == 0) gstat[ng] = make_float2((float)smean[0], (float)(1.0 / sqrt(sm2[0] / sn[0] + (double)eps)));
}

// ---- host side

constexpr int kMaxResLds = 64 * 1024;  // keep at least two workgroups per CU

template <int R, int S, int MB, int CP>
constexpr int res_lds_bytes() {
    return 4 * (32 * MB * ((CP * R * S) | 1) + 2 * (CP * (kTH + R - 1) * ((kTW + S - 1 + 3) & ~3) + 4));
}

ResParams make_params(const gconv_desc *d) {
    ResParams p;
    p.C = d->C; p.H = d->H; p.W = d->W; p.K = d->K; p.Ho = d->Ho; p.Wo = d->Wo; p.pad = d->pad;
    p.cin = d->cin; p.cout = d->cout;
    p.n_tw = (d->Wo + kTW - 1) / kTW;
    p.n_tiles = p.n_tw * ((d->Ho + kTH - 1) / kTH);
    p.units = d->N * p.n_tiles;
    p.store = 1;
    p.vec = 0;
    return p;
}

ResParams make_params(const gconv_desc *d, const float *x) {
    ResParams p = make_params(d);
    p.vec = (d->W % 4 == 0) && (d->pad % 4 == 0) && (((uintptr_t)x & 15u) == 0);
    return p;
}

int res_mb(const gconv_desc *d) { return d->cout > 32 ? 2 : 1; }
int res_cp(const gconv_desc *d) { return d->cin <= 4 ? 4 : 8; }

template <int R, int S, int MB, int CP, int MODE>
hipError_t launch_t(const ResParams &p, const float *x, const float *w, float *y, const ResEpilogue &ep,
                    hipStream_t st) {
    static_assert(res_lds_bytes<R, S, MB, CP>() <= kMaxResLds, "LDS budget");
    auto kern = igemm_res_kernel<R, S, MB, CP, MODE>;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipErrorInvalidDevice;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBlock, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    const long long want = (long long)cus * per_cu;
    const int grid = (int)(p.units < want ? p.units : want);
    clear_stale_launch_error();
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlock), 0, st, x, w, y, p, ep);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const gconv_desc *d, const ResParams &p, const float *x, const float *w, float *y,
                       const ResEpilogue &ep, hipStream_t st) {
    const int mb = res_mb(d), cp = res_cp(d);
    if (d->R == 3 && d->S == 3) {
        if (mb == 1) return cp == 4 ? launch_t<3, 3, 1, 4, MODE>(p, x, w, y, ep, st) : launch_t<3, 3, 1, 8, MODE>(p, x, w, y, ep, st);
        return cp == 4 ? launch_t<3, 3, 2, 4, MODE>(p, x, w, y, ep, st) : launch_t<3, 3, 2, 8, MODE>(p, x, w, y, ep, st);
    }
    if (d->R == 1 && d->S == 1) {
        if (mb == 1) return cp == 4 ? launch_t<1, 1, 1, 4, MODE>(p, x, w, y, ep, st) : launch_t<1, 1, 1, 8, MODE>(p, x, w, y, ep, st);
        return cp == 4 ? launch_t<1, 1, 2, 4, MODE>(p, x, w, y, ep, st) : launch_t<1, 1, 2, 8, MODE>(p, x, w, y, ep, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool igemm_res_supported(const gconv_desc *d) {
    return d->groups == 1 && d->stride == 1 && d->dil == 1 && d->cin >= 4 && d->cin <= 8 &&
           d->cout >= 8 && d->cout <= 64 && ((d->R == 3 && d->S == 3) || (d->R == 1 && d->S == 1));
}

bool igemm_res_fused_supported(const gconv_desc *d, int gn_groups) {
    return igemm_res_supported(d) && d->cout % (32 * res_mb(d)) == 0 && d->K / gn_groups == 4;
}

int igemm_res_parts_per_group(const gconv_desc *d) { return 4 * make_params(d).n_tiles; }

hipError_t launch_igemm_res(const gconv_desc *d, const float *x, const float *w, const float *bias, float *y,
                            hipStream_t st) {
    if (!igemm_res_supported(d)) return hipErrorInvalidValue;
    ResEpilogue ep{};
    ep.bias = bias;
    return launch_mode<kPlain>(d, make_params(d, x), x, w, y, ep, st);
}

hipError_t launch_igemm_res_stats(const gconv_desc *d, const float *x, const float *w, float *y, bool store,
                                  const FusedEpilogue &fe, hipStream_t st) {
    if (!igemm_res_fused_supported(d, fe.gn_groups)) return hipErrorInvalidValue;
    ResParams p = make_params(d, x);
    p.store = store ? 1 : 0;
    ResEpilogue ep{};
    ep.bias = fe.bias;
    ep.scale = fe.scale;
    ep.parts = fe.parts;
    ep.gn_groups = fe.gn_groups;
    return launch_mode<kStats>(d, p, x, w, y, ep, st);
}

hipError_t launch_gn_merge(const gconv_desc *d, const Partial *parts, int gn_groups, int parts_per_group,
                           float eps, float2 *gstat, hipStream_t st) {
    const long long ng = (long long)d->N * gn_groups;
    if (ng > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    clear_stale_launch_error();
    hipLaunchKernelGGL(gn_merge_kernel, dim3((unsigned)ng), dim3(kBlock), 0, st, parts, parts_per_group, eps, gstat);
    return hipGetLastError();
}

hipError_t launch_igemm_res_normalize(const gconv_desc *d, const float *x, const float *w, float *y,
                                      const FusedEpilogue &fe, const float2 *gstat, const float *gamma,
                                      const float *beta, hipStream_t st) {
    if (!igemm_res_fused_supported(d, fe.gn_groups)) return hipErrorInvalidValue;
    ResEpilogue ep{};
    ep.bias = fe.bias;
    ep.scale = fe.scale;
    ep.gstat = gstat;
    ep.gamma = gamma;
    ep.beta = beta;
    ep.gn_groups = fe.gn_groups;
    return launch_mode<kNormalize>(d, make_params(d, x), x, w, y, ep, st);
}

}  // namespace gconv
