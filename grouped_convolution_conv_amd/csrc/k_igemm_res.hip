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
//    pieces) is prefetched into registers two tiles ahead and written to one
//    of two LDS band buffers after the current tile's MFMAs, so the global
//    loads of tile u+2 are in flight during the epilogue of tile u and the
//    MFMAs of tile u+1;
//  - every global access goes through a buffer resource, and an element
//    outside the image (padding, tile overhang, idle lanes) gets an offset
//    beyond the resource's range: the hardware reads it as zero and drops a
//    store to it.  The code has no branches around memory instructions, so
//    the compiler waits for exactly the loads a step needs (a partial
//    vmcnt) instead of for every outstanding load and store;
//  - the barriers between tiles order LDS only, so no wave waits for its own
//    output stores before starting the next tile.
// The fused 3x3 passes with 32 output channels (WG) multiply in the Winograd
// form F(2x2, 3x3) instead (see winograd_tile below): 16 products per 2x2
// outputs and input channel, against 36 for the direct sum.
// Epilogue modes:
//  kPlain       y = acc (+ bias)
//  kStats       v = sigmoid((acc + bias) * scale) and, per wave (two rows of
//               the tile), the (count, mean, M2) of each GroupNorm group of 4
//               channels, two passes over the registers, no cross-wave
//               reduction (no barrier in the epilogue)
//  kStatsStore  kStats, and v is stored to y
//  kNormalize   v as above, then out = (v - mean) * rstd * gamma + beta with
//               the group statistics already merged, stored to y
//  kOnePass     the whole chain in one conv pass: v is stored as in
//               kStatsStore and each wave publishes its tile's partials
//               (device-scope stores, then an arrival count per image); the
//               wave whose arrival completes an image merges its partials
//               and publishes (mean, rstd).  A fixed number of tiles later
//               the workgroup reads the tile's v back (from the last-level
//               cache, where it still is) and normalizes it in place.  A wave
//               whose image is not ready after a bounded wait leaves v and
//               lists its rows for a trailing in-place pass, so no wave ever
//               waits on work that is not running: the result never depends
//               on how many workgroups are resident.
#include <atomic>
#include <type_traits>

#include "dev_common.h"
#include "internal.h"

namespace gconv {
namespace {

constexpr int kBlock = 256;
constexpr int kNBR = 2;  // output rows per wave
constexpr int kNBC = 2;  // 32-column blocks per wave row
constexpr int kTH = 4 * kNBR;
constexpr int kTW = 32 * kNBC;
constexpr int kLag = 3;   // kOnePass: tiles between a tile's conv and its normalization

constexpr int kPlain = 0, kStats = 1, kNormalize = 2, kStatsStore = 3, kOnePass = 4;
constexpr int kResWaves = 3;  // waves per SIMD the register budget is sized for

// buffer resource descriptor word 3 for raw (untyped, unswizzled) 32-bit
// access on gfx9-family GPUs, and a byte offset beyond every range used here
constexpr int kBufferWord3 = 0x00020000;
constexpr int kOutOfRange = 0x7fffffff;
constexpr int kStoreOutOfRange = 0x40000000;  // with a scalar offset below 1 GB added
constexpr float kLog2e = 1.44269504088896340736f;
// cache policy of a device-scope (all XCDs) access on gfx950: sc1.  The
// one-pass chain publishes partials, statistics and flags with such accesses
// and orders them with explicit vmcnt waits (a device-scope access has
// completed at device scope when the wait returns), instead of C++
// release/acquire atomics: at agent scope those write back the whole L2
// (buffer_wbl2) on every release and invalidate it (buffer_inv) on every
// acquire, which on this path would cost more than the conv's stores
// themselves.
constexpr int kCpolSc1 = 16;
// s_waitcnt immediate that waits for vmcnt = 0 only (gfx9 encoding: expcnt
// and lgkmcnt fields at their maxima)
constexpr int kWaitVmcnt0 = 0x0F70;

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct ResParams {
    int C, H, W, K, Ho, Wo;
    int pad_h, pad_w;  // zero padding above/below and left/right
    int cin, cout;
    int n_tw, n_tiles, units;   // tiles per image row band, per image, in total
    int parts_stride;           // partials per (image, group) in the workspace
    int x_bytes;                // bytes of one input image (C * H * W floats)
    int y_bytes;                // bytes of one output image (K * Ho * Wo floats)
    int parts_bytes;            // bytes of one image's GroupNorm partials
};

struct ResEpilogue {
    const float *bias;      // kPlain: nullable conv bias; other modes: required
    const float *scale;     // all modes but kPlain
    Partial *parts;         // kStats*, kOnePass: [N][gn_groups][n_tiles * 4 waves]
    const float2 *gstat;    // kNormalize: (mean, rstd) per (n, gn group)
    const float *gamma;     // kNormalize, kOnePass: nullable
    const float *beta;      // kNormalize, kOnePass: nullable
    int gn_groups;
    // kOnePass only
    float2 *gstat_out;      // (mean, rstd) per (n, gn group), written by the merging wave
    int *arrive;            // [N] tiles whose partial is published, zero at launch
    int *ready;             // [N] 1 once gstat_out of the image is published, zero at launch
    int *ndefer;            // [1] entries of defer, zero at launch
    int *defer;             // [N * n_tiles * 4] (tile * 4 + wave) left for the trailing pass
    float eps;
    int wait_ticks;         // bounded wait for an image's statistics, in 100 MHz ticks;
                            // < 0: never normalize in the conv pass
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, kBufferWord3);
}

// Sum over one 32-lane half of a wavefront; every lane of the half gets the
// same total.  The steps inside a 16-lane row (partner lanes xor 1 and xor 2,
// then the mirrored lane within 8 and within 16) are DPP operands of the
// additions themselves; only the step between the half's two rows is a lane
// shuffle.  The two lanes of every exchange add the same two partial sums in
// swapped order, so the totals agree bit for bit.
template <int CTRL>
__device__ __forceinline__ float dpp_from(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float half_sum_dpp(float v) {
    v += dpp_from<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp_from<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp_from<0x141>(v);  // row_half_mirror
    v += dpp_from<0x140>(v);  // row_mirror
    return v + __shfl_xor(v, 16, 64);
}

// Workgroup barrier that orders LDS only: unlike __syncthreads() it does not
// wait for the wave's outstanding global loads and stores.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// GroupNorm moments merged by Chan-Golub-LeVeque pairwise updates, in double.
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

// One-pass chain: merges one image's per-tile partials (group g's T
// partials at parts[g * stride + t]) into (mean, rstd) per group, publishes
// them, then the image's ready flag.  Run by the wave whose arrival completed
// the image (all 64 lanes).  Eight lanes per GroupNorm group (at most 8
// groups) take every eighth partial; the total count and sum, then the sum of
// squared deviations from the merged mean, are accumulated in double in a
// fixed order and summed over the eight lanes by xor shuffles (addition
// commutes exactly, so every lane holds the same bits): the result does not
// depend on which wave merges.  Partials, statistics and flag are read and
// written at device scope (sc1); the flag is stored after the statistics
// complete.
__device__ __forceinline__ void onepass_merge_image(const Partial *parts, int stride, int T, int gn_groups,
                                                               float eps, float2 *gstat, int *ready) {
    constexpr int kBatch = 16;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 3, sub = lane & 7;
    const __amdgpu_buffer_rsrc_t ps = rsrc(parts, stride * gn_groups * (int)sizeof(Partial));
    const int base = g * stride * (int)sizeof(Partial);
    float cnt[kBatch], mean[kBatch], m2[kBatch];
    auto load_batch = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            // a slot past the end reads zeros: an empty partial
            const int i = i0 + 8 * b;
            const int off = g < gn_groups && i < T ? base + i * (int)sizeof(Partial) : kOutOfRange;
            const u32x4 pt = __builtin_amdgcn_raw_buffer_load_b128(ps, off, 0, kCpolSc1);
            const unsigned int c0 = pt.x, c1 = pt.y, c2 = pt.z;
            cnt[b] = __builtin_bit_cast(float, c0);
            mean[b] = __builtin_bit_cast(float, c1);
            m2[b] = __builtin_bit_cast(float, c2);
        }
    };
    auto lane_sum = [&](double v) __attribute__((always_inline)) {
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) v += __shfl_xor(v, o);
        return v;
    };
    const bool one_batch = T <= 8 * kBatch;
    double n = 0.0, sum = 0.0;
    for (int i0 = sub; i0 < T; i0 += 8 * kBatch) {
        load_batch(i0);
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            n += (double)cnt[b];
            sum = fma((double)cnt[b], (double)mean[b], sum);
        }
    }
    n = lane_sum(n);
    const double mu = lane_sum(sum) / n;
    double dev = 0.0;
    for (int i0 = sub; i0 < T; i0 += 8 * kBatch) {
        if (!one_batch) load_batch(i0);
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const double d = (double)mean[b] - mu;
            dev += fma((double)cnt[b] * d, d, (double)m2[b]);
        }
    }
    const double var = lane_sum(dev) / n;
    if (sub == 0 && g < gn_groups) {
        const float mf = (float)mu, rf = (float)(1.0 / sqrt(var + (double)eps));
        __hip_atomic_store(&gstat[g].x, mf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&gstat[g].y, rf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (lane == 0) __hip_atomic_store(ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Winograd F(2x2, 3x3) weights of one (output channel, input channel):
// U = G g G^T with G = [1 0 0; 1/2 1/2 1/2; 1/2 -1/2 1/2; 0 0 1], in FP32.
// (Lavin and Gray, "Fast Algorithms for Convolutional Neural Networks".)
// U[u][v] goes to out[4 * v + u]: the four row positions u of one column
// position v are one 16-byte piece.
__device__ __forceinline__ void winograd_weights(const float (&g)[9], float *out) {
    float t[4][3];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        t[0][s] = g[s];
        t[1][s] = 0.5f * (g[s] + g[3 + s] + g[6 + s]);
        t[2][s] = 0.5f * (g[s] - g[3 + s] + g[6 + s]);
        t[3][s] = g[6 + s];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        out[0 * 4 + u] = t[u][0];
        out[1 * 4 + u] = 0.5f * (t[u][0] + t[u][1] + t[u][2]);
        out[2 * 4 + u] = 0.5f * (t[u][0] - t[u][1] + t[u][2]);
        out[3 * 4 + u] = t[u][2];
    }
}

template <int R, int S, int MB, int CP, int MODE, bool VEC, bool WG = false>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(MB == 1 && MODE != kOnePass && !WG ? kResWaves : 2))) void igemm_res_kernel(const float *__restrict__ x,
                                                           const float *__restrict__ w,
                                                           float *__restrict__ y, ResParams p,
                                                           ResEpilogue ep) {
    constexpr int RS = R * S;
    constexpr int NBC = kNBC;  // 32-column blocks per wave row
    constexpr int TW = kTW;    // tile width
    constexpr int KW = 32 * MB;
    constexpr int NROW = kNBR + R - 1;        // band rows one wave reads
    constexpr int TIH = kTH + R - 1;          // band rows of a workgroup tile
    constexpr int TIW = TW + S - 1;
    constexpr int PITCH = (TIW + 3) & ~3;     // LDS row pitch: whole 16-byte pieces
    constexpr int P4 = PITCH / 4;
    constexpr int XE4 = CP * TIH * P4;        // 16-byte pieces of a tile's band
    constexpr int NSLOT = (XE4 + kBlock - 1) / kBlock;
    // weight row pitch: odd (direct form, 32 lanes reading 32 output
    // channels' weight q hit 32 banks), or 16*CP + 4 (Winograd form, 16-byte
    // reads of 32 channels at a pitch of 4 mod 64 words)
    constexpr int WP = WG ? 16 * CP + 4 : (CP * RS) | 1;
    constexpr int NB = kNBR * NBC;
    constexpr int HALF = CP / 2;
    constexpr int NWAVE = kBlock / 64;
    constexpr int NGS = 16 * MB;              // kNormalize: floats of (mean, rstd) per image
    constexpr bool kStatsMode = MODE == kStats || MODE == kStatsStore || MODE == kOnePass;
    static_assert(MODE != kOnePass || MB == 1, "one-pass chain: 32 output channels, 8 groups of 4");
    static_assert(!WG || (R == 3 && S == 3 && MB == 1 && MODE != kOnePass && MODE != kPlain),
                  "Winograd form: 3x3, 32 output channels, the statistics and normalize passes");

    __shared__ __attribute__((aligned(16))) float wl[KW * WP];
    // per-channel constants, staged once: LDS reads in the epilogue count on
    // lgkmcnt, whereas per-lane global loads would count on vmcnt and make
    // the epilogue wait for the next tile's loads
    __shared__ float2 chan_bs[KW];   // (bias, scale); kPlain: (bias or 0, unused)
    __shared__ float2 chan_gb[KW];   // kNormalize: (gamma or 1, beta or 0)
    // two band buffers (the tile being multiplied and the next one) and,
    // for kNormalize, the tiles' group statistics; distinct LDS objects, so
    // the compiler never makes reads of one wait for writes to the other
    __shared__ float4 bufA4[XE4];
    __shared__ float4 bufB4[XE4];
    __shared__ float gsA[NGS];
    __shared__ float gsB[NGS];
    // kOnePass: each wave's (count, mean, M2) per group of the current tile,
    // merged by wave 0 into the tile's one partial
    __shared__ float4 wstage[MODE == kOnePass ? NWAVE * 8 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, j = lane & 31;
    const int HW = p.H * p.W;
    const int plane = p.Ho * p.Wo;

    // ---- weights, once: w[k][c][r][s] for k < cout, c < cin, zero elsewhere
    if constexpr (WG) {
        // one (output channel, input channel) per thread: its 16 Winograd
        // weights at wl[k * WP + c * 16 ..], times the channel's sigmoid
        // slope -scale * log2(e), so that the accumulators hold the
        // exponent of the sigmoid (its offset enters as a chain's start
        // value, see winograd_tile)
        for (int e = tid; e < KW * CP; e += kBlock) {
            const int k = e / CP, c = e - k * CP;
            float g[9];
#pragma unroll
            for (int q = 0; q < 9; ++q)
                g[q] = (k < p.cout && c < p.cin) ? w[((size_t)k * p.cin + c) * 9 + q] : 0.0f;
            float *uk = wl + k * WP + c * 16;
            winograd_weights(g, uk);
            const float slope = k < p.cout ? -ep.scale[k] * kLog2e : 0.0f;
#pragma unroll
            for (int q = 0; q < 16; ++q) uk[q] *= slope;
        }
    } else {
        for (int e = tid; e < KW * CP * RS; e += kBlock) {
            const int k = e / (CP * RS), q = e - k * (CP * RS);
            const int c = q / RS;
            float v = 0.0f;
            if (k < p.cout && c < p.cin) v = w[((size_t)k * p.cin + c) * RS + (q - c * RS)];
            wl[k * WP + q] = v;
        }
    }
    for (int k = tid; k < KW; k += kBlock) {
        float b = 0.0f, sc = 1.0f, ga = 1.0f, be = 0.0f;
        if (k < p.cout) {
            if (ep.bias) b = ep.bias[k];
            if constexpr (MODE != kPlain) sc = ep.scale[k];
            if constexpr (MODE == kNormalize || MODE == kOnePass) {
                if (ep.gamma) ga = ep.gamma[k];
                if (ep.beta) be = ep.beta[k];
            }
        }
        // fused modes: sigmoid((acc + b) * sc) = 1 / (1 + 2^(acc * sA + sB))
        // with sA = -sc * log2(e), sB = -b * sc * log2(e): one FMA feeds
        // the exponential
        if constexpr (MODE == kPlain)
            chan_bs[k] = make_float2(b, sc);
        else
            chan_bs[k] = make_float2(-sc * kLog2e, -b * sc * kLog2e);
        chan_gb[k] = make_float2(ga, be);
    }
    // The grid walks workgroup tiles (n, kTH output rows, TW columns); wave
    // w computes rows kNBR*w .. kNBR*w + kNBR-1 of its tile.
    const int G = gridDim.x;
    // Tile of round k for this workgroup.  Rounds that every workgroup runs
    // (k < kfull) are XCD-aware: the hardware deals consecutive workgroup ids
    // to the 8 XCDs in turn, and a bijection pb of [0, G) gives each XCD a
    // contiguous run of tiles instead, so an XCD works on neighbouring tiles,
    // whose bands share halo rows.  The last, partial round keeps the plain
    // order, which spreads its tiles over every XCD.
    const int kfull = p.units / G;
    int pb;
    {
        const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
        const int per = G >> 3, rem = G & 7;
        pb = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    }
    auto tile_of = [&](int k) __attribute__((always_inline)) {
        return k * G + (k < kfull ? pb : (int)blockIdx.x);
    };
    int u = tile_of(0);

    // ---- band prefetch through registers: pf holds this lane's 16-byte
    //      pieces of a tile's band, zero outside the image
    float4 pf[NSLOT];
    float gpf = 0.0f;
    // Tiles whose band lies wholly inside the image (VEC): a piece's offset
    // is a per-lane part (channel, band row, column), the same for every
    // tile and computed once here, plus the tile's corner, which is uniform
    // and goes in the instruction's scalar offset.  Pieces past the band or
    // past the input channels get an offset beyond every range.
    int lane_off[NSLOT];
#pragma unroll
    for (int i = 0; i < NSLOT; ++i) {
        const int f = i * kBlock + tid;
        const int cl = f / (TIH * P4), rem = f - cl * (TIH * P4);
        const int lr = rem / P4, c4 = rem - lr * P4;
        lane_off[i] = f < XE4 && cl < p.cin ? (cl * HW + lr * p.W + 4 * c4) * (int)sizeof(float) : kOutOfRange;
    }
    auto load = [&](int v) __attribute__((always_inline)) {
        const int t = v % p.n_tiles, n = v / p.n_tiles;
        const int th = t / p.n_tw, tw = t - th * p.n_tw;
        const int ih0 = th * kTH - p.pad_h, iw0 = tw * TW - p.pad_w;
        const __amdgpu_buffer_rsrc_t rs = rsrc(x + (size_t)n * p.C * HW, p.x_bytes);
        if constexpr (MODE == kNormalize) {
            const __amdgpu_buffer_rsrc_t gr = rsrc(ep.gstat + (size_t)n * ep.gn_groups, NGS * (int)sizeof(float));
            gpf = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                gr, tid < NGS ? tid * (int)sizeof(float) : kOutOfRange, 0, 0));
        }
        if constexpr (VEC) {
            if (ih0 >= 0 && ih0 + TIH <= p.H && iw0 >= 0 && iw0 + 4 * P4 <= p.W) {
                const int corner = (ih0 * p.W + iw0) * (int)sizeof(float);
                if constexpr (MODE == kOnePass) {
                    // the held accumulator set leaves no registers for the
                    // per-slot offsets: recompute them from an opaque
                    // copy of the thread id
                    int tid_o = tid;
                    asm volatile("" : "+v"(tid_o));
#pragma unroll
                    for (int i = 0; i < NSLOT; ++i) {
                        const int f = i * kBlock + tid_o;
                        const int cl = f / (TIH * P4), rem = f - cl * (TIH * P4);
                        const int lr = rem / P4, c4 = rem - lr * P4;
                        const int lo = f < XE4 && cl < p.cin ? (cl * HW + lr * p.W + 4 * c4) * (int)sizeof(float)
                                                             : kOutOfRange;
                        pf[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, lo, corner, 0));
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < NSLOT; ++i) {
                        const int lo = lane_off[i];
                        pf[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, lo, corner, 0));
                    }
                }
                return;
            }
        }
        // an opaque copy of the thread id: the per-slot offsets are the same
        // for every tile, and hoisting them out of the tile loop would keep
        // them live across the MFMA loop
        int tid_o = tid;
        asm volatile("" : "+v"(tid_o));
#pragma unroll
        for (int i = 0; i < NSLOT; ++i) {
            // piece f = (cl*TIH + lr)*P4 + c4: input columns iw0 + 4*c4 .. +3
            // of row ih0 + lr, channel cl
            const int f = i * kBlock + tid_o;
            const int cl = f / (TIH * P4), rem = f - cl * (TIH * P4);
            const int lr = rem / P4, c4 = rem - lr * P4;
            const int ih = ih0 + lr, iw = iw0 + 4 * c4;
            const bool row_ok = f < XE4 && cl < p.cin && ih >= 0 && ih < p.H;
            const int rowb = (cl * HW + ih * p.W) * (int)sizeof(float);
            if constexpr (VEC) {
                // W and iw0 multiples of 4: the piece is wholly in or out
                const int off = (row_ok && iw >= 0 && iw < p.W) ? rowb + iw * (int)sizeof(float) : kOutOfRange;
                pf[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
            } else {
                float e4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int off = (row_ok && iw + e >= 0 && iw + e < p.W) ? rowb + (iw + e) * (int)sizeof(float)
                                                                            : kOutOfRange;
                    e4[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
                }
                pf[i] = make_float4(e4[0], e4[1], e4[2], e4[3]);
            }
        }
    };
    auto commit = [&](float4 *buf4, float *gsb) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NSLOT; ++i) {
            const int f = i * kBlock + tid;
            if (f < XE4) buf4[f] = pf[i];
        }
        if constexpr (MODE == kNormalize) {
            if (tid < NGS) gsb[tid] = gpf;
        }
    };

    // The sigmoid's offset -bias * scale * log2(e) per accumulator row, the
    // start value of the chain of M[1][1]: A^T[a][1] = A^T[b][1] = 1 for
    // every output (a, b) of the block, so each output receives it once.
    floatx16 offs = {};
    if constexpr (WG) {
        lds_barrier();
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) offs[vv] = chan_bs[8 * (vv >> 2) + 4 * h + (vv & 3)].y;
    }
    // ---- MFMAs of the tile whose band is in LDS
    floatx16 accs[1][MB][NB];
    // Winograd form: lane j of a wave owns the 2x2 outputs (rows 0-1 of the
    // wave's rows, columns 2j, 2j+1), acc[0][2a + b] the output at row a,
    // column 2j + b, for the 32 channels of the MFMA layout.  Per column
    // position v of the 4x4 transform domain, and per input channel, the
    // lane forms the four B operands V[u][v] = (B^T d B)[u][v] of its 4x4
    // input patch d (B^T = [1 0 -1 0; 0 1 1 0; 0 -1 1 0; 0 1 0 -1]: the
    // column combination s[r] of two patch columns, then the same combination
    // down the rows), and four MFMA chains accumulate M[u][v] = sum over input
    // channels of U[u][v] V[u][v].  The output transform A^T M A (A^T =
    // [1 1 1 0; 0 1 -1 -1]) is then folded in per v: T_a = sum_u A^T[a][u]
    // M[u][v] and out[a][b] += A^T[b][v] T_a, in a fixed order.
    auto winograd_tile = [&](const float4 *buf4, floatx16 (&acc)[MB][NB]) __attribute__((always_inline)) {
        const float *band = reinterpret_cast<const float *>(buf4);
        // the lane's band and weight offsets, opaque so that the compiler
        // forms each channel's address in the loop instead of keeping one
        // register per channel (and buffer) across the tile loop
        int xb = (h * HALF * TIH + wave * kNBR) * PITCH + 2 * j;
        int wb = j * WP + h * HALF * 16;
        asm volatile("" : "+v"(xb), "+v"(wb));
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            // patch columns of column position v and their combination
            constexpr int kc0[4] = {0, 1, 1, 1};
            constexpr int kc1[4] = {2, 2, 2, 3};
            floatx16 mv[4];
#pragma unroll
            for (int ci = 0; ci < HALF; ++ci) {
                const float *xq = band + xb + ci * TIH * PITCH;
                float sr[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float d0 = xq[r * PITCH + kc0[v]], d1 = xq[r * PITCH + kc1[v]];
                    sr[r] = v == 0 ? d0 - d1 : v == 1 ? d0 + d1 : v == 2 ? d1 - d0 : d0 - d1;
                }
                const float vb[4] = {sr[0] - sr[2], sr[1] + sr[2], sr[2] - sr[1], sr[1] - sr[3]};
                const float4 a4 = *reinterpret_cast<const float4 *>(wl + wb + ci * 16 + v * 4);
                const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (ci == 0 && v == 1 && u == 1) {
                        mv[u] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[u], vb[u], offs, 0, 0, 0);
                    } else if (ci == 0) {
                        const floatx16 zero = {};
                        mv[u] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[u], vb[u], zero, 0, 0, 0);
                    } else {
                        mv[u] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[u], vb[u], mv[u], 0, 0, 0);
                    }
                }
            }
            // T_0 = M0 + M1 + M2, T_1 = M1 - M2 - M3
            const floatx16 t0 = (mv[0] + mv[1]) + mv[2];
            const floatx16 t1 = (mv[1] - mv[2]) - mv[3];
            if (v == 0) {
                acc[0][0] = t0;
                acc[0][2] = t1;
            } else if (v == 1) {
                acc[0][0] += t0;
                acc[0][2] += t1;
                acc[0][1] = t0;
                acc[0][3] = t1;
            } else if (v == 2) {
                acc[0][0] += t0;
                acc[0][2] += t1;
                acc[0][1] -= t0;
                acc[0][3] -= t1;
            } else {
                acc[0][1] -= t0;
                acc[0][3] -= t1;
            }
            // one column position's four chains live at a time: the fold is
            // pinned here (without the empty asm the compiler sinks it to the
            // epilogue, keeping all sixteen positions' 256 accumulator
            // registers live, and spills)
            if (v == 0)
                asm volatile("" : "+v"(acc[0][0]), "+v"(acc[0][2]));
            else
                asm volatile("" : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[0][2]), "+v"(acc[0][3]));
        }
    };
    auto mfma_tile = [&](const float4 *buf4, floatx16 (&acc)[MB][NB]) __attribute__((always_inline)) {
        if constexpr (WG) {
            winograd_tile(buf4, acc);
            return;
        }
        const float *band = reinterpret_cast<const float *>(buf4);
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[m][b][v] = 0.0f;
#pragma unroll
        for (int ci = 0; ci < HALF; ++ci) {
            // operands of one input channel (per half): the weights of the
            // lane's output channel at every tap, and the NROW band rows x
            // NBC column blocks x S shifts of the lane's input column
            float A[MB][RS];
            float B[NROW][NBC][S];
            const int cl = h * HALF + ci;
            const float *xq = band + (cl * TIH + wave * kNBR) * PITCH + j;
            const float *wq = wl + j * WP + cl * RS;
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int q = 0; q < RS; ++q) A[m][q] = wq[m * 32 * WP + q];
#pragma unroll
            for (int row = 0; row < NROW; ++row)
#pragma unroll
                for (int bc = 0; bc < NBC; ++bc)
#pragma unroll
                    for (int s = 0; s < S; ++s) B[row][bc][s] = xq[row * PITCH + bc * 32 + s];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < S; ++s)
#pragma unroll
                    for (int m = 0; m < MB; ++m)
#pragma unroll
                        for (int br = 0; br < kNBR; ++br)
#pragma unroll
                            for (int bc = 0; bc < NBC; ++bc)
                                acc[m][br * NBC + bc] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                    A[m][r * S + s], B[br + r][bc][s], acc[m][br * NBC + bc], 0, 0, 0);
        }
    };

    // ---- epilogue of tile v from acc
    auto epilogue = [&](int v, floatx16 (&acc)[MB][NB], const float2 (&gst)[MB][4]) __attribute__((always_inline)) {
        const int t = v % p.n_tiles, n = v / p.n_tiles;
        const int th = t / p.n_tw, tw = t - th * p.n_tw;
        const int oh0 = th * kTH + wave * kNBR, ow0 = tw * TW;
        const __amdgpu_buffer_rsrc_t ys = rsrc(y + (size_t)n * p.K * plane, p.y_bytes);
        // byte offset of (channel 0, row oh, column ow) for this lane's
        // pixels, or -1 where the pixel is outside the output
        int pix[NB];
#pragma unroll
        for (int br = 0; br < kNBR; ++br)
#pragma unroll
            for (int bc = 0; bc < NBC; ++bc) {
                // direct form: column block bc, lane j; Winograd form: the
                // lane's 2x2 outputs, column 2j + bc
                const int oh = oh0 + br, ow = ow0 + (WG ? 2 * j + bc : bc * 32 + j);
                pix[br * NBC + bc] = (oh < p.Ho && ow < p.Wo) ? (oh * p.Wo + ow) * (int)sizeof(float) : -1;
            }
        auto store = [&](int nb, int k, float val) __attribute__((always_inline)) {
            const int off = pix[nb] >= 0 && k < p.cout ? pix[nb] + k * plane * (int)sizeof(float) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, val), ys, off, 0, 0);
        };
        // fused modes (every accumulator row is a real channel): the lane's
        // part of the address (pixel, and 4h channels) goes in the vector
        // offset once per tile, the register's channel m*32 + 8(v/4) + v%4
        // in the scalar offset, so a store costs no VALU work.  Outside the
        // output the vector offset alone is beyond the range (y images are
        // below 1 GB, so adding the scalar offset cannot wrap).
        int vofs[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            vofs[nb] = pix[nb] >= 0 ? pix[nb] + 4 * h * plane * (int)sizeof(float) : kStoreOutOfRange;
        auto store_fast = [&](int nb, int m, int vv, float val) __attribute__((always_inline)) {
            const int so = (m * 32 + 8 * (vv >> 2) + (vv & 3)) * plane * (int)sizeof(float);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, val), ys, vofs[nb], so, 0);
        };
        // Winograd form with an even output width and y 8-byte aligned (VEC):
        // the lane's two outputs of a row, columns 2j and 2j + 1, are
        // neighbours and inside or outside the output together, so one 8-byte
        // store writes both and each store instruction covers whole lines
        auto store_pair = [&](int nb, int m, int vv, float v0, float v1) __attribute__((always_inline)) {
            const int so = (m * 32 + 8 * (vv >> 2) + (vv & 3)) * plane * (int)sizeof(float);
            const u32x2 pv = {__builtin_bit_cast(unsigned int, v0), __builtin_bit_cast(unsigned int, v1)};
            __builtin_amdgcn_raw_buffer_store_b64(pv, ys, vofs[nb], so, 0);
        };
        constexpr bool kPairStore = WG && VEC && (MODE == kStatsStore || MODE == kNormalize);
        // accumulator register v of block m holds channel m*32 + 8(v/4) +
        // 4h + v%4, local GroupNorm group lg = 8m + 2(v/4) + h (4 channels
        // per group)
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) {
                const int k = m * 32 + 8 * (vv >> 2) + 4 * h + (vv & 3);
                const float2 bs = chan_bs[k];
                if constexpr (MODE == kPlain) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) store(nb, k, acc[m][nb][vv] + bs.x);
                } else {
                    // kNormalize: out = v * gk + ck with gk = rstd * gamma,
                    // ck = beta - mean * gk
                    float gk = 1.0f, ck = 0.0f;
                    if constexpr (MODE == kNormalize) {
                        const float2 gb = chan_gb[k];
                        gk = gst[m][vv >> 2].y * gb.x;
                        ck = fmaf(-gst[m][vv >> 2].x, gk, gb.y);
                    }
                    float o[NB];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        // the Winograd form has the slope and offset in the accumulator
                        const float e2 = __builtin_amdgcn_exp2f(WG ? acc[m][nb][vv] : fmaf(acc[m][nb][vv], bs.x, bs.y));
                        const float val = __builtin_amdgcn_rcpf(1.0f + e2);
                        if constexpr (kStatsMode) acc[m][nb][vv] = val;
                        o[nb] = MODE == kNormalize ? fmaf(val, gk, ck) : val;
                        if constexpr (!kPairStore && (MODE == kStatsStore || MODE == kNormalize))
                            store_fast(nb, m, vv, o[nb]);
                    }
                    if constexpr (kPairStore) {
#pragma unroll
                        for (int nb = 0; nb < NB; nb += 2) store_pair(nb, m, vv, o[nb], o[nb + 1]);
                    }
                }
            }
        if constexpr (kStatsMode) {
            // statistics of the wave's kNBR rows of the tile, two passes over
            // the registers, no cross-wave reduction: one partial per (tile,
            // wave, group)
            const int rows_ok = max(0, min(kNBR, p.Ho - oh0));
            const int cols_ok = min(TW, p.Wo - ow0);
            const float count = 4.0f * (float)(rows_ok * cols_ok);
            const float inv = count > 0.0f ? 1.0f / count : 0.0f;
            const __amdgpu_buffer_rsrc_t ps = rsrc(ep.parts + (size_t)n * ep.gn_groups * p.parts_stride,
                                                   p.parts_bytes);
            // both passes skip the pixel masks when the wave's rows lie wholly
            // inside the output (most tiles), which the masks would otherwise
            // cost once per output and pass
            auto stats = [&](auto masked) __attribute__((always_inline)) {
                constexpr bool kMask = decltype(masked)::value;
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float sq = 0.0f;
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                            for (int uu = 0; uu < 4; ++uu) {
                                const float v = acc[m][nb][4 * q + uu];
                                sq += kMask ? (pix[nb] >= 0 ? v : 0.0f) : v;
                            }
                        const float mu = half_sum_dpp(sq) * inv;
                        float tq = 0.0f;
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
                            for (int uu = 0; uu < 4; ++uu) {
                                const float d = acc[m][nb][4 * q + uu] - mu;
                                const float dv = kMask ? (pix[nb] >= 0 ? d : 0.0f) : d;
                                tq = fmaf(dv, dv, tq);
                            }
                        }
                        const float m2 = half_sum_dpp(tq);
                        const int idx = (8 * m + 2 * q + h) * p.parts_stride + t * NWAVE + wave;
                        const u32x4 pt = {__builtin_bit_cast(unsigned int, count), __builtin_bit_cast(unsigned int, mu),
                                          __builtin_bit_cast(unsigned int, m2), 0u};
                        if constexpr (MODE == kOnePass) {
                            if (j == 0) wstage[wave * 8 + 2 * q + h] = make_float4(count, mu, m2, 0.0f);
                        } else {
                            __builtin_amdgcn_raw_buffer_store_b128(
                                pt, ps, j == 0 ? idx * (int)sizeof(Partial) : kOutOfRange, 0, 0);
                        }
                    }
            };
            if (oh0 + kNBR <= p.Ho && ow0 + TW <= p.Wo)
                stats(std::false_type{});
            else
                stats(std::true_type{});
            if constexpr (MODE == kOnePass) {
                // wave 0 merges the four waves' partials of each group (in
                // wave order, in double) into the tile's partial, stores it
                // at device scope, waits for the store to complete, then
                // counts the tile's arrival on the image; the wave whose
                // arrival completes the count merges the image
                lds_barrier();
                if (__builtin_amdgcn_readfirstlane(wave) == 0) {
                    Moments mt = {0.0, 0.0, 0.0};
                    if (lane < 8) {
#pragma unroll
                        for (int wv = 0; wv < NWAVE; ++wv) {
                            const float4 f = wstage[wv * 8 + lane];
                            mt = merge_m(mt, Moments{(double)f.x, (double)f.y, (double)f.z});
                        }
                    }
                    const u32x4 pt = {__builtin_bit_cast(unsigned int, (float)mt.n),
                                      __builtin_bit_cast(unsigned int, (float)mt.mean),
                                      __builtin_bit_cast(unsigned int, (float)mt.m2), 0u};
                    const int idx = lane * p.parts_stride + t;
                    __builtin_amdgcn_raw_buffer_store_b128(pt, ps, lane < ep.gn_groups ? idx * (int)sizeof(Partial)
                                                                                      : kOutOfRange,
                                                           0, kCpolSc1);
                    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                    int old = 0;
                    if (lane == 0) old = __hip_atomic_fetch_add(ep.arrive + n, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (__builtin_amdgcn_readfirstlane(old) == p.n_tiles - 1)
                        onepass_merge_image(ep.parts + (size_t)n * ep.gn_groups * p.parts_stride, p.parts_stride,
                                            p.n_tiles, ep.gn_groups, ep.eps, ep.gstat_out + (size_t)n * ep.gn_groups,
                                            ep.ready + n);
                }
                // v to y after the arrival, so the arrival's wait for its
                // partial store does not wait for these stores
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int vv = 0; vv < 16; ++vv)
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) store_fast(nb, m, vv, acc[m][nb][vv]);
            }
        }
    };

    // ---- kOnePass: tile v, whose v is in y, is normalized in place once
    //      its image's (mean, rstd) is published; after the bounded wait it
    //      is left as v, its wave's rows listed for the trailing pass, which
    //      applies the same fmaf(v, gk, ck) and so gives the same bits.  The
    //      check, the statistics loads and the loads of v are issued before
    //      the next band's loads, so waiting for them never waits for those.
    auto finish_check = [&](int v, int &rd, float (&gk4)[4], float (&ck4)[4]) __attribute__((always_inline)) {
        if constexpr (MODE == kOnePass) {
            const int n = v / p.n_tiles;
            rd = 0;
            if (ep.wait_ticks >= 0) {
                auto ready_now = [&]() __attribute__((always_inline)) {
                    return __builtin_amdgcn_readfirstlane(
                        __hip_atomic_load(ep.ready + n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                };
                rd = ready_now();
                if (!rd) {
                    const long long t0 = (long long)__builtin_amdgcn_s_memrealtime();
                    while (!rd && (long long)__builtin_amdgcn_s_memrealtime() - t0 < (long long)ep.wait_ticks) {
                        __builtin_amdgcn_s_sleep(4);
                        rd = ready_now();
                    }
                }
            }
            if (rd) {
                // (mean, rstd) of the lane's groups 2q + h, device-scope loads
                const __amdgpu_buffer_rsrc_t gs =
                    rsrc(ep.gstat_out + (size_t)n * ep.gn_groups, ep.gn_groups * (int)sizeof(float2));
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const unsigned long long raw = __builtin_bit_cast(
                        unsigned long long,
                        __builtin_amdgcn_raw_buffer_load_b64(gs, (2 * q + h) * (int)sizeof(float2), 0, kCpolSc1));
                    gk4[q] = __builtin_bit_cast(float, (unsigned int)(raw >> 32));   // rstd
                    ck4[q] = __builtin_bit_cast(float, (unsigned int)raw);           // mean
                }
            }
        }
    };
    float lv[NB][16];
    auto lag_load = [&](int v, int rd) __attribute__((always_inline)) {
        if constexpr (MODE == kOnePass) {
            if (rd) {
                const int t = v % p.n_tiles, n = v / p.n_tiles;
                const int th = t / p.n_tw, tw = t - th * p.n_tw;
                const int oh0 = th * kTH + wave * kNBR, ow0 = tw * TW;
                const __amdgpu_buffer_rsrc_t ys = rsrc(y + (size_t)n * p.K * plane, p.y_bytes);
#pragma unroll
                for (int br = 0; br < kNBR; ++br)
#pragma unroll
                    for (int bc = 0; bc < NBC; ++bc) {
                        const int oh = oh0 + br, ow = ow0 + bc * 32 + j;
                        const int vo = (oh < p.Ho && ow < p.Wo) ? (oh * p.Wo + ow + 4 * h * plane) * (int)sizeof(float)
                                                               : kStoreOutOfRange;
#pragma unroll
                        for (int vv = 0; vv < 16; ++vv) {
                            const int so = (8 * (vv >> 2) + (vv & 3)) * plane * (int)sizeof(float);
                            lv[br * NBC + bc][vv] =
                                __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ys, vo, so, 0));
                        }
                    }
            }
        }
    };
    auto lag_store = [&](int v, int rd, const float (&gk4)[4], const float (&ck4)[4]) __attribute__((always_inline)) {
        if constexpr (MODE == kOnePass) {
            if (rd) {
                const int t = v % p.n_tiles, n = v / p.n_tiles;
                const int th = t / p.n_tw, tw = t - th * p.n_tw;
                const int oh0 = th * kTH + wave * kNBR, ow0 = tw * TW;
                const __amdgpu_buffer_rsrc_t ys = rsrc(y + (size_t)n * p.K * plane, p.y_bytes);
                int vofs[NB];
#pragma unroll
                for (int br = 0; br < kNBR; ++br)
#pragma unroll
                    for (int bc = 0; bc < NBC; ++bc) {
                        const int oh = oh0 + br, ow = ow0 + bc * 32 + j;
                        vofs[br * NBC + bc] = (oh < p.Ho && ow < p.Wo)
                                                  ? (oh * p.Wo + ow + 4 * h * plane) * (int)sizeof(float)
                                                  : kStoreOutOfRange;
                    }
#pragma unroll
                for (int vv = 0; vv < 16; ++vv) {
                    const int k = 8 * (vv >> 2) + 4 * h + (vv & 3);
                    const float2 gb = chan_gb[k];
                    const float gk = gk4[vv >> 2] * gb.x;
                    const float ck = fmaf(-ck4[vv >> 2], gk, gb.y);
                    const int so = (8 * (vv >> 2) + (vv & 3)) * plane * (int)sizeof(float);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, fmaf(lv[nb][vv], gk, ck)),
                                                              ys, vofs[nb], so, 0);
                }
            } else if (lane == 0) {
                const int e = __hip_atomic_fetch_add(ep.ndefer, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ep.defer[e] = v * NWAVE + wave;
            }
        }
    };

    auto read_gstat = [&](const float *gsb, float2 (&gst)[MB][4]) __attribute__((always_inline)) {
        if constexpr (MODE == kNormalize) {
            const float2 *gs = reinterpret_cast<const float2 *>(gsb);
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int q = 0; q < 4; ++q) gst[m][q] = gs[8 * m + 2 * q + h];
        }
    };

    // ---- tile loop: barrier (LDS only) -> MFMAs of tile u from one buffer
    //      -> (kNormalize) its group statistics to registers -> commit tile
    //      u+G (loaded one iteration earlier) into the other buffer -> start
    //      loading tile u+2G -> epilogue of tile u.  The loads have an
    //      epilogue and a whole MFMA phase to land; the barriers order LDS
    //      only, so no wave ever waits for its output stores.  Past the last
    //      tile the indices are clamped and the work is redundant, which
    //      keeps the code free of branches around the loads.
    if (u >= p.units) return;
    float2 gst[MB][4];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) gst[m][q] = make_float2(0.0f, 0.0f);
    int k = 0;
    load(u);
    commit(bufA4, gsA);
    load(min(tile_of(1), p.units - 1));
    if constexpr (MODE == kOnePass) {
        // kOnePass: barrier -> MFMAs of tile u -> commit the next band ->
        // sigmoid, partials, arrival and stores of v of tile u -> check the
        // image of the tile kLag tiles back and load its v -> start loading
        // the band after next -> normalize that tile in place.  A
        // workgroup's tiles are a whole round of the grid apart (the host
        // sizes the grid to whole images per round), so that tile's image
        // was completed by tiles every workgroup multiplied kLag - 1 rounds
        // earlier, and its v (kLag rounds of output back) is still in the
        // last-level cache.
        int rd = 0;
        float gk4[4] = {0.0f, 0.0f, 0.0f, 0.0f}, ck4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        auto step = [&](const float4 *bcur, float4 *bnext, float *gnext) __attribute__((always_inline)) {
            lds_barrier();
            mfma_tile(bcur, accs[0]);
            commit(bnext, gnext);
            epilogue(u, accs[0], gst);
            const bool lag = k >= kLag;
            const int vl = lag ? tile_of(k - kLag) : 0;
            if (lag) {
                finish_check(vl, rd, gk4, ck4);
                lag_load(vl, rd);
            }
            load(min(tile_of(k + 2), p.units - 1));
            if (lag) lag_store(vl, rd, gk4, ck4);
            u = tile_of(++k);
            return u < p.units;
        };
        while (step(bufA4, bufB4, gsB) && step(bufB4, bufA4, gsA)) {
        }
        // the last kLag tiles
        for (int jj = max(0, k - kLag); jj < k; ++jj) {
            const int vl = tile_of(jj);
            finish_check(vl, rd, gk4, ck4);
            lag_load(vl, rd);
            lag_store(vl, rd, gk4, ck4);
        }
        return;
    }
    while (true) {
        lds_barrier();
        mfma_tile(bufA4, accs[0]);
        read_gstat(gsA, gst);
        commit(bufB4, gsB);
        load(min(tile_of(k + 2), p.units - 1));
        epilogue(u, accs[0], gst);
        u = tile_of(++k);
        if (u >= p.units) break;
        lds_barrier();
        mfma_tile(bufB4, accs[0]);
        read_gstat(gsB, gst);
        commit(bufA4, gsA);
        load(min(tile_of(k + 2), p.units - 1));
        epilogue(u, accs[0], gst);
        u = tile_of(++k);
        if (u >= p.units) break;
    }
}

// Merged (mean, rstd) of every (n, GroupNorm group) from the per-tile
// partials, in a fixed order.
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

// Clears the one-pass chain's arrival counts, ready flags and deferral
// count (a kernel, not a memset, so that captured graphs replay it).
__global__ __launch_bounds__(kBlock) void onepass_clear_kernel(int *__restrict__ sync, int count) {
    for (int i = blockIdx.x * kBlock + threadIdx.x; i < count; i += gridDim.x * kBlock) sync[i] = 0;
}

// Trailing pass of the one-pass chain: normalizes in place the rows of the
// (tile, wave) units whose wave stored v because its image's statistics were
// not published within the bounded wait.  Same arithmetic as the conv pass's
// own normalization: out = fmaf(v, gk, ck), gk = rstd * gamma,
// ck = fmaf(-mean, gk, beta).
__global__ __launch_bounds__(kBlock) void onepass_fixup_kernel(float *__restrict__ y, const int *__restrict__ defer,
                                                               const int *__restrict__ ndefer,
                                                               const float2 *__restrict__ gstat,
                                                               const float *__restrict__ gamma,
                                                               const float *__restrict__ beta, ResParams p,
                                                               int gn_groups) {
    constexpr int NWAVE = kBlock / 64;
    const int cnt = *ndefer;
    const int cpg = p.K / gn_groups;
    const int plane = p.Ho * p.Wo;
    for (int e = blockIdx.x; e < cnt; e += gridDim.x) {
        const int unit = defer[e];
        const int v = unit / NWAVE, wave = unit - v * NWAVE;
        const int t = v % p.n_tiles, n = v / p.n_tiles;
        const int th = t / p.n_tw, tw = t - th * p.n_tw;
        const int oh0 = th * kTH + wave * kNBR, ow0 = tw * kTW;
        float *yn = y + (size_t)n * p.K * plane;
        for (int i = threadIdx.x; i < p.K * kNBR * kTW; i += kBlock) {
            const int k = i / (kNBR * kTW), rc = i - k * (kNBR * kTW);
            const int oh = oh0 + rc / kTW, ow = ow0 + rc % kTW;
            if (oh < p.Ho && ow < p.Wo) {
                const float2 st = gstat[(size_t)n * gn_groups + k / cpg];
                const float ga = gamma ? gamma[k] : 1.0f, be = beta ? beta[k] : 0.0f;
                const float gk = st.y * ga;
                const float ck = fmaf(-st.x, gk, be);
                float *o = yn + (size_t)k * plane + (size_t)oh * p.Wo + ow;
                *o = fmaf(*o, gk, ck);
            }
        }
    }
}

// ---- host side

constexpr int kMaxResLds = 80 * 1024;  // keep at least two workgroups per CU
constexpr int kMaxDevices = 64;

template <int R, int S, int MB, int CP, int MODE, bool WG>
constexpr int res_lds_bytes() {
    return 4 * (32 * MB * (WG ? 16 * CP + 4 : (CP * R * S) | 1) +
                2 * (CP * (kTH + R - 1) * ((kTW + S - 1 + 3) & ~3) + 16 * MB)) +
           2 * 8 * 32 * MB + (MODE == kOnePass ? 16 * (kBlock / 64) * 8 : 0);
}

// The fused statistics and normalize passes of a 3x3 conv with one block of
// 32 output channels multiply in the Winograd form.
constexpr bool kResWinograd = true;

// one GroupNorm partial per (tile of kTH rows x kTW columns, wave, group)
int res_parts_per_group(const gconv_desc *d) {
    const int n_tw = (d->Wo + kTW - 1) / kTW;
    return (kBlock / 64) * n_tw * ((d->Ho + kTH - 1) / kTH);
}

// tiles (kTH rows x kTW columns) per image
int res_tiles(const gconv_desc *d) { return ((d->Wo + kTW - 1) / kTW) * ((d->Ho + kTH - 1) / kTH); }

ResParams make_params(const gconv_desc *d, int gn_groups) {
    ResParams p;
    p.C = d->C; p.H = d->H; p.W = d->W; p.K = d->K; p.Ho = d->Ho; p.Wo = d->Wo;
    p.pad_h = d->pad_h; p.pad_w = d->pad_w;
    p.cin = d->cin; p.cout = d->cout;
    p.n_tw = (d->Wo + kTW - 1) / kTW;
    p.parts_stride = res_parts_per_group(d);
    p.n_tiles = p.n_tw * ((d->Ho + kTH - 1) / kTH);
    p.units = d->N * p.n_tiles;
    p.x_bytes = (int)((size_t)d->C * d->H * d->W * sizeof(float));
    p.y_bytes = (int)((size_t)d->K * d->Ho * d->Wo * sizeof(float));
    p.parts_bytes = (int)((size_t)gn_groups * res_parts_per_group(d) * sizeof(Partial));
    return p;
}

// 16-byte band loads; in the fused modes also y 8-byte aligned, for the
// paired stores of the Winograd form (W % 4 == 0 and pad_w % 4 == 0 make the
// output width of a 3x3 conv even)
bool res_vec(const gconv_desc *d, const float *x, const float *y, bool fused) {
    return (d->W % 4 == 0) && (d->pad_w % 4 == 0) && (((uintptr_t)x & 15u) == 0) &&
           (!fused || ((uintptr_t)y & 7u) == 0);
}

int res_mb(const gconv_desc *d) { return d->cout > 32 ? 2 : 1; }
int res_cp(const gconv_desc *d) { return d->cin <= 4 ? 4 : 8; }

template <int R, int S, int MB, int CP, int MODE, bool VEC, bool WG = false>
hipError_t launch_t(const ResParams &p, const float *x, const float *w, float *y, const ResEpilogue &ep,
                    hipStream_t st) {
    static_assert(res_lds_bytes<R, S, MB, CP, MODE, WG>() <= kMaxResLds, "LDS budget");
    auto kern = igemm_res_kernel<R, S, MB, CP, MODE, VEC, WG>;
    // resident workgroups per device for this kernel: queried once per
    // device and kept (the query costs host time on every launch otherwise)
    static std::atomic<int> capacity[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return hipErrorInvalidDevice;
    int cap = dev < kMaxDevices ? capacity[dev].load(std::memory_order_relaxed) : 0;
    if (cap == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return hipErrorInvalidDevice;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBlock, 0) != hipSuccess || per_cu < 1)
            per_cu = 1;
        cap = cus * per_cu;
        if (dev < kMaxDevices) capacity[dev].store(cap, std::memory_order_relaxed);
    }
    long long want = cap;
    if constexpr (MODE == kOnePass) {
        // whole images per round of the grid, so that a workgroup's previous
        // tile belongs to an image every workgroup has finished multiplying
        // (an image of more tiles than the capacity still computes
        // correctly: its tiles then wait and leave more to the trailing pass)
        const long long per_round = cap / p.n_tiles;
        if (per_round >= 1) want = per_round * p.n_tiles;
    }
    const int grid = (int)(p.units < want ? p.units : want);
    clear_stale_launch_error();
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlock), 0, st, x, w, y, p, ep);
    return hipGetLastError();
}

template <int MODE, bool VEC>
hipError_t launch_mode_v(const gconv_desc *d, const ResParams &p, const float *x, const float *w, float *y,
                         const ResEpilogue &ep, hipStream_t st) {
    const int mb = res_mb(d), cp = res_cp(d);
    if constexpr (MODE == kOnePass) {
        // one accumulator block only (igemm_res_onepass_supported)
        if (mb != 1) return hipErrorInvalidValue;
        if (d->R == 3 && d->S == 3)
            return cp == 4 ? launch_t<3, 3, 1, 4, MODE, VEC>(p, x, w, y, ep, st)
                           : launch_t<3, 3, 1, 8, MODE, VEC>(p, x, w, y, ep, st);
        if (d->R == 1 && d->S == 1)
            return cp == 4 ? launch_t<1, 1, 1, 4, MODE, VEC>(p, x, w, y, ep, st)
                           : launch_t<1, 1, 1, 8, MODE, VEC>(p, x, w, y, ep, st);
        return hipErrorInvalidValue;
    } else {
        if (d->R == 3 && d->S == 3) {
            if constexpr (kResWinograd && MODE != kPlain) {
                if (mb == 1)
                    return cp == 4 ? launch_t<3, 3, 1, 4, MODE, VEC, true>(p, x, w, y, ep, st)
                                   : launch_t<3, 3, 1, 8, MODE, VEC, true>(p, x, w, y, ep, st);
            }
            if (mb == 1)
                return cp == 4 ? launch_t<3, 3, 1, 4, MODE, VEC>(p, x, w, y, ep, st)
                               : launch_t<3, 3, 1, 8, MODE, VEC>(p, x, w, y, ep, st);
            return cp == 4 ? launch_t<3, 3, 2, 4, MODE, VEC>(p, x, w, y, ep, st)
                           : launch_t<3, 3, 2, 8, MODE, VEC>(p, x, w, y, ep, st);
        }
        if (d->R == 1 && d->S == 1) {
            if (mb == 1)
                return cp == 4 ? launch_t<1, 1, 1, 4, MODE, VEC>(p, x, w, y, ep, st)
                               : launch_t<1, 1, 1, 8, MODE, VEC>(p, x, w, y, ep, st);
            return cp == 4 ? launch_t<1, 1, 2, 4, MODE, VEC>(p, x, w, y, ep, st)
                           : launch_t<1, 1, 2, 8, MODE, VEC>(p, x, w, y, ep, st);
        }
        return hipErrorInvalidValue;
    }
}

template <int MODE>
hipError_t launch_mode(const gconv_desc *d, const ResParams &p, const float *x, const float *w, float *y,
                       const ResEpilogue &ep, hipStream_t st) {
    return res_vec(d, x, y, MODE != kPlain) ? launch_mode_v<MODE, true>(d, p, x, w, y, ep, st)
                         : launch_mode_v<MODE, false>(d, p, x, w, y, ep, st);
}

}  // namespace

bool igemm_res_supported(const gconv_desc *d) {
    // buffer offsets are signed 32-bit: one image of x and of y (and the
    // partials of one image) must stay below 2 GB
    const long long lim = 0x7fffffffLL - 64;
    return d->groups == 1 && d->stride_h == 1 && d->stride_w == 1 && d->dil_h == 1 && d->dil_w == 1 && d->cin >= 4 && d->cin <= 8 &&
           d->cout >= 8 && d->cout <= 64 && ((d->R == 3 && d->S == 3) || (d->R == 1 && d->S == 1)) &&
           (long long)d->C * d->H * d->W * 4 < lim && (long long)d->K * d->Ho * d->Wo * 4 < lim;
}

bool igemm_res_fused_supported(const gconv_desc *d, int gn_groups) {
    return igemm_res_supported(d) && d->cout % (32 * res_mb(d)) == 0 && d->K / gn_groups == 4 &&
           (long long)d->K * d->Ho * d->Wo * (long long)sizeof(float) < kStoreOutOfRange &&
           (long long)gn_groups * res_parts_per_group(d) * (long long)sizeof(Partial) < 0x7fffffffLL - 64;
}

int igemm_res_parts_per_group(const gconv_desc *d) { return res_parts_per_group(d); }

bool igemm_res_onepass_supported(const gconv_desc *d, int gn_groups) {
    // one accumulator block of 32 output channels (8 groups of 4); the
    // deferral list indexes (tile, wave) units with an int
    return igemm_res_fused_supported(d, gn_groups) && res_mb(d) == 1 && d->cout == 32 &&
           (long long)d->N * (kBlock / 64) * res_tiles(d) < 0x7fffffffLL;
}

size_t igemm_res_onepass_sync_ints(const gconv_desc *d) {
    return 2 * (size_t)d->N + 1 + (size_t)d->N * (size_t)(kBlock / 64) * (size_t)res_tiles(d);
}

hipError_t launch_igemm_res(const gconv_desc *d, const float *x, const float *w, const float *bias, float *y,
                            hipStream_t st) {
    if (!igemm_res_supported(d)) return hipErrorInvalidValue;
    ResEpilogue ep{};
    ep.bias = bias;
    return launch_mode<kPlain>(d, make_params(d, 1), x, w, y, ep, st);
}

hipError_t launch_igemm_res_stats(const gconv_desc *d, const float *x, const float *w, float *y, bool store,
                                  const FusedEpilogue &fe, hipStream_t st) {
    if (!igemm_res_fused_supported(d, fe.gn_groups)) return hipErrorInvalidValue;
    const ResParams p = make_params(d, fe.gn_groups);
    ResEpilogue ep{};
    ep.bias = fe.bias;
    ep.scale = fe.scale;
    ep.parts = fe.parts;
    ep.gn_groups = fe.gn_groups;
    if (store) return launch_mode<kStatsStore>(d, p, x, w, y, ep, st);
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

hipError_t launch_igemm_res_onepass(const gconv_desc *d, const float *x, const float *w, float *y,
                                    const FusedEpilogue &fe, float2 *gstat, int *sync, const float *gamma,
                                    const float *beta, float eps, int wait_us, hipStream_t st) {
    if (!igemm_res_onepass_supported(d, fe.gn_groups)) return hipErrorInvalidValue;
    const ResParams p = make_params(d, fe.gn_groups);
    const int nsync = 2 * d->N + 1;
    clear_stale_launch_error();
    hipLaunchKernelGGL(onepass_clear_kernel, dim3((unsigned)((nsync + kBlock - 1) / kBlock < 1024 ? (nsync + kBlock - 1) / kBlock : 1024)),
                       dim3(kBlock), 0, st, sync, nsync);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ResEpilogue ep{};
    ep.bias = fe.bias;
    ep.scale = fe.scale;
    ep.parts = fe.parts;
    ep.gamma = gamma;
    ep.beta = beta;
    ep.gn_groups = fe.gn_groups;
    ep.gstat_out = gstat;
    ep.arrive = sync;
    ep.ready = sync + d->N;
    ep.ndefer = sync + 2 * d->N;
    ep.defer = sync + nsync;
    ep.eps = eps;
    // the wait in ticks of the 100 MHz real-time counter
    ep.wait_ticks = wait_us < 0 ? -1 : (wait_us > 10000000 ? 1000000000 : wait_us * 100);
    e = launch_mode<kOnePass>(d, p, x, w, y, ep, st);
    if (e != hipSuccess) return e;
    const int units = p.units * (kBlock / 64);
    clear_stale_launch_error();
    hipLaunchKernelGGL(onepass_fixup_kernel, dim3((unsigned)(units < 1024 ? units : 1024)), dim3(kBlock), 0, st, y,
                       ep.defer, ep.ndefer, (const float2 *)gstat, gamma, beta, p, fe.gn_groups);
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
    return launch_mode<kNormalize>(d, make_params(d, fe.gn_groups), x, w, y, ep, st);
}

}  // namespace gconv
