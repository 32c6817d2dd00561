// k_igemm.hip -- FP32 MFMA implicit GEMM for dense and wide-group
// convolution (dilation 1, any padding; stride 1, and stride 2 at 1x1 and
// 3x3 in the DMA-staged kernel).
//
// The implicit-GEMM view of the POPCORNBENCH traces ("Kimi-K2.6 l2_p21",
// GEMM framing; "Kimi-K2.6 l1_p62", output-channel blocking): per group,
//   D[k][p] = sum_q Wt[k][q] * X[q][p],   q = (c, r, s),  p = (oh, ow),
// with Wt the weights viewed as [K][C/G*R*S] and X gathered on the fly from
// an LDS input band (no im2col buffer).
//
// gfx950 mapping:
//  - v_mfma_f32_32x32x2f32: A = 32 output channels x 2 reduction slots,
//    B = 2 reduction slots x 32 pixels along W.  The two reduction slots are
//    the two 32-lane halves of the wave; each half walks its own half of the
//    input-channel chunk, so every tap offset (r, s) is a compile-time LDS
//    immediate for both operands.
//  - Workgroup = 4 waves; wave w owns NBR output rows x (32*NBC) columns x
//    (32*MB) output channels, i.e. MB*NBR*NBC accumulator blocks of 16
//    floats per lane.  The workgroup tile is (4*NBR) x (32*NBC) pixels.
//  - Input channels are streamed through LDS CC at a time: the input band
//    [CC][TH+R-1][TW+S-1] and the weights [32*MB][CC*R*S] (row pitch made
//    odd so that the 32 lanes reading 32 output channels hit 32 banks).
//  - Output: lane (half h, column j) holds rows i = 8*(v/4) + 4*h + v%4 of
//    each 32x32 block; every store instruction writes two runs of 32
//    consecutive pixels of two channels.
//  - The fused variant applies (acc + bias) * scale -> sigmoid before the
//    store and writes, per workgroup and GroupNorm group of 4 channels, the
//    count, mean and M2 of its values (two passes over the registers).
#include "dev_common.h"
#include "internal.h"

namespace gconv {
namespace {

constexpr int kBlock = 256;
constexpr int kBatch = 8;  // global loads in flight per lane while staging
constexpr int kNBR = 2;  // output rows per wave
constexpr int kNBC = 2;  // 32-column blocks per wave row
constexpr int kTH = 4 * kNBR;
constexpr int kTW = 32 * kNBC;

typedef float floatx16 __attribute__((ext_vector_type(16)));

struct IgParams {
    int C, H, W, K, Ho, Wo;
    int pad_h, pad_w;  // zero padding above/below and left/right
    int cin, cout;
    int n_kb;          // output-channel blocks of 32*MB per group
    int n_tw;          // column tiles per image
    int n_tiles;       // spatial tiles per image
    int pitch;         // LDS row pitch of the input band (floats)
    int vec;           // W, pad multiples of 4 and x 16-byte aligned: 16-byte band loads
    int G;             // groups
    int n_wg;          // workgroups of the DMA kernel's 1-D grid: N * G * n_tiles * n_kb
    int st;            // stride (both axes): 1, or 2 for the DMA kernel at 1x1 and 3x3
    int nbc;           // 32-column blocks per wave row of the DMA kernel (1 on outputs at most 32 wide)
    int nbr;           // output rows per wave of the DMA kernel (1 at stride 2 and on small grids)
};

template <int R, int S, int MB, int CC, bool FUSED>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void igemm_kernel(const float *__restrict__ x,
                                                       const float *__restrict__ w,
                                                       const float *__restrict__ bias,
                                                       float *__restrict__ y, IgParams p,
                                                       FusedEpilogue ep) {
    constexpr int RS = R * S;
    constexpr int KW = 32 * MB;
    constexpr int TIH = kTH + R - 1;
    constexpr int TIW = kTW + S - 1;
    constexpr int NB = kNBR * kNBC;
    constexpr int HALF = CC / 2;

    extern __shared__ float4 lds4[];
    float *xin = reinterpret_cast<float *>(lds4);   // [CC][TIH][pitch]
    float *wl = xin + CC * TIH * p.pitch;            // [KW][CC*RS], pitch WP

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, j = lane & 31;
    const int n = blockIdx.z;
    const int th = blockIdx.x / p.n_tw, tw = blockIdx.x - th * p.n_tw;
    const int oh0 = th * kTH, ow0 = tw * kTW;
    const int g = blockIdx.y / p.n_kb, kb = blockIdx.y - g * p.n_kb;
    const int kg0 = kb * KW;                 // first output channel within the group
    const int k0 = g * p.cout + kg0;         // first global output channel
    const int kvalid = min(KW, p.cout - kg0);

    const size_t HW = (size_t)p.H * p.W;
    const float *xg = x + ((size_t)n * p.C + (size_t)g * p.cin) * HW;
    const float *wg = w + (size_t)k0 * p.cin * RS;

    floatx16 acc[MB][NB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[m][b][v] = 0.0f;

    // Staging of one channel chunk into LDS.  Each lane issues kBatch
    // independent global loads before writing any of them, so a chunk costs
    // a few load round trips rather than one per element.
    constexpr int XE = CC * TIH * TIW;                  // input elements per chunk
    constexpr int WE = KW * CC * RS;                    // weight elements per chunk
    // weights stay [k][c][r][s] in LDS with an odd row pitch WP: the fill
    // writes consecutive floats and the 32 lanes reading 32 consecutive
    // output channels land on 32 different banks
    constexpr int WP = (CC * RS) | 1;
    for (int c0 = 0; c0 < p.cin; c0 += CC) {
        __syncthreads();  // previous chunk fully consumed
        for (int base = tid; base < XE; base += kBatch * kBlock) {
            float v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int e = base + u * kBlock;
                const int row = e / TIW, col = e - row * TIW;  // row = cl * TIH + lr
                const int cl = row / TIH, lr = row - cl * TIH;
                const int ih = oh0 - p.pad_h + lr, iw = ow0 - p.pad_w + col;
                v[u] = 0.0f;
                if (e < XE && c0 + cl < p.cin && ih >= 0 && ih < p.H && iw >= 0 && iw < p.W)
                    v[u] = xg[(size_t)(c0 + cl) * HW + (size_t)ih * p.W + iw];
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int e = base + u * kBlock;
                const int row = e / TIW, col = e - row * TIW;
                if (e < XE) xin[row * p.pitch + col] = v[u];
            }
        }
        // weights of output channels k0 .. k0+KW-1 and channels c0 .. c0+CC-1
        for (int base = tid; base < WE; base += kBatch * kBlock) {
            float v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int e = base + u * kBlock;
                const int k = e / (CC * RS), rem = e - k * (CC * RS);  // rem = cl * RS + t
                const int cl = rem / RS;
                v[u] = 0.0f;
                if (e < WE && k < kvalid && c0 + cl < p.cin)
                    v[u] = wg[(size_t)k * p.cin * RS + (size_t)c0 * RS + rem];
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int e = base + u * kBlock;
                const int k = e / (CC * RS), rem = e - k * (CC * RS);
                if (e < WE) wl[k * WP + rem] = v[u];
            }
        }
        __syncthreads();

#pragma unroll
        for (int ci = 0; ci < HALF; ++ci) {
            const int cl = h * HALF + ci;
            const float *xb = xin + (cl * TIH + wave * kNBR) * p.pitch + j;
            const float *wb = wl + j * WP + cl * RS;
#pragma unroll
            for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    float a[MB], b[NB];
#pragma unroll
                    for (int m = 0; m < MB; ++m) a[m] = wb[m * 32 * WP + r * S + s];
#pragma unroll
                    for (int br = 0; br < kNBR; ++br)
#pragma unroll
                        for (int bc = 0; bc < kNBC; ++bc)
                            b[br * kNBC + bc] = xb[(br + r) * p.pitch + bc * 32 + s];
#pragma unroll
                    for (int m = 0; m < MB; ++m)
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[m][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[m], b[nb], acc[m][nb], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue
    const size_t plane = (size_t)p.Ho * p.Wo;
    float *yb = y + ((size_t)n * p.K + k0) * plane;
    if constexpr (!FUSED) {
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
                        if (k < kvalid) {
                            float o = acc[m][br * kNBC + bc][v];
                            if (bias) o += bias[k0 + k];
                            yb[(size_t)k * plane + (size_t)oh * p.Wo + ow] = o;
                        }
                    }
                }
            }
    } else {
        // Every output channel of the block is valid here (cout % (32*MB) == 0)
        // and a GroupNorm group is 4 channels: rows 8q + 4h + (0..3) of a
        // 32x32 block, i.e. local group lg = 8m + 2q + h.
        __shared__ float red[4][8 * MB];
        __shared__ float mean_s[8 * MB];
        const int rows_ok = min(kTH, p.Ho - oh0), cols_ok = min(kTW, p.Wo - ow0);
        const float count = 4.0f * (float)(rows_ok * cols_ok);
        float s1[MB][4];
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) s1[m][q] = 0.0f;
#pragma unroll
        for (int m = 0; m < MB; ++m) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int k = k0 + m * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                const float bk = ep.bias[k], sk = ep.scale[k];
#pragma unroll
                for (int br = 0; br < kNBR; ++br)
#pragma unroll
                    for (int bc = 0; bc < kNBC; ++bc) {
                        const int oh = oh0 + wave * kNBR + br, ow = ow0 + bc * 32 + j;
                        const bool ok = oh < p.Ho && ow < p.Wo;
                        const float val = sigmoidf((acc[m][br * kNBC + bc][v] + bk) * sk);
                        acc[m][br * kNBC + bc][v] = val;
                        if (ok) {
                            yb[(size_t)(k - k0) * plane + (size_t)oh * p.Wo + ow] = val;
                            s1[m][v >> 2] += val;
                        }
                    }
            }
        }
        // pass 1: tile means per local group
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float t = half_wave_sum(s1[m][q]);
                if (j == 0) red[wave][8 * m + 2 * q + h] = t;
            }
        __syncthreads();
        if (tid < 8 * MB) mean_s[tid] = ((red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid])) / count;
        __syncthreads();
        // pass 2: squared deviations from the tile mean
        float s2[MB][4];
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float mu = mean_s[8 * m + 2 * q + h];
                float t = 0.0f;
#pragma unroll
                for (int br = 0; br < kNBR; ++br)
#pragma unroll
                    for (int bc = 0; bc < kNBC; ++bc) {
                        const int oh = oh0 + wave * kNBR + br, ow = ow0 + bc * 32 + j;
                        if (oh < p.Ho && ow < p.Wo) {
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                const float dv = acc[m][br * kNBC + bc][4 * q + u] - mu;
                                t = fmaf(dv, dv, t);
                            }
                        }
                    }
                s2[m][q] = t;
            }
        __syncthreads();  // red[] reused
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float t = half_wave_sum(s2[m][q]);
                if (j == 0) red[wave][8 * m + 2 * q + h] = t;
            }
        __syncthreads();
        if (tid < 8 * MB) {
            const int gg = k0 / 4 + tid;  // global GroupNorm group (4 channels each)
            Partial pt;
            pt.count = count;
            pt.mean = mean_s[tid];
            pt.m2 = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
            pt.pad = 0.0f;
            ep.parts[((size_t)n * ep.gn_groups + gg) * ep.parts_per_group + blockIdx.x] = pt;
        }
    }
}

// ---------------------------------------------------------------------------
// Pipelined kernel for the plain convolution (no fused epilogue).  Same MFMA
// mapping and tile as igemm_kernel; what changes is the staging of the
// channel chunks, which there leaves the matrix pipe idle for about a
// quarter of the time:
//  - two LDS buffers per operand (input band, weights), statically
//    allocated so the compiler sees that reads of one never alias the DMA
//    into the other;
//  - chunk c+1 goes from global memory straight into the free buffer (buffer
//    loads with the LDS bit: lane l of a wave writes its 4 or 16 bytes at the
//    instruction's LDS base + l*size, and an out-of-range offset, used for
//    padding and missing channels, writes zero) while chunk c is multiplied;
//    one wait and one LDS-only barrier per chunk;
//  - no registers hold the next chunk and no VALU work copies it into LDS;
//  - weights sit in LDS as [tap][output channel], so the 32 lanes reading 32
//    output channels of one tap read 32 consecutive words.

constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer access, gfx9 family
// output-channel blocks per workgroup of the plain kernel: with two, the
// MFMA loop's operands spill at two waves per SIMD (measured slower)
constexpr int kPlainMB = 1;
constexpr int kOutOfRange = 0x7fffffff;
// below this many workgroups the DMA kernel takes 4-row tiles (two per CU)
constexpr long long kSmallGridWorkgroups = 512;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, kBufferWord3);
}

// Workgroup barrier that orders LDS only: unlike __syncthreads() it does not
// wait for the wave's outstanding global loads.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

typedef __attribute__((address_space(3))) void lds_void_t;

// ST: stride (1 or 2, both axes).  At stride 2 the band holds the input rows
// ST*oh0 - pad ... of the tile, and each row's columns in two phases, even
// input columns first, then odd ones (HW2 of each): output column ow at tap s
// reads input column 2*ow + s, which is phase s%2, position ow + s/2, so the
// 32 lanes of a block still read 32 consecutive LDS words.  Stride 2 takes
// the 4-byte (gather) band loads.
// NBR output rows per wave (a 4*NBR-row tile): 2, or 1 at stride 2 and on
// grids too small to fill the chip.
template <int R, int S, int MB, int CC, bool VEC, int ST, int NBC, int NBR>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void igemm_dma_kernel(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ y, IgParams p) {
    static_assert(ST == 1 || (ST == 2 && !VEC), "stride 2 gathers its band with 4-byte loads");
    constexpr int RS = R * S;
    constexpr int KW = 32 * MB;
    constexpr int TH = 4 * NBR;
    // NBC 32-column blocks per wave row (1 on outputs at most 32 wide)
    constexpr int TW = 32 * NBC;
    constexpr int TIH = ST * (TH - 1) + R;
    constexpr int HW2 = TW + (S - 1) / 2;   // stride 2: columns per phase
    constexpr int TIW = ST == 1 ? TW + S - 1 : 2 * HW2;
    constexpr int PITCH = (TIW + 3) & ~3;    // band row pitch: whole 16-byte pieces
    constexpr int P4 = PITCH / 4;
    constexpr int XE4 = CC * TIH * P4;       // 16-byte pieces of a chunk's band
    constexpr int XI = (XE4 + 63) / 64;      // band DMA instructions (16-byte pieces)
    constexpr int XE = XE4 * 4;
    constexpr int XI1 = (XE + 63) / 64;      // band DMA instructions (4-byte elements)
    constexpr int WE = CC * RS * KW;         // weight words of a chunk, [q][KW]
    constexpr int WI = (WE + 63) / 64;       // weight DMA instructions
    constexpr int NB = NBR * NBC;
    constexpr int HALF = CC / 2;
    constexpr int NWAVE = kBlock / 64;

    // buffers padded to whole DMA instructions (idle lanes write zeros there)
    __shared__ float4 xA4[XI * 64];
    __shared__ float4 xB4[XI * 64];
    __shared__ float wA[WI * 64];
    __shared__ float wB[WI * 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, j = lane & 31;
    // Workgroup -> work item, XCD-aware.  The hardware deals consecutive
    // workgroup ids to the 8 XCDs in turn, so XCD i receives ids i, i + 8,
    // i + 16, ...  Each XCD is given a contiguous run of work items instead,
    // ordered (n, group, tile row, tile column, channel block) with the
    // channel block fastest: the blocks of one tile, and the tiles whose
    // bands share halo rows, then run on one XCD close in time and its L2
    // serves the rows they have in common.
    const int L = blockIdx.x;
    const int xcd = L & 7, slot = L >> 3;
    const int per = p.n_wg >> 3, rem = p.n_wg & 7;
    const int item = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    const int kb = item % p.n_kb;
    const int t1 = item / p.n_kb;
    const int tile = t1 % p.n_tiles;
    const int t2 = t1 / p.n_tiles;
    const int g = t2 % p.G, n = t2 / p.G;
    const int th = tile / p.n_tw, tw = tile - th * p.n_tw;
    const int oh0 = th * TH, ow0 = tw * TW;
    const int kg0 = kb * KW;
    const int k0 = g * p.cout + kg0;
    const int kvalid = min(KW, p.cout - kg0);
    const int HW = p.H * p.W;
    const __amdgpu_buffer_rsrc_t xs = make_rsrc(x + ((size_t)n * p.C + (size_t)g * p.cin) * HW,
                                                p.cin * HW * (int)sizeof(float));
    const __amdgpu_buffer_rsrc_t ws = make_rsrc(w + (size_t)k0 * p.cin * RS, kvalid * p.cin * RS * (int)sizeof(float));
    const int nchunks = (p.cin + CC - 1) / CC;

    // DMA of chunk c into (xb4, wb): wave w issues instructions w, w+4, ...
    auto dma = [&](int c, float4 *xb4, float *wb) __attribute__((always_inline)) {
        const int c0 = c * CC;
        if constexpr (VEC) {
            for (int ii = wave; ii < XI; ii += NWAVE) {
                const int f = ii * 64 + lane;
                const int cl = f / (TIH * P4), rem = f - cl * (TIH * P4);
                const int lr = rem / P4, c4 = rem - lr * P4;
                const int ih = oh0 - p.pad_h + lr, iw = ow0 - p.pad_w + 4 * c4;
                const bool ok = f < XE4 && c0 + cl < p.cin && ih >= 0 && ih < p.H && iw >= 0 && iw < p.W;
                const int off = ok ? ((c0 + cl) * HW + ih * p.W + iw) * (int)sizeof(float) : kOutOfRange;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xs, (lds_void_t *)(xb4 + ii * 64), 16, off, 0, 0, 0);
            }
        } else {
            float *xb = reinterpret_cast<float *>(xb4);
            for (int ii = wave; ii < XI1; ii += NWAVE) {
                const int e = ii * 64 + lane;
                const int row = e / PITCH, col = e - row * PITCH;  // row = cl * TIH + lr
                const int cl = row / TIH, lr = row - cl * TIH;
                const int ih = ST * oh0 - p.pad_h + lr;
                int iw;
                if constexpr (ST == 1) {
                    iw = ow0 - p.pad_w + col;
                } else {
                    // band column col: phase col / HW2, position col % HW2
                    // (columns past both phases read zero)
                    const int ph = col >= HW2 ? 1 : 0;
                    iw = col < 2 * HW2 ? ST * ow0 - p.pad_w + 2 * (col - ph * HW2) + ph : -1;
                }
                const bool ok = e < XE && c0 + cl < p.cin && ih >= 0 && ih < p.H && iw >= 0 && iw < p.W;
                const int off = ok ? ((c0 + cl) * HW + ih * p.W + iw) * (int)sizeof(float) : kOutOfRange;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xs, (lds_void_t *)(xb + ii * 64), 4, off, 0, 0, 0);
            }
        }
        for (int ii = wave; ii < WI; ii += NWAVE) {
            const int e = ii * 64 + lane;            // e = q * KW + k
            const int q = e / KW, k = e - q * KW;    // q = cl * RS + t
            const int cl = q / RS;
            const bool ok = e < WE && k < kvalid && c0 + cl < p.cin;
            const int off = ok ? (k * p.cin * RS + c0 * RS + q) * (int)sizeof(float) : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ws, (lds_void_t *)(wb + ii * 64), 4, off, 0, 0, 0);
        }
    };

    // Full chunks (c0 + CC <= cin): the part of every DMA offset that
    // depends on the lane and the instruction is the same for every chunk;
    // the chunk adds c0*HW floats (band) or c0*RS floats (weights), which go
    // in the instruction's scalar offset.  The per-lane offsets are computed
    // once here, so a full chunk's DMA costs no vector instructions.  An
    // element outside the image or past kvalid gets an offset beyond every
    // range (kOutOfRange plus a scalar offset below 2^31 does not wrap).
    // band instructions per wave: 16-byte pieces (VEC) or 4-byte elements
    constexpr int XPW = VEC ? (XI + NWAVE - 1) / NWAVE : (XI1 + NWAVE - 1) / NWAVE;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int xo[XPW];
#pragma unroll
    for (int t = 0; t < XPW; ++t) {
        const int ii = wv + t * NWAVE;
        if constexpr (VEC) {
            const int f = ii * 64 + lane;
            const int cl = f / (TIH * P4), rem = f - cl * (TIH * P4);
            const int lr = rem / P4, c4 = rem - lr * P4;
            const int ih = oh0 - p.pad_h + lr, iw = ow0 - p.pad_w + 4 * c4;
            const bool ok = f < XE4 && ih >= 0 && ih < p.H && iw >= 0 && iw < p.W;  // then cl < CC
            xo[t] = ok ? (cl * HW + ih * p.W + iw) * (int)sizeof(float) : kOutOfRange;
        } else {
            // element e of the band, as in dma() but without the chunk
            const int e = ii * 64 + lane;
            const int row = e / PITCH, col = e - row * PITCH;  // row = cl * TIH + lr
            const int cl = row / TIH, lr = row - cl * TIH;
            const int ih = ST * oh0 - p.pad_h + lr;
            int iw;
            if constexpr (ST == 1) {
                iw = ow0 - p.pad_w + col;
            } else {
                const int ph = col >= HW2 ? 1 : 0;
                iw = col < 2 * HW2 ? ST * ow0 - p.pad_w + 2 * (col - ph * HW2) + ph : -1;
            }
            const bool ok = e < XE && ih >= 0 && ih < p.H && iw >= 0 && iw < p.W;  // then cl < CC
            xo[t] = ok ? (cl * HW + ih * p.W + iw) * (int)sizeof(float) : kOutOfRange;
        }
    }
    // weights: element e = ii*64 + lane of a chunk is (q, k) = (e / KW, e % KW),
    // so lane l holds k = l % KW and q = ii*(64/KW) + l / KW
    const int kl = lane % KW, ql = lane / KW;
    const int wo = kl < kvalid ? (kl * p.cin * RS + ql) * (int)sizeof(float) : kOutOfRange;
    auto dma_full = [&](int c, float4 *xb4, float *wb) __attribute__((always_inline)) {
        const int c0 = c * CC;
        const int xso = c0 * HW * (int)sizeof(float);
#pragma unroll
        for (int t = 0; t < XPW; ++t) {
            const int ii = wv + t * NWAVE;
            // (an array element passed straight to the builtin makes the
            // host compilation drop this kernel's launch stub)
            const int vo = xo[t];
            if constexpr (VEC) {
                if (ii < XI)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(xs, (lds_void_t *)(xb4 + ii * 64), 16, vo, xso, 0, 0);
            } else {
                if (ii < XI1)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        xs, (lds_void_t *)(reinterpret_cast<float *>(xb4) + ii * 64), 4, vo, xso, 0, 0);
            }
        }
        const int wso = c0 * RS * (int)sizeof(float);
        for (int ii = wv; ii < WI; ii += NWAVE)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ws, (lds_void_t *)(wb + ii * 64), 4, wo,
                                                     wso + ii * (64 / KW) * (int)sizeof(float), 0, 0);
    };
    auto dma_any = [&](int c, float4 *xb4, float *wb) __attribute__((always_inline)) {
        if (c * CC + CC <= p.cin)
            dma_full(c, xb4, wb);
        else
            dma(c, xb4, wb);
    };

    floatx16 acc[MB][NB];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[m][b][v] = 0.0f;
    auto mfma_chunk = [&](const float4 *xb4, const float *wb) __attribute__((always_inline)) {
        const float *xin = reinterpret_cast<const float *>(xb4);
#pragma unroll
        for (int ci = 0; ci < HALF; ++ci) {
            const int cl = h * HALF + ci;
            const float *xq = xin + (cl * TIH + ST * wave * NBR) * PITCH + j;
            const float *wq = wb + cl * RS * KW + j;
            // kernel rows one at a time: unrolling them all lets the compiler
            // hoist every row's LDS reads and spill with two output blocks
#pragma unroll 1
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    float a[MB], b[NB];
#pragma unroll
                    for (int m = 0; m < MB; ++m) a[m] = wq[(r * S + s) * KW + m * 32];
#pragma unroll
                    for (int br = 0; br < NBR; ++br)
#pragma unroll
                        for (int bc = 0; bc < NBC; ++bc)
                            b[br * NBC + bc] = xq[(ST * br + r) * PITCH +
                                                   (ST == 1 ? bc * 32 + s : (s & 1) * HW2 + bc * 32 + (s >> 1))];
#pragma unroll
                    for (int m = 0; m < MB; ++m)
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[m][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[m], b[nb], acc[m][nb], 0, 0, 0);
                }
        }
    };

    // chunk c: wait for this wave's DMA of chunk c, barrier (every wave's
    // DMA has landed and every wave is done with chunk c-1's buffer) ->
    // DMA chunk c+1 into that buffer -> MFMAs of chunk c.
    dma_any(0, xA4, wA);
    for (int c = 0; c < nchunks; c += 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        if (c + 1 < nchunks) dma_any(c + 1, xB4, wB);
        mfma_chunk(xA4, wA);
        if (c + 1 >= nchunks) break;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        if (c + 2 < nchunks) dma_any(c + 2, xA4, wA);
        mfma_chunk(xB4, wB);
    }

    // ---- epilogue
    const size_t plane = (size_t)p.Ho * p.Wo;
    float *yb = y + ((size_t)n * p.K + k0) * plane;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int br = 0; br < NBR; ++br) {
            const int oh = oh0 + wave * NBR + br;
#pragma unroll
            for (int bc = 0; bc < NBC; ++bc) {
                const int ow = ow0 + bc * 32 + j;
                if (oh >= p.Ho || ow >= p.Wo) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int k = m * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                    if (k < kvalid) {
                        float o = acc[m][br * NBC + bc][v];
                        if (bias) o += bias[k0 + k];
                        yb[(size_t)k * plane + (size_t)oh * p.Wo + ow] = o;
                    }
                }
            }
        }
}

// Input-channel chunk for a kernel size: the weights of one chunk stay
// within about 24 KB for a 64-channel block.
template <int R, int S>
constexpr int chunk_for() {
    return R * S <= 9 ? 8 : (R * S <= 25 ? 4 : 2);
}

size_t lds_bytes(int R, int S, int MB, int CC, int pitch) {
    return sizeof(float) * ((size_t)CC * (kTH + R - 1) * pitch + (size_t)((CC * R * S) | 1) * 32 * MB);
}

template <int R, int S, int MB, bool FUSED>
hipError_t launch_t(const IgParams &p, dim3 grid, const float *x, const float *w, const float *bias,
                    float *y, const FusedEpilogue &ep, hipStream_t st) {
    constexpr int CC = chunk_for<R, S>();
    if constexpr (!FUSED) {
        // one-dimensional grid of p.n_wg workgroups (the kernel maps ids to
        // work items itself)
        const dim3 g1((unsigned)p.n_wg);
        clear_stale_launch_error();
        if (p.st == 2) {
            // a stride-2 band is twice as wide per channel: fewer channels
            // per chunk at 3x3 keep the two buffers within 64 KB
            if constexpr ((R == 1 && S == 1) || (R == 3 && S == 3)) {
                constexpr int CC2 = R * S == 1 ? 8 : 4;
                if (p.nbc == 1)
                    hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC2, false, 2, 1, 1>), g1, dim3(kBlock), 0, st, x,
                                       w, bias, y, p);
                else
                    hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC2, false, 2, kNBC, 1>), g1, dim3(kBlock), 0, st,
                                       x, w, bias, y, p);
            } else {
                return hipErrorInvalidValue;
            }
        } else if (p.vec) {
            if (p.nbc == 1)
                hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC, true, 1, 1, kNBR>), g1, dim3(kBlock), 0, st, x, w,
                                   bias, y, p);
            else if (p.nbr == 1)
                hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC, true, 1, kNBC, 1>), g1, dim3(kBlock), 0, st, x, w,
                                   bias, y, p);
            else
                hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC, true, 1, kNBC, kNBR>), g1, dim3(kBlock), 0, st, x,
                                   w, bias, y, p);
        } else {
            if (p.nbc == 1)
                hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC, false, 1, 1, kNBR>), g1, dim3(kBlock), 0, st, x, w,
                                   bias, y, p);
            else if (p.nbr == 1)
                hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC, false, 1, kNBC, 1>), g1, dim3(kBlock), 0, st, x, w,
                                   bias, y, p);
            else
                hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC, false, 1, kNBC, kNBR>), g1, dim3(kBlock), 0, st, x,
                                   w, bias, y, p);
        }
        return hipGetLastError();
    } else {
        const size_t lds = lds_bytes(R, S, MB, CC, p.pitch);
        clear_stale_launch_error();
        hipLaunchKernelGGL((igemm_kernel<R, S, MB, CC, FUSED>), grid, dim3(kBlock), lds, st, x, w, bias,
                           y, p, ep);
        return hipGetLastError();
    }
}

template <int R, int S, bool FUSED>
hipError_t launch_mb(int MB, const IgParams &p, dim3 grid, const float *x, const float *w,
                     const float *bias, float *y, const FusedEpilogue &ep, hipStream_t st) {
    if constexpr (FUSED || kPlainMB == 2) {
        if (MB == 2) return launch_t<R, S, 2, FUSED>(p, grid, x, w, bias, y, ep, st);
    }
    return launch_t<R, S, 1, FUSED>(p, grid, x, w, bias, y, ep, st);
}

template <bool FUSED>
hipError_t launch_rs(const gconv_desc *d, const IgParams &p, int MB, dim3 grid, const float *x,
                     const float *w, const float *bias, float *y, const FusedEpilogue &ep,
                     hipStream_t st) {
    const int rs = d->R * 16 + d->S;
    switch (rs) {
        case 1 * 16 + 1: return launch_mb<1, 1, FUSED>(MB, p, grid, x, w, bias, y, ep, st);
        case 3 * 16 + 3: return launch_mb<3, 3, FUSED>(MB, p, grid, x, w, bias, y, ep, st);
        case 5 * 16 + 5: return launch_mb<5, 5, FUSED>(MB, p, grid, x, w, bias, y, ep, st);
        case 5 * 16 + 9: return launch_mb<5, 9, FUSED>(MB, p, grid, x, w, bias, y, ep, st);
        case 7 * 16 + 7: return launch_mb<7, 7, FUSED>(MB, p, grid, x, w, bias, y, ep, st);
        default: return hipErrorInvalidValue;
    }
}

bool rs_instantiated(int R, int S) {
    return (R == 1 && S == 1) || (R == 3 && S == 3) || (R == 5 && S == 5) || (R == 5 && S == 9) ||
           (R == 7 && S == 7);
}

int pick_mb(const gconv_desc *d) { return d->cout > 32 ? 2 : 1; }

IgParams make_params(const gconv_desc *d, int MB) {
    IgParams p;
    p.C = d->C; p.H = d->H; p.W = d->W; p.K = d->K; p.Ho = d->Ho; p.Wo = d->Wo;
    p.pad_h = d->pad_h; p.pad_w = d->pad_w;
    p.cin = d->cin; p.cout = d->cout;
    p.n_kb = (d->cout + 32 * MB - 1) / (32 * MB);
    // kTH x kTW tiles (the fused kernel's; launch_igemm sets the DMA
    // kernel's own)
    p.nbc = kNBC;
    p.nbr = kNBR;
    p.n_tw = (d->Wo + kTW - 1) / kTW;
    p.n_tiles = p.n_tw * ((d->Ho + kTH - 1) / kTH);
    p.pitch = kTW + d->S - 1;
    p.vec = 0;
    p.G = d->groups;
    p.n_wg = 0;
    p.st = d->stride_h;
    return p;
}

}  // namespace

bool igemm_supported(const gconv_desc *d) {
    // buffer offsets are signed 32-bit: one group's input channels of one
    // image must stay below 2 GB
    // stride 1, or stride 2 on both axes at 1x1 and 3x3
    const bool stride_ok = d->stride_h == d->stride_w &&
                           (d->stride_h == 1 || (d->stride_h == 2 && d->R == d->S && (d->R == 1 || d->R == 3)));
    return stride_ok && d->dil_h == 1 && d->dil_w == 1 && rs_instantiated(d->R, d->S) && d->cin >= 4 &&
           d->cout >= 8 && (long long)d->cin * d->H * d->W * (long long)sizeof(float) < 0x7fffffffLL - 64;
}

bool igemm_fused_supported(const gconv_desc *d, int gn_groups) {
    // every output channel of every 32*MB block must exist, and a GroupNorm
    // group must be 4 channels
    // (the fused kernel runs at stride 1 only)
    // its grid is (tiles, group x channel block, n), within the hardware's
    // 65535 limit on y and z
    const long long gy = (long long)d->groups * ((d->cout + 32 * pick_mb(d) - 1) / (32 * pick_mb(d)));
    return igemm_supported(d) && d->stride_h == 1 && d->cout % (32 * pick_mb(d)) == 0 && d->K / gn_groups == 4 &&
           gy <= 65535 && d->N <= 65535;
}

int igemm_fused_parts_per_group(const gconv_desc *d, int) {
    return make_params(d, pick_mb(d)).n_tiles;
}

hipError_t launch_igemm(const gconv_desc *d, const float *x, const float *w, const float *bias,
                        float *y, hipStream_t st) {
    if (!igemm_supported(d)) return hipErrorInvalidValue;
    // one 32-channel block per workgroup (kPlainMB): each input band is
    // read once per block, in exchange for no register spills
    const int MB = kPlainMB == 2 ? pick_mb(d) : 1;
    IgParams p = make_params(d, MB);
    p.vec = d->stride_h == 1 && (d->W % 4 == 0) && (d->pad_w % 4 == 0) && (((uintptr_t)x & 15u) == 0);
    // the DMA kernel's tile: 8 rows (4 at stride 2) by 64 columns, or by one
    // 32-column block on outputs at most 32 wide; 4 rows as well when 8-row
    // tiles would leave fewer than two workgroups per CU (more, smaller
    // workgroups keep more loads in flight)
    p.nbc = d->Wo <= 32 ? 1 : kNBC;
    p.nbr = d->stride_h == 2 ? 1 : kNBR;
    const long long gy = (long long)d->groups * p.n_kb;
    auto tiles = [&]() {
        const int th = 4 * p.nbr, tw = 32 * p.nbc;
        p.n_tw = (d->Wo + tw - 1) / tw;
        p.n_tiles = p.n_tw * ((d->Ho + th - 1) / th);
        return gy * p.n_tiles * d->N;
    };
    long long n_wg = tiles();
    if (p.nbr == kNBR && p.nbc == kNBC && n_wg < kSmallGridWorkgroups) {
        p.nbr = 1;
        n_wg = tiles();
    }
    // the DMA kernel runs a one-dimensional grid of n_wg workgroups (below
    // 2^31 for every valid descriptor: each holds at least one output)
    if (n_wg > 0x7fffffffLL) return launch_direct(d, x, w, bias, y, st);
    p.n_wg = (int)n_wg;
    dim3 grid((unsigned)p.n_tiles, (unsigned)gy, (unsigned)d->N);
    FusedEpilogue none{};
    return launch_rs<false>(d, p, MB, grid, x, w, bias, y, none, st);
}

hipError_t launch_igemm_fused(const gconv_desc *d, const float *x, const float *w, float *y,
                              const FusedEpilogue &ep, hipStream_t st) {
    if (!igemm_fused_supported(d, ep.gn_groups)) return hipErrorInvalidValue;
    const int MB = pick_mb(d);
    const IgParams p = make_params(d, MB);
    const long long gy = (long long)d->groups * p.n_kb;
    if (gy > 65535 || d->N > 65535) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)p.n_tiles, (unsigned)gy, (unsigned)d->N);
    return launch_rs<true>(d, p, MB, grid, x, w, nullptr, y, ep, st);
}

}  // namespace gconv
