// k_igemm.hip -- FP32 MFMA implicit GEMM for dense and wide-group
// convolution (any padding and number of input channels; dilation 1 with
// stride 1, or stride 2 at square 1x1-7x7, in the DMA-staged tile kernel;
// 3x3 at dilation 2, and at stride 1 dilation 3 and 4, in the
// flattened-pixel kernel).
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
//  - Narrow 1x1 and 3x3 outputs, which rows x 32-column tiles fit badly,
//    take tiles of consecutive pixels of the flattened batch instead
//    (igemm_flat_kernel).
#include <algorithm>
#include <climits>

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
    int st;            // stride (both axes): 1, or 2 for the DMA kernel at 1x1, 3x3, 5x5 and 7x7
    int nbc;           // 32-column blocks per wave row of the DMA kernel (1 on outputs at most 32 wide)
    int nbr;           // output rows per wave of the DMA kernel (1 at stride 2 and on small grids)
    int wvec;          // C/G*R*S a multiple of 4 and w 16-byte aligned: 16-byte weight loads
    int ds;            // stride 2 with 16-byte band loads: the band's column shift (0..3)
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
// ST*oh0 - pad ... of the tile.  With 4-byte (gather) band loads each row's
// columns are in two phases, even input columns first, then odd ones (HW2 of
// each): output column ow at tap s reads input column 2*ow + s, which is
// phase s%2, position ow + s/2, so the 32 lanes of a block still read 32
// consecutive LDS words.  With 16-byte band loads (VEC: W % 4 == 0, x
// 16-byte aligned) the columns stay in order from input column 2*ow0 - pad_w
// - ds, ds (0..3) aligning it to a 16-byte piece: output column ow at tap s
// is band column 2*(ow - ow0) + s + ds, and a block reads every other word.
// NBR output rows per wave (a 4*NBR-row tile): 2, or 1 at stride 2 and on
// grids too small to fill the chip.
//
// WG: the columns in the Winograd form F(2, 3) (Lavin and Gray, "Fast
// Algorithms for Convolutional Neural Networks"), for kernels 3 wide at
// stride 1 on 64-column tiles with one row per wave.  Lane j owns output
// columns 2j and 2j+1 of its row; for each kernel row r and input channel
// the lane forms the four B operands V = B^T d of its 4-column input patch
// d (B^T = [1 0 -1 0; 0 1 1 0; 0 -1 1 0; 0 1 0 -1]) and the four A operands
// U = G g of the kernel row's 3 weights (G = [1 0 0; 1/2 1/2 1/2; 1/2 -1/2
// 1/2; 0 0 1]), and four MFMA chains accumulate M[u] = sum over kernel rows
// and channels of U[u] V[u].  The output transform A^T M (A^T = [1 1 1 0;
// 0 1 -1 -1]) runs once, in the epilogue: 12 MFMAs per kernel row and
// channel pair where the direct form takes 18 for the same 64 outputs.
template <int R, int S, int MB, int CC, bool VEC, int ST, int NBC, int NBR, bool WG = false>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void igemm_dma_kernel(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ y, IgParams p) {
    static_assert(ST == 1 || ST == 2, "stride 1 or 2");
    static_assert(!WG || (ST == 1 && S == 3 && MB == 1 && NBC == 2 && NBR == 1), "Winograd columns: 3 wide, stride 1");
    constexpr int RS = R * S;
    constexpr int KW = 32 * MB;
    constexpr int TH = 4 * NBR;
    // NBC 32-column blocks per wave row (1 on outputs at most 32 wide)
    constexpr int TW = 32 * NBC;
    constexpr int TIH = ST * (TH - 1) + R;
    constexpr int HW2 = TW + (S - 1) / 2;   // stride 2: columns per phase
    constexpr int TIW = ST == 1 ? TW + S - 1 : VEC ? 2 * (TW - 1) + S + 3 : 2 * HW2;
    constexpr int PITCH = (TIW + 3) & ~3;    // band row pitch: whole 16-byte pieces
    constexpr int P4 = PITCH / 4;
    constexpr int XE4 = CC * TIH * P4;       // 16-byte pieces of a chunk's band
    constexpr int XI = (XE4 + 63) / 64;      // band DMA instructions (16-byte pieces)
    constexpr int XE = XE4 * 4;
    constexpr int XI1 = (XE + 63) / 64;      // band DMA instructions (4-byte elements)
    constexpr int WE = CC * RS * KW;         // weight words of a chunk, [q][KW]
    constexpr int WI = (WE + 63) / 64;       // weight DMA instructions
    // Where a chunk's QP = CC*R*S weights per output channel are whole
    // 16-byte pieces (QP % 4 == 0: 1x1, 3x3, 5x5), the weights sit in LDS as
    // [output channel][WQP] instead, WQP = QP or QP + 4 (4 mod 8, so the 32
    // lanes reading 32 channels' weight q touch at most two words per
    // bank), and a full chunk loads them in 16-byte pieces: a quarter of the
    // DMA instructions, which on small layers are what the time follows.
    constexpr int QP = CC * RS;
    constexpr bool WK = QP % 4 == 0;
    constexpr int WQP = QP % 8 == 0 ? QP + 4 : QP;
    constexpr int WL = KW * WQP;             // (WK) weight floats of a chunk in LDS
    constexpr int WI16 = (WL / 4 + 63) / 64; // (WK) 16-byte weight DMA instructions
    constexpr int WI4 = (WL + 63) / 64;      // (WK) 4-byte weight DMA instructions
    constexpr int WPW = (WI16 + 3) / 4;      // (WK) 16-byte weight DMA instructions per wave
    constexpr int WCAP = WK ? WI16 * 256 : WI * 64;
    // accumulator blocks: NBR x NBC of 32 pixels, or (WG) the four Winograd
    // positions of 32 column pairs
    constexpr int NB = WG ? 4 : NBR * NBC;
    constexpr int HALF = CC / 2;
    constexpr int NWAVE = kBlock / 64;

    // buffers padded to whole DMA instructions (idle lanes write zeros there)
    __shared__ float4 xA4[XI * 64];
    __shared__ float4 xB4[XI * 64];
    __shared__ float wA[WCAP];
    __shared__ float wB[WCAP];

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
                const int ih = ST * oh0 - p.pad_h + lr, iw = ST * ow0 - p.pad_w - (ST == 2 ? p.ds : 0) + 4 * c4;
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
        if constexpr (WK) {
            for (int ii = wave; ii < WI4; ii += NWAVE) {
                const int e = ii * 64 + lane;            // e = k * WQP + q
                const int k = e / WQP, q = e - k * WQP;  // q = cl * RS + t
                const bool ok = e < WL && k < kvalid && q < QP && c0 + q / RS < p.cin;
                const int off = ok ? (k * p.cin * RS + c0 * RS + q) * (int)sizeof(float) : kOutOfRange;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ws, (lds_void_t *)(wb + ii * 64), 4, off, 0, 0, 0);
            }
        } else {
            for (int ii = wave; ii < WI; ii += NWAVE) {
                const int e = ii * 64 + lane;            // e = q * KW + k
                const int q = e / KW, k = e - q * KW;    // q = cl * RS + t
                const int cl = q / RS;
                const bool ok = e < WE && k < kvalid && c0 + cl < p.cin;
                const int off = ok ? (k * p.cin * RS + c0 * RS + q) * (int)sizeof(float) : kOutOfRange;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ws, (lds_void_t *)(wb + ii * 64), 4, off, 0, 0, 0);
            }
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
            const int ih = ST * oh0 - p.pad_h + lr, iw = ST * ow0 - p.pad_w - (ST == 2 ? p.ds : 0) + 4 * c4;
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
    // (WK) 16-byte weight piece f = ii*64 + lane: channel f / (WQP/4),
    // weights 4*(f % (WQP/4)) ..+3 of the chunk
    int wo16[WK ? WPW : 1];
    if constexpr (WK) {
#pragma unroll
        for (int t = 0; t < WPW; ++t) {
            const int f = (wv + t * NWAVE) * 64 + lane;
            const int k = f / (WQP / 4), q4 = f - k * (WQP / 4);
            wo16[t] = (k < kvalid && 4 * q4 < QP) ? (k * p.cin * RS + 4 * q4) * (int)sizeof(float) : kOutOfRange;
        }
    }
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
        if constexpr (WK) {
#pragma unroll
            for (int t = 0; t < WPW; ++t) {
                const int ii = wv + t * NWAVE;
                const int vo = wo16[t];
                if (ii < WI16)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(ws, (lds_void_t *)(wb + ii * 256), 16, vo, wso, 0, 0);
            }
        } else {
            for (int ii = wv; ii < WI; ii += NWAVE)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ws, (lds_void_t *)(wb + ii * 64), 4, wo,
                                                         wso + ii * (64 / KW) * (int)sizeof(float), 0, 0);
        }
    };
    auto dma_any = [&](int c, float4 *xb4, float *wb) __attribute__((always_inline)) {
        // 16-byte weight pieces need the tensor's pieces aligned (p.wvec)
        if (c * CC + CC <= p.cin && (!WK || p.wvec))
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
        if constexpr (WG) {
#pragma unroll
            for (int ci = 0; ci < HALF; ++ci) {
                const int cl = h * HALF + ci;
                // band row (wave's output row) + r, columns 2j .. 2j+3
                const float *xq = xin + (cl * TIH + wave) * PITCH + 2 * j;
                const float *wq = WK ? wb + j * WQP + cl * RS : wb + cl * RS * KW + j;
                // kernel rows one at a time, as in the direct form
#pragma unroll 1
                for (int r = 0; r < R; ++r) {
                    float d[4], g[3];
#pragma unroll
                    for (int c = 0; c < 4; ++c) d[c] = xq[r * PITCH + c];
#pragma unroll
                    for (int s = 0; s < 3; ++s) g[s] = WK ? wq[r * 3 + s] : wq[(r * 3 + s) * KW];
                    const float vb[4] = {d[0] - d[2], d[1] + d[2], d[2] - d[1], d[1] - d[3]};
                    const float t = g[0] + g[2];
                    const float ua[4] = {g[0], 0.5f * (t + g[1]), 0.5f * (t - g[1]), g[2]};
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        acc[0][u] = __builtin_amdgcn_mfma_f32_32x32x2f32(ua[u], vb[u], acc[0][u], 0, 0, 0);
                }
            }
            return;
        }
#pragma unroll
        for (int ci = 0; ci < HALF; ++ci) {
            const int cl = h * HALF + ci;
            const float *xq = xin + (cl * TIH + ST * wave * NBR) * PITCH + (ST == 2 && VEC ? 2 * j + p.ds : j);
            const float *wq = WK ? wb + j * WQP + cl * RS : wb + cl * RS * KW + j;
            // kernel rows one at a time: unrolling them all lets the compiler
            // hoist every row's LDS reads and spill with two output blocks
#pragma unroll 1
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    float a[MB], b[NB];
#pragma unroll
                    for (int m = 0; m < MB; ++m) a[m] = WK ? wq[m * 32 * WQP + r * S + s] : wq[(r * S + s) * KW + m * 32];
#pragma unroll
                    for (int br = 0; br < NBR; ++br)
#pragma unroll
                        for (int bc = 0; bc < NBC; ++bc)
                            b[br * NBC + bc] = xq[(ST * br + r) * PITCH +
                                                   (ST == 1 ? bc * 32 + s
                                                    : VEC    ? 64 * bc + s
                                                             : (s & 1) * HW2 + bc * 32 + (s >> 1))];
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
    if constexpr (ST == 1 && R * S > 1) {
        // One call site of the MFMA loop, the buffers chosen by the chunk's
        // parity: with a call per buffer the compiler gave each inlined
        // kernel-row loop its own accumulator registers and copied all of
        // them in and out around every chunk (64 moves after an MFMA drain).
        // The 1x1 and stride-2 chunks are short, and keep two chunks per
        // iteration (measured faster there).
        for (int c = 0; c < nchunks; ++c) {
            const bool odd = c & 1;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();
            if (c + 1 < nchunks) dma_any(c + 1, odd ? xA4 : xB4, odd ? wA : wB);
            mfma_chunk(odd ? xB4 : xA4, odd ? wB : wA);
        }
    } else {
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
    }

    // ---- epilogue
    const size_t plane = (size_t)p.Ho * p.Wo;
    float *yb = y + ((size_t)n * p.K + k0) * plane;
    if constexpr (WG) {
        // output transform: column 2j gets M0 + M1 + M2, column 2j+1 gets
        // M1 - M2 - M3
        const int oh = oh0 + wave;
        // an even output width with y 8-byte aligned: the lane's two columns
        // are neighbours, inside or outside the output together, and one
        // 8-byte store writes both (each store instruction then covers whole
        // lines instead of every other word)
        if (oh < p.Ho && p.Wo % 2 == 0 && ((uintptr_t)yb & 7u) == 0) {
            const int ow = ow0 + 2 * j;
            if (ow < p.Wo) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int k = 8 * (v >> 2) + 4 * h + (v & 3);
                    if (k < kvalid) {
                        float2 o = make_float2((acc[0][0][v] + acc[0][1][v]) + acc[0][2][v],
                                               (acc[0][1][v] - acc[0][2][v]) - acc[0][3][v]);
                        if (bias) {
                            const float bk = bias[k0 + k];
                            o.x += bk;
                            o.y += bk;
                        }
                        *reinterpret_cast<float2 *>(yb + (size_t)k * plane + (size_t)oh * p.Wo + ow) = o;
                    }
                }
            }
        } else if (oh < p.Ho) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int ow = ow0 + 2 * j + b;
                if (ow >= p.Wo) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int k = 8 * (v >> 2) + 4 * h + (v & 3);
                    if (k < kvalid) {
                        float o = b == 0 ? (acc[0][0][v] + acc[0][1][v]) + acc[0][2][v]
                                         : (acc[0][1][v] - acc[0][2][v]) - acc[0][3][v];
                        if (bias) o += bias[k0 + k];
                        yb[(size_t)k * plane + (size_t)oh * p.Wo + ow] = o;
                    }
                }
            }
        }
        return;
    }
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

// ---- Flattened-pixel tiles (outputs that rows x 32-column tiles fit badly)
//
// The tiles above waste lanes where the output is narrow: a 28-wide output
// fills 28 of a block's 32 columns, a 14-wide one 14.  Here the batch's
// output pixels are numbered in NCHW order, P = (n*Ho + oh)*Wo + ow, and a
// workgroup takes T = 128*NB consecutive ones: wave w's NB blocks of 32
// pixels are P0 + (w*NB + b)*32 + j.  A block may run over row and image
// boundaries, so only the batch's last tile has idle lanes.  The GEMM is the
// same: the pixel axis of D[k][p] is just enumerated across rows and images.
//
// The band holds whole input rows of "virtual" row numbers: the batch's
// images stacked with their zero padding, image n's padded row ihp (input row
// ihp - pad_h) being virtual row n*HV + ihp, HV = H + 2*pad_h.  Output pixel
// (n, oh, ow) at kernel row r reads virtual row n*HV + ST*oh + r*DIL, so each
// lane's operands sit at a fixed offset from the band's first row, which is
// that of the tile's first pixel.  The host bounds the band's height (tih
// rows, at most 64) over every tile.  The same addressing serves 1x1 and 3x3
// at stride 1 and 2, 3x3 at dilation 2 (and 3 and 4 at stride 1), 5x5 and
// 7x7 at stride 2, and 1x3, 3x1, 1x7 and 7x1 at stride 1.
//
// Band layout: [band row][channel of the chunk][pitch], the pitch a power of
// two so that a lane finds its element with shifts:
//  - band column c holds input column c - pad_w - ds, where ds (0..3) makes
//    pad_w + ds a multiple of 4, so 16-byte pieces of the band are 16-byte
//    pieces of x (VEC: W % 4 == 0, x 16-byte aligned); pixel ow's tap s is
//    column ST*ow + s*DIL + ds (at stride 2 the 32 lanes of a block read
//    every other word);
//  - stride 2 with 4-byte loads (W % 4 != 0 or x unaligned): two phases as
//    in the tile kernel, band column c < pitch/2 holding padded column 2c
//    and pitch/2 + c padded column 2c+1, so a block reads consecutive words.
// The 16-byte pieces take a quarter of the DMA instructions of 4-byte
// loads (at stride 2 on MI355X: 40.5 -> 34.3 us on a 14-wide 32-channel-group
// layer, 76.7 -> 58.2 us on a 28-wide dense one).
// Each band row's input row offset (or "none": padding, or past the batch)
// is computed once per workgroup by lane = row and fetched with a lane
// shuffle, so no lane divides while it finds its DMA elements.
struct FlatParams {
    int C, H, W, K, Ho, Wo;
    int pad_h, pad_w;
    int cin, cout;
    int n_kb;     // output-channel blocks of 32 per group
    int G, N;
    int np;       // output pixels of the batch, N*Ho*Wo
    int howo;     // Ho*Wo
    int hv;       // virtual rows per image, H + 2*pad_h
    int lp;       // log2 of the band pitch (floats)
    int tih;      // band rows, at most 64
    int ds;       // column shift of the band (0 unless 16-byte pieces)
    int xi;       // band DMA instructions of 64 lanes per chunk
    int n_tf;     // tiles of the batch, ceil(np / T)
    int n_wg;     // G * n_tf * n_kb
    int x_bytes;  // bytes of x from the group's first channel of image 0 to the end of image N-1's group
    int wvec;     // weights in 16-byte pieces: C/G*R*S a multiple of 4 and w 16-byte aligned
};

// band DMA instructions per chunk, at most: 64 (16 per wave, one offset
// register each), or 128 for 4-byte loads where the band is taller for its
// pixels (stride 2, dilation 2, 5x5 and 7x7)
constexpr int flat_max_band_insts(int R, int ST, int DIL, bool VEC) {
    return VEC || (ST == 1 && DIL == 1 && R <= 3) ? 64 : 128;
}

template <int R, int S, int CC, bool VEC, int ST, int NB, int DIL>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void igemm_flat_kernel(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ y, FlatParams p) {
    static_assert(ST == 1 || ST == 2, "stride 1 or 2");
    static_assert(DIL >= 1 && DIL <= 4, "dilation 1 to 4");
    static_assert((CC & (CC - 1)) == 0, "the chunk is a power of two");
    constexpr int RS = R * S;
    constexpr int KW = 32;
    constexpr int NWAVE = kBlock / 64;
    constexpr int T = 32 * NB * NWAVE;
    constexpr int UNIT = VEC ? 4 : 1;  // floats per lane of a band DMA instruction
    // Weights of a chunk in LDS as [output channel][QP] with row pitch WQP:
    // a channel's QP = CC*R*S weights of the chunk are contiguous in w, so
    // they load in 16-byte pieces (pieces past QP read zero).  WQP is 4 mod
    // 8, so the 32 lanes reading 32 channels' weight q touch at most two
    // words per bank.
    constexpr int QP = CC * RS;
    constexpr int WQP = ((QP + 3) / 4 * 4) % 8 == 0 ? (QP + 3) / 4 * 4 + 4 : (QP + 3) / 4 * 4;
    // a chunk's weights start on a 16-byte boundary only when QP % 4 == 0
    // (7x7 chunks of 2 channels, 98 weights, take 4-byte loads)
    constexpr bool WV16 = QP % 4 == 0;
    constexpr int WL = KW * WQP;            // weight floats of a chunk in LDS
    constexpr int WI16 = (WL / 4 + 63) / 64;  // 16-byte weight DMA instructions
    constexpr int WI4 = (WL + 63) / 64;       // 4-byte weight DMA instructions
    constexpr int WPW = (WI16 + NWAVE - 1) / NWAVE;
    constexpr int HALF = CC / 2;
    constexpr int XPW = flat_max_band_insts(R, ST, DIL, VEC) / NWAVE;
    // stride 2 with 4-byte loads: the band's columns in two phases
    constexpr bool PHASES = ST == 2 && !VEC;

    // two band buffers of p.xi*64*UNIT floats each (dynamic), two weight buffers
    extern __shared__ float4 flat_band4[];
    __shared__ float4 wA4[WI16 * 64];
    __shared__ float4 wB4[WI16 * 64];
    float *const wA = reinterpret_cast<float *>(wA4);
    float *const wB = reinterpret_cast<float *>(wB4);
    float *const bandA = reinterpret_cast<float *>(flat_band4);
    float *const bandB = bandA + p.xi * 64 * UNIT;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, j = lane & 31;
    // workgroup -> (group, tile, channel block), each XCD taking a contiguous
    // run (as in the tile kernel): neighbouring tiles share band rows in L2
    const int L = blockIdx.x;
    const int xcd = L & 7, slot = L >> 3;
    const int per = p.n_wg >> 3, rem = p.n_wg & 7;
    const int item = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    const int kb = item % p.n_kb;
    const int t1 = item / p.n_kb;
    const int tile = t1 % p.n_tf;
    const int g = t1 / p.n_tf;
    const int kg0 = kb * KW;
    const int k0 = g * p.cout + kg0;
    const int kvalid = min(KW, p.cout - kg0);
    const int HW = p.H * p.W;
    const int CHW = p.C * HW;
    const int pitch = 1 << p.lp;
    const __amdgpu_buffer_rsrc_t xs = make_rsrc(x + (size_t)g * p.cin * HW, p.x_bytes);
    const __amdgpu_buffer_rsrc_t ws = make_rsrc(w + (size_t)k0 * p.cin * RS, kvalid * p.cin * RS * (int)sizeof(float));
    const int nchunks = (p.cin + CC - 1) / CC;

    // the tile's first pixel and the virtual row of its kernel row 0
    const int P0 = tile * T;
    const int n0 = P0 / p.howo;
    const int oh0 = (P0 - n0 * p.howo) / p.Wo;
    const int vr0 = n0 * p.hv + ST * oh0;
    // lane l: element offset (from the group's first channel of image 0) of
    // band row l's input row, or -1 for a row of zeros
    int rb;
    {
        const int vr = vr0 + lane;
        const int nl = vr / p.hv;
        const int ih = vr - nl * p.hv - p.pad_h;
        rb = (lane < p.tih && nl < p.N && ih >= 0 && ih < p.H) ? nl * CHW + ih * p.W : -1;
    }

    // Per-lane band DMA offsets for a full chunk (the chunk's first channel
    // goes in the scalar offset): instruction ii = wave + t*4 writes band
    // floats [ii*64*UNIT, (ii+1)*64*UNIT).
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int xo[XPW];
#pragma unroll
    for (int t = 0; t < XPW; ++t) {
        const int ii = wv + t * NWAVE;
        const int u = (ii * 64 + lane) * UNIT;
        const int row = u >> p.lp, c = u & (pitch - 1);
        const int i = row / CC, cl = row & (CC - 1);
        const int rbi = __shfl(rb, i & 63);
        int iw;
        if constexpr (!PHASES) {
            iw = c - p.pad_w - p.ds;
        } else {
            const int hp = pitch >> 1;
            const int ph = c >= hp ? 1 : 0;
            iw = 2 * (c - ph * hp) + ph - p.pad_w;
        }
        const bool ok = ii < p.xi && i < p.tih && rbi >= 0 && iw >= 0 && iw < p.W;
        xo[t] = ok ? (rbi + cl * HW + iw) * (int)sizeof(float) : kOutOfRange;
    }
    // 16-byte weight pieces of a full chunk: piece f = ii*64 + lane is
    // (channel f / (WQP/4), weights 4*(f % (WQP/4)) ..+3); the chunk's first
    // channel goes in the scalar offset
    int wo[WPW];
#pragma unroll
    for (int t = 0; t < WPW; ++t) {
        const int f = (wv + t * NWAVE) * 64 + lane;
        const int k = f / (WQP / 4), q4 = f - k * (WQP / 4);
        wo[t] = (k < kvalid && 4 * q4 < QP) ? (k * p.cin * RS + 4 * q4) * (int)sizeof(float) : kOutOfRange;
    }
    auto dma = [&](int c, float *xb, float *wb) __attribute__((always_inline)) {
        const int c0 = c * CC;
        const bool full = c0 + CC <= p.cin;
        const int xso = c0 * HW * (int)sizeof(float);
#pragma unroll
        for (int t = 0; t < XPW; ++t) {
            const int ii = wv + t * NWAVE;
            if (ii < p.xi) {
                int vo = xo[t];
                if (!full) {
                    // the last, partial chunk: channels past cin read zero
                    const int cl = (((ii * 64 + lane) * UNIT) >> p.lp) & (CC - 1);
                    if (c0 + cl >= p.cin) vo = kOutOfRange;
                }
                if constexpr (VEC)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(xs, (lds_void_t *)(xb + ii * 64 * UNIT), 16, vo, xso, 0, 0);
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(xs, (lds_void_t *)(xb + ii * 64 * UNIT), 4, vo, xso, 0, 0);
            }
        }
        const int wso = c0 * RS * (int)sizeof(float);
        if (WV16 && full && p.wvec) {
#pragma unroll
            for (int t = 0; t < WPW; ++t) {
                const int ii = wv + t * NWAVE;
                const int vo = wo[t];
                if (ii < WI16)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(ws, (lds_void_t *)(wb + ii * 256), 16, vo, wso, 0, 0);
            }
        } else {
            // the last, partial chunk (its channels past cin read zero), or
            // weights that are not in 16-byte pieces: 4-byte loads
            for (int ii = wv; ii < WI4; ii += NWAVE) {
                const int e = ii * 64 + lane;
                const int k = e / WQP, q = e - k * WQP;
                const bool ok = e < WL && k < kvalid && q < QP && c0 + q / RS < p.cin;
                const int vo = ok ? (k * p.cin * RS + c0 * RS + q) * (int)sizeof(float) : kOutOfRange;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ws, (lds_void_t *)(wb + ii * 64), 4, vo, 0, 0, 0);
            }
        }
    };

    // Per-lane band offset of each block's pixel (kernel row 0, channel
    // h*HALF, tap column 0).  A pixel past the batch takes the batch's last
    // one (its result is not stored).
    int bo[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int P = min(P0 + (wave * NB + b) * 32 + j, p.np - 1);
        const int n = P / p.howo, q = P - n * p.howo;
        const int oh = q / p.Wo, ow = q - oh * p.Wo;
        const int vrow = n * p.hv + ST * oh;
        bo[b] = (((vrow - vr0) * CC + h * HALF) << p.lp) + (PHASES ? ow : ST * ow + p.ds);
    }
    const int hp = pitch >> 1;

    floatx16 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][v] = 0.0f;
    auto mfma_chunk = [&](const float *xb, const float *wb) __attribute__((always_inline)) {
#pragma unroll
        for (int ci = 0; ci < HALF; ++ci) {
            const float *wq = wb + j * WQP + (h * HALF + ci) * RS;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                // kernel row r reads band row (pixel's) + r*DIL, kernel
                // column s padded column (pixel's) + s*DIL
                const int ro = (r * DIL * CC + ci) << p.lp;
                const float *xq[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) xq[b] = xb + bo[b] + ro;
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const float a = wq[r * S + s];
                    float bv[NB];
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        bv[b] = !PHASES ? xq[b][s * DIL]
                                        : (((s * DIL) & 1) ? xq[b][hp + ((s * DIL) >> 1)] : xq[b][(s * DIL) >> 1]);
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        acc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bv[b], acc[b], 0, 0, 0);
                }
            }
        }
    };

    // the tile kernel's two-buffer chunk pipeline
    dma(0, bandA, wA);
    if constexpr (ST == 1 && R * S > 1 && DIL == 1) {
        // one call site of the MFMA loop, as in igemm_dma_kernel (dilated
        // kernels keep two chunks per iteration: measured faster there)
        for (int c = 0; c < nchunks; ++c) {
            const bool odd = c & 1;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();
            if (c + 1 < nchunks) dma(c + 1, odd ? bandA : bandB, odd ? wA : wB);
            mfma_chunk(odd ? bandB : bandA, odd ? wB : wA);
        }
    } else {
        for (int c = 0; c < nchunks; c += 2) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();
            if (c + 1 < nchunks) dma(c + 1, bandB, wB);
            mfma_chunk(bandA, wA);
            if (c + 1 >= nchunks) break;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();
            if (c + 2 < nchunks) dma(c + 2, bandA, wA);
            mfma_chunk(bandB, wB);
        }
    }

    // ---- epilogue: lanes j of a block store 32 consecutive pixels of the
    // batch (consecutive addresses within an image)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int P = P0 + (wave * NB + b) * 32 + j;
        if (P >= p.np) continue;
        const int n = P / p.howo, q = P - n * p.howo;
        float *yp = y + ((size_t)n * p.K + k0) * p.howo + q;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int k = 8 * (v >> 2) + 4 * h + (v & 3);
            if (k < kvalid) {
                float o = acc[b][v];
                if (bias) o += bias[k0 + k];
                yp[(size_t)k * p.howo] = o;
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

// Plain convs 3 wide (1x3, 3x3) at stride 1 take Winograd columns on
// 64-column tiles (see igemm_dma_kernel).
constexpr bool kIgWinograd = true;
template <int R, int S, int MB>
constexpr bool ig_winograd() {
    return kIgWinograd && S == 3 && (R == 1 || R == 3) && MB == 1;
}

template <int R, int S, int MB, bool FUSED>
hipError_t launch_t(const IgParams &p, dim3 grid, const float *x, const float *w, const float *bias,
                    float *y, const FusedEpilogue &ep, hipStream_t st) {
    constexpr int CC = chunk_for<R, S>();
    if constexpr (!FUSED) {
        // stride 1: 1x1 chunks of 16 channels (8 gave each wave only 8 MFMAs
        // between waits for its loads; 16 took a C256 -> 64 56x56 layer at
        // batch 16 from 28.0 to 23.8 us on MI355X)
        constexpr int CC1 = R * S == 1 ? 16 : CC;
        // one-dimensional grid of p.n_wg workgroups (the kernel maps ids to
        // work items itself)
        const dim3 g1((unsigned)p.n_wg);
        clear_stale_launch_error();
        if (p.st == 2) {
            // a stride-2 band is twice as wide per channel: fewer channels
            // per chunk at 3x3 keep the two buffers within 64 KB (5x5 and 7x7
            // keep their stride-1 chunks of 4 and 2)
            if constexpr (R == S && (R == 1 || R == 3 || R == 5 || R == 7)) {
                constexpr int CC2 = R * S == 1 ? 8 : R * S == 9 ? 4 : CC;
                if (p.vec) {
                    if (p.nbc == 1)
                        hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC2, true, 2, 1, 1>), g1, dim3(kBlock), 0, st,
                                           x, w, bias, y, p);
                    else
                        hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC2, true, 2, kNBC, 1>), g1, dim3(kBlock), 0,
                                           st, x, w, bias, y, p);
                } else if (p.nbc == 1) {
                    hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC2, false, 2, 1, 1>), g1, dim3(kBlock), 0, st, x,
                                       w, bias, y, p);
                } else {
                    hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC2, false, 2, kNBC, 1>), g1, dim3(kBlock), 0, st,
                                       x, w, bias, y, p);
                }
            } else {
                return hipErrorInvalidValue;
            }
        } else if (ig_winograd<R, S, MB>() && p.nbc == kNBC && p.nbr == 1) {
            if constexpr (ig_winograd<R, S, MB>()) {
                if (p.vec)
                    hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC1, true, 1, kNBC, 1, true>), g1, dim3(kBlock), 0,
                                       st, x, w, bias, y, p);
                else
                    hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC1, false, 1, kNBC, 1, true>), g1, dim3(kBlock),
                                       0, st, x, w, bias, y, p);
            }
        } else if (p.vec) {
            if (p.nbc == 1)
                hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC1, true, 1, 1, kNBR>), g1, dim3(kBlock), 0, st, x, w,
                                   bias, y, p);
            else if (p.nbr == 1)
                hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC1, true, 1, kNBC, 1>), g1, dim3(kBlock), 0, st, x, w,
                                   bias, y, p);
            else
                hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC1, true, 1, kNBC, kNBR>), g1, dim3(kBlock), 0, st, x,
                                   w, bias, y, p);
        } else {
            if (p.nbc == 1)
                hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC1, false, 1, 1, kNBR>), g1, dim3(kBlock), 0, st, x, w,
                                   bias, y, p);
            else if (p.nbr == 1)
                hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC1, false, 1, kNBC, 1>), g1, dim3(kBlock), 0, st, x, w,
                                   bias, y, p);
            else
                hipLaunchKernelGGL((igemm_dma_kernel<R, S, MB, CC1, false, 1, kNBC, kNBR>), g1, dim3(kBlock), 0, st, x,
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
        default: break;
    }
    // the factorized kernels of Inception-style blocks, plain convolution only
    if constexpr (!FUSED) {
        switch (rs) {
            case 1 * 16 + 3: return launch_mb<1, 3, false>(MB, p, grid, x, w, bias, y, ep, st);
            case 3 * 16 + 1: return launch_mb<3, 1, false>(MB, p, grid, x, w, bias, y, ep, st);
            case 1 * 16 + 7: return launch_mb<1, 7, false>(MB, p, grid, x, w, bias, y, ep, st);
            case 7 * 16 + 1: return launch_mb<7, 1, false>(MB, p, grid, x, w, bias, y, ep, st);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}

// kernel sizes of the fused chain's chunked kernel, and of the tile kernel,
// which adds the 1x3, 3x1, 1x7 and 7x1 of factorized (Inception-style) blocks
bool rs_fused_instantiated(int R, int S) {
    return (R == 1 && S == 1) || (R == 3 && S == 3) || (R == 5 && S == 5) || (R == 5 && S == 9) ||
           (R == 7 && S == 7);
}

bool rs_instantiated(int R, int S) {
    return rs_fused_instantiated(R, S) || (R == 1 && (S == 3 || S == 7)) || (S == 1 && (R == 3 || R == 7));
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
    p.wvec = 0;
    p.ds = 0;
    return p;
}


// ---- Flattened-pixel launch

// below this fraction of useful lanes in the row x column tiles (per image),
// a narrow output takes flattened-pixel tiles.  Their band carries more rows
// per pixel (whole rows, the tallest tile's height) and they run one block
// per wave, so they pay only where the tiles waste more than a fifth of
// their lanes (measured on MI355X at batch 16: a 28-wide 32-channel-group
// 3x3 layer 63.7 -> 56.6 us and a 14-wide stride-2 one 65.9 -> 34.3 us,
// while 56-wide and 28-wide dense layers, their tiles 87.5 % full, ran
// 5-25 % slower flattened)
constexpr int kFlatBelowPercent = 80;
// two blocks per wave once the grid still has this many workgroups, or on
// reductions of this many channel chunks, whose length amortizes a
// workgroup's set-up and first loads, while the grid keeps one workgroup per
// CU (measured on MI355X, batch 16: a dilated 3x3 C256 28x28 layer, 32
// chunks, 214 -> 181 us at 392 instead of 784 workgroups; a 28x28
// 32-channel-group layer, 4 chunks, 48.1 -> 52.5 us the other way; a 1x7
// C160 17x17 layer, 20 chunks, 30.6 us at 185 workgroups, 49.2 at 95)
constexpr long long kFlatTwoBlockWorkgroups = 1024;
constexpr int kFlatTwoBlockChunks = 16;
constexpr long long kFlatTwoBlockMinWorkgroups = 256;
constexpr long long kFlatMaxLds = 64 * 1024;

// channels per chunk: as in the tile kernel (16 at 1x1 stride 1; 8 at 3x3
// and the 1x3, 3x1, 1x7 and 7x1 of factorized blocks), and 4 at 5x5, 2 at
// 7x7; 4 at 3x3 dilation 3 and 4, whose bands are taller
constexpr int flat_chunk_c(int R, int S, int ST, int DIL) {
    return R * S == 1 ? (ST == 1 ? 16 : 8)
                      : R * S <= 9 ? (ST == 1 && DIL <= 2 ? 8 : 4) : R * S <= 25 ? 4 : 2;
}

// Geometries with a flattened-pixel kernel: square 1x1 and 3x3 at stride 1
// and 2, 3x3 at dilation 2 (which the tile kernel does not take) and, at
// stride 1, dilation 3 and 4, 5x5 and 7x7 at stride 2, and the 1x3, 3x1, 1x7
// and 7x1 of factorized blocks at stride 1.  A 1x1 kernel's dilation changes
// nothing.
int flat_dil(const gconv_desc *d) { return d->R == 1 && d->S == 1 ? 1 : d->dil_h; }

bool flat_factorized(int R, int S) { return (R == 1 && (S == 3 || S == 7)) || (S == 1 && (R == 3 || R == 7)); }

bool flat_geometry(const gconv_desc *d) {
    if (d->stride_h != d->stride_w || d->dil_h != d->dil_w) return false;
    if (flat_factorized(d->R, d->S)) return d->stride_h == 1 && d->dil_h == 1;
    if (d->R != d->S) return false;
    if (d->stride_h != 1 && d->stride_h != 2) return false;
    const int dil = flat_dil(d);
    switch (d->R) {
        case 1: return true;
        case 3: return dil == 1 || dil == 2 || (d->stride_h == 1 && (dil == 3 || dil == 4));
        case 5:
        case 7: return dil == 1 && d->stride_h == 2;
        default: return false;
    }
}

// The flattened-pixel plan for NB blocks per wave, or false where it does
// not apply: other geometries, a band over 64 rows or over the LDS budget,
// offsets past int32.
bool flat_plan(const gconv_desc *d, int NB, bool vec, FlatParams &p) {
    const int ST = d->stride_h;
    if (!flat_geometry(d) || d->cout < 8) return false;
    const int dil = flat_dil(d);
    const long long T = 128LL * NB;
    const long long np = (long long)d->N * d->Ho * d->Wo;
    const long long xbytes = (long long)d->N * d->C * d->H * d->W * (long long)sizeof(float);
    if (np + T > INT_MAX || xbytes > INT_MAX - 64) return false;
    const int CC = flat_chunk_c(d->R, d->S, ST, dil);
    // band rows: T consecutive pixels span at most dmax + 1 output rows of
    // the batch; each step down a row moves ST virtual rows, and a step into
    // the next image hv - ST*Ho more (at most cross such steps); the last
    // pixel's kernel rows reach (R-1)*dil further
    const int hv = d->H + 2 * d->pad_h;
    const long long extra = std::max(0, hv - ST * d->Ho);
    const long long dmax = (d->Wo - 1 + T - 1) / d->Wo;
    const long long cross = (dmax + d->Ho - 1) / d->Ho;
    const long long tih = ST * dmax + cross * extra + (long long)(d->R - 1) * dil + 1;
    if (tih > 64) return false;
    const int ds = vec ? (4 - d->pad_w % 4) % 4 : 0;
    const int width = ST == 2 && !vec ? 2 * (d->Wo + (d->S - 1) * dil / 2) : ST * (d->Wo - 1) + (d->S - 1) * dil + 1 + ds;
    int lp = 2;
    while ((1 << lp) < width) ++lp;
    const int unit = vec ? 4 : 1;
    const long long band = (tih * CC) << lp;
    const long long xi = (band + 64 * unit - 1) / (64 * unit);
    if (xi > flat_max_band_insts(d->R, ST, dil, vec)) return false;
    const long long qp = (long long)CC * d->R * d->S;
    const long long wqp = (qp + 3) / 4 * 4 + (((qp + 3) / 4 * 4) % 8 == 0 ? 4 : 0);
    const long long wwords = (32 * wqp / 4 + 63) / 64 * 256;
    if (2 * xi * 64 * unit * (long long)sizeof(float) + 2 * wwords * (long long)sizeof(float) > kFlatMaxLds) return false;
    const long long n_tf = (np + T - 1) / T;
    const int n_kb = (d->cout + 31) / 32;
    const long long n_wg = (long long)d->groups * n_tf * n_kb;
    if (n_wg > INT_MAX) return false;
    p.C = d->C; p.H = d->H; p.W = d->W; p.K = d->K; p.Ho = d->Ho; p.Wo = d->Wo;
    p.pad_h = d->pad_h; p.pad_w = d->pad_w;
    p.cin = d->cin; p.cout = d->cout;
    p.n_kb = n_kb;
    p.G = d->groups; p.N = d->N;
    p.np = (int)np;
    p.howo = d->Ho * d->Wo;
    p.hv = hv;
    p.lp = lp;
    p.tih = (int)tih;
    p.ds = ds;
    p.xi = (int)xi;
    p.n_tf = (int)n_tf;
    p.n_wg = (int)n_wg;
    p.x_bytes = (int)(((long long)(d->N - 1) * d->C + d->cin) * d->H * d->W * (long long)sizeof(float));
    p.wvec = 0;
    return true;
}

template <int R, int S, int ST, int DIL>
hipError_t launch_flat_t(const FlatParams &p, bool vec, int nb, const float *x, const float *w, const float *bias,
                         float *y, hipStream_t st) {
    constexpr int CC = flat_chunk_c(R, S, ST, DIL);
    const size_t lds = 2 * (size_t)p.xi * 64 * (vec ? 4 : 1) * sizeof(float);
    const dim3 g1((unsigned)p.n_wg);
    clear_stale_launch_error();
    if (vec) {
        if (nb == 2)
            hipLaunchKernelGGL((igemm_flat_kernel<R, S, CC, true, ST, 2, DIL>), g1, dim3(kBlock), lds, st, x, w, bias, y, p);
        else
            hipLaunchKernelGGL((igemm_flat_kernel<R, S, CC, true, ST, 1, DIL>), g1, dim3(kBlock), lds, st, x, w, bias, y, p);
        return hipGetLastError();
    }
    if (nb == 2)
        hipLaunchKernelGGL((igemm_flat_kernel<R, S, CC, false, ST, 2, DIL>), g1, dim3(kBlock), lds, st, x, w, bias, y, p);
    else
        hipLaunchKernelGGL((igemm_flat_kernel<R, S, CC, false, ST, 1, DIL>), g1, dim3(kBlock), lds, st, x, w, bias, y, p);
    return hipGetLastError();
}

// Flattened-pixel tiles where the row x column tiles (area per image, in
// pixels; 0 where the tile kernel does not take the geometry) leave too many
// lanes idle and the plan applies; returns false to keep the tiles.
bool try_launch_flat(const gconv_desc *d, long long tile_area, const float *x, const float *w, const float *bias,
                     float *y, hipStream_t st, hipError_t *err) {
    if (tile_area > 0 && 100LL * d->Ho * d->Wo >= kFlatBelowPercent * tile_area) return false;
    // 16-byte band pieces unless their column shift widens the pitch (a
    // 28-wide 3x3 layer with padding 1 needs 33 columns for them, 30 for
    // 4-byte loads: 64 against 32, and measured 7 % slower)
    FlatParams p, pv, p4;
    // (or where only the 16-byte plan fits)
    const bool vec = d->W % 4 == 0 && (((uintptr_t)x & 15u) == 0) && flat_plan(d, 1, true, pv) &&
                     (!flat_plan(d, 1, false, p4) || pv.lp == p4.lp);
    int nb = 2;
    const int cc = flat_chunk_c(d->R, d->S, d->stride_h, flat_dil(d));
    const int nchunks = (d->cin + cc - 1) / cc;
    if (!flat_plan(d, 2, vec, p) ||
        (p.n_wg < kFlatTwoBlockWorkgroups && (nchunks < kFlatTwoBlockChunks || p.n_wg < kFlatTwoBlockMinWorkgroups))) {
        nb = 1;
        if (!flat_plan(d, 1, vec, p)) return false;
    }
    p.wvec = (d->cin * d->R * d->S) % 4 == 0 && (((uintptr_t)w & 15u) == 0);
    const bool s1 = d->stride_h == 1;
    const int dil = flat_dil(d);
    if (flat_factorized(d->R, d->S)) {
        const int rs = d->R * 16 + d->S;
        *err = rs == 1 * 16 + 3   ? launch_flat_t<1, 3, 1, 1>(p, vec, nb, x, w, bias, y, st)
               : rs == 3 * 16 + 1 ? launch_flat_t<3, 1, 1, 1>(p, vec, nb, x, w, bias, y, st)
               : rs == 1 * 16 + 7 ? launch_flat_t<1, 7, 1, 1>(p, vec, nb, x, w, bias, y, st)
                                  : launch_flat_t<7, 1, 1, 1>(p, vec, nb, x, w, bias, y, st);
        return true;
    }
    switch (d->R) {
        case 1:
            *err = s1 ? launch_flat_t<1, 1, 1, 1>(p, vec, nb, x, w, bias, y, st)
                      : launch_flat_t<1, 1, 2, 1>(p, vec, nb, x, w, bias, y, st);
            break;
        case 3:
            if (dil == 4)
                *err = launch_flat_t<3, 3, 1, 4>(p, vec, nb, x, w, bias, y, st);
            else if (dil == 3)
                *err = launch_flat_t<3, 3, 1, 3>(p, vec, nb, x, w, bias, y, st);
            else if (dil == 2)
                *err = s1 ? launch_flat_t<3, 3, 1, 2>(p, vec, nb, x, w, bias, y, st)
                          : launch_flat_t<3, 3, 2, 2>(p, vec, nb, x, w, bias, y, st);
            else
                *err = s1 ? launch_flat_t<3, 3, 1, 1>(p, vec, nb, x, w, bias, y, st)
                          : launch_flat_t<3, 3, 2, 1>(p, vec, nb, x, w, bias, y, st);
            break;
        case 5: *err = launch_flat_t<5, 5, 2, 1>(p, vec, nb, x, w, bias, y, st); break;
        default: *err = launch_flat_t<7, 7, 2, 1>(p, vec, nb, x, w, bias, y, st); break;
    }
    return true;
}

}  // namespace

namespace {

// The tile kernels (and the fused chain's chunked kernel): dilation 1,
// stride 1, or stride 2 on both axes at 1x1, 3x3, 5x5 and 7x7.
bool igemm_tile_supported(const gconv_desc *d) {
    // buffer offsets are signed 32-bit: one group's input channels of one
    // image must stay below 2 GB.  Any number of input channels: a chunk's
    // channels past C/G read zero (a 3-channel first layer fills 3 of a
    // 4-channel chunk).
    const bool stride_ok = d->stride_h == d->stride_w &&
                           (d->stride_h == 1 ||
                            (d->stride_h == 2 && d->R == d->S && (d->R == 1 || d->R == 3 || d->R == 5 || d->R == 7)));
    return stride_ok && d->dil_h == 1 && d->dil_w == 1 && rs_instantiated(d->R, d->S) && d->cin >= 1 &&
           d->cout >= 8 && (long long)d->cin * d->H * d->W * (long long)sizeof(float) < 0x7fffffffLL - 64;
}

// Geometries only the flattened-pixel kernel takes (3x3 at dilation 2 to 4,
// 5x5 and 7x7 at stride 2), where its plan fits: with 16-byte band pieces when W
// is a multiple of 4 (a call whose x is not 16-byte aligned, and whose
// 4-byte plan does not fit, runs the direct kernel), else with 4-byte loads.
bool igemm_flat_only(const gconv_desc *d) {
    FlatParams p;
    return !igemm_tile_supported(d) && (flat_plan(d, 1, false, p) || (d->W % 4 == 0 && flat_plan(d, 1, true, p)));
}

}  // namespace

bool igemm_supported(const gconv_desc *d) { return igemm_tile_supported(d) || igemm_flat_only(d); }

bool igemm_fused_supported(const gconv_desc *d, int gn_groups) {
    // every output channel of every 32*MB block must exist, and a GroupNorm
    // group must be 4 channels
    // (the fused kernel runs at stride 1 only)
    // its grid is (tiles, group x channel block, n), within the hardware's
    // 65535 limit on y and z
    const long long gy = (long long)d->groups * ((d->cout + 32 * pick_mb(d) - 1) / (32 * pick_mb(d)));
    return igemm_tile_supported(d) && rs_fused_instantiated(d->R, d->S) && d->cin >= 4 && d->stride_h == 1 && d->cout % (32 * pick_mb(d)) == 0 && d->K / gn_groups == 4 &&
           gy <= 65535 && d->N <= 65535;
}

int igemm_fused_parts_per_group(const gconv_desc *d, int) {
    return make_params(d, pick_mb(d)).n_tiles;
}

hipError_t launch_igemm(const gconv_desc *d, const float *x, const float *w, const float *bias,
                        float *y, hipStream_t st) {
    if (!igemm_supported(d)) return hipErrorInvalidValue;
    if (!igemm_tile_supported(d)) {
        hipError_t err = hipErrorInvalidValue;
        if (!try_launch_flat(d, 0, x, w, bias, y, st, &err)) return launch_direct(d, x, w, bias, y, st);
        return err;
    }
    // one 32-channel block per workgroup (kPlainMB): each input band is
    // read once per block, in exchange for no register spills
    const int MB = kPlainMB == 2 ? pick_mb(d) : 1;
    IgParams p = make_params(d, MB);
    // 16-byte band loads: at stride 1 when W and the padding are multiples of
    // 4, at stride 2 when W is (the band then starts pad_w + ds columns left
    // of 2*ow0, a 16-byte boundary)
    p.vec = (d->W % 4 == 0) && (((uintptr_t)x & 15u) == 0) && (d->stride_h == 2 || d->pad_w % 4 == 0);
    p.ds = d->stride_h == 2 ? (4 - d->pad_w % 4) % 4 : 0;
    p.wvec = (d->cin * d->R * d->S) % 4 == 0 && (((uintptr_t)w & 15u) == 0);
    // the DMA kernel's tile: 8 rows (4 at stride 2) by 64 columns, or by one
    // 32-column block on outputs at most 32 wide; 4 rows as well when 8-row
    // tiles would leave fewer than two workgroups per CU (more, smaller
    // workgroups keep more loads in flight)
    p.nbc = d->Wo <= 32 ? 1 : kNBC;
    p.nbr = d->stride_h == 2 ? 1 : kNBR;
    // kernels 3 wide at stride 1 on 64-column tiles take Winograd columns,
    // which run one row per wave
    if (kIgWinograd && d->S == 3 && (d->R == 1 || d->R == 3) && d->stride_h == 1 && p.nbc == kNBC) p.nbr = 1;
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
    hipError_t err = hipSuccess;
    if (try_launch_flat(d, (long long)p.n_tiles * (4 * p.nbr) * (32 * p.nbc), x, w, bias, y, st, &err)) return err;
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
