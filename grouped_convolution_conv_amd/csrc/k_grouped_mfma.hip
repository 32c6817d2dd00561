// k_grouped_mfma.hip -- grouped 3x3 convolution (stride 1, padding 1,
// dilation 1) with 16 input and 16 output channels per group on the FP32
// matrix cores.
//
// The grouped convolution of the GroupConv Atlas page, at the width where
// its per-group sum (16 channels x 9 taps = 144 products per output) makes
// the vector-FMA kernels bound by their arithmetic: on gfx950 the non-packed
// FP32 VALU runs at half the FP32 matrix rate.  Per group the convolution is
// a small GEMM, D[k][p] = sum_q W[k][q] X[q][p], with k the group's 16 output
// channels, p output pixels and q = (input channel, tap); it maps onto
// v_mfma_f32_16x16x4f32 exactly (M = 16 output channels, N = 16 pixels along
// a row, K = 4 input channels at one tap), so no MFMA row is idle.
//
// Two kernels.  grouped16_mfma_lds_kernel (W a multiple of 4, x 16-byte
// aligned) loads a workgroup's band straight into LDS with 16-byte buffer
// loads and reads every B operand from LDS.  grouped16_mfma_kernel (any
// other W or alignment) reads B straight from memory, described next.
// Measured on the 16 cpg-16 shapes of the grouped 3x3 grid, the two beat the
// VALU register kernel everywhere (N8 C256 112x112: 78 us against 126;
// N8 C256 14x14: 6.5 against 18.9); the direct-load form alone was slower
// than the VALU kernel at N8 C256 112x112 (129 against 125 us): its dword
// load per B operand keeps the texture address units and the load latency,
// not the matrix cores, in charge.
//
// grouped16_mfma_kernel's data movement follows the register kernel of
// k_grouped3x3.hip: no LDS, no barriers.  A wave owns RB = 2 output rows x NB blocks of 16 columns of one
// (image, group).  Its 36 A operands (the group's weights, lane = (output
// channel, input channel within a quad)) are loaded once.  Its B operands
// are read straight from the input with buffer loads: lane (kq, j) of a load
// reads channel 4q + kq, column (block start + j + s - 1) of one input row,
// one load per (row, block, shift s).  The per-lane part of every offset
// (channel within the quad, column) is computed once; the row and the
// channel quad go in the instruction's scalar offset, so a load costs no
// vector instruction.  Columns outside the image get an offset beyond the
// buffer (the hardware returns zero: the padding), and a row outside the
// image gets a scalar offset beyond it.  The next quad's loads are issued
// before the current quad's 72 MFMAs.  The 3 loads of an input row (one per
// shift) hit the L1; the halo rows shared by neighbouring waves come from
// the L2.
#include "dev_common.h"
#include "internal.h"

namespace gconv {
namespace {

constexpr int kBlock = 256;
constexpr int kBufferWord3 = 0x00020000;     // raw 32-bit buffer access, gfx9 family
constexpr int kOutOfRange = 0x7fffffff;      // a per-lane offset beyond every range
constexpr int kRowOutOfRange = 0x40000000;   // a scalar offset beyond every range (images < 1 GB)
constexpr int kRB = 2;                       // output rows per wave


typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

struct GmParams {
    int C, H, W, K, G;
    int n_seg;    // column segments (NB blocks of 16) per row
    int n_rp;     // row pairs per image
    int units;    // waves: N * G * n_rp * n_seg
};

template <int NB>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void grouped16_mfma_kernel(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ y, GmParams p) {
    const int lane = threadIdx.x & 63;
    const int unit = __builtin_amdgcn_readfirstlane((int)blockIdx.x * (kBlock / 64) + (int)(threadIdx.x >> 6));
    if (unit >= p.units) return;  // whole waves only
    // wave -> (image, group, row pair, column segment), segment fastest
    const int seg = unit % p.n_seg;
    int t = unit / p.n_seg;
    const int rp = t % p.n_rp;
    t /= p.n_rp;
    const int g = t % p.G, n = t / p.G;
    const int oh0 = kRB * rp, ow0 = 16 * NB * seg;
    const int j = lane & 15, kq = lane >> 4;
    const int HW = p.H * p.W;

    // A operands: lane (row j, k = kq) of the quad-q, tap-t MFMA holds the
    // weight of output channel g*16 + j for input channel 4q + kq
    float A[4][9];
    {
        const float *wl = w + ((size_t)(g * 16 + j) * 16 + kq) * 9;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int tp = 0; tp < 9; ++tp) A[q][tp] = wl[q * 36 + tp];
    }

    // the group's 16 input planes
    const __amdgpu_buffer_rsrc_t xs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(x + ((size_t)n * p.C + (size_t)g * 16) * HW), (short)0, 16 * HW * (int)sizeof(float),
        kBufferWord3);
    // per-lane offsets of (block b, shift s): channel kq of the quad, column
    // ow0 + 16b + j + s - 1; beyond the buffer outside the image
    int co[NB][3];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            const int iw = ow0 + 16 * b + j + s - 1;
            co[b][s] = (iw >= 0 && iw < p.W) ? (kq * HW + iw) * (int)sizeof(float) : kOutOfRange;
        }
    // scalar part of a load: channel quad q, input row oh0 - 1 + i
    auto soff = [&](int q, int i) __attribute__((always_inline)) {
        const int ih = oh0 - 1 + i;
        return (ih >= 0 && ih < p.H) ? (4 * q * HW + ih * p.W) * (int)sizeof(float) : kRowOutOfRange;
    };

    // accumulators start at the bias: register v of block b holds output
    // channel g*16 + 4kq + v at column ow0 + 16b + j
    floatx4 acc[kRB][NB];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const float bv = bias ? bias[g * 16 + 4 * kq + v] : 0.0f;
#pragma unroll
        for (int rr = 0; rr < kRB; ++rr)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[rr][b][v] = bv;
    }

    constexpr int NIR = kRB + 2;  // input rows
    float B0[NIR][NB][3], B1[NIR][NB][3];
    auto load = [&](float (&B)[NIR][NB][3], int q) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NIR; ++i) {
            const int so = soff(q, i);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int s = 0; s < 3; ++s)
                    B[i][b][s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xs, co[b][s], so, 0));
        }
    };
    auto mma = [&](const float (&B)[NIR][NB][3], int q) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 3; ++r)
#pragma unroll
            for (int s = 0; s < 3; ++s)
#pragma unroll
                for (int rr = 0; rr < kRB; ++rr)
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        acc[rr][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[q][r * 3 + s], B[rr + r][b][s],
                                                                          acc[rr][b], 0, 0, 0);
    };
    load(B0, 0);
    load(B1, 1);
    mma(B0, 0);
    load(B0, 2);
    mma(B1, 1);
    load(B1, 3);
    mma(B0, 2);
    mma(B1, 3);

    // stores: the pixel in the per-lane offset (beyond the range outside
    // the output), the register's channel in the scalar offset
    const __amdgpu_buffer_rsrc_t ys = __builtin_amdgcn_make_buffer_rsrc(
        y + ((size_t)n * p.K + (size_t)g * 16) * HW, (short)0, 16 * HW * (int)sizeof(float), kBufferWord3);
#pragma unroll
    for (int rr = 0; rr < kRB; ++rr) {
        const int oh = oh0 + rr;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int ow = ow0 + 16 * b + j;
            const int vo = (oh < p.H && ow < p.W) ? ((4 * kq) * HW + oh * p.W + ow) * (int)sizeof(float)
                                                  : kRowOutOfRange;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                // copy the element out first: a bit cast applied to the
                // vector element expression itself reads element 0
                const float val = acc[rr][b][v];
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, val), ys, vo,
                                                      v * HW * (int)sizeof(float), 0);
            }
        }
    }
}

// LDS-staged form (W a multiple of 4 and x 16-byte aligned): a workgroup of
// 4 waves owns 4*RBW output rows x 16*NBW columns of one (image, group);
// RBW = 1 output row per wave, NBW = 4 blocks of 16 columns, 2 on rows at
// most 32 wide (a 28-wide row filled 28 of 64 columns), or 7 on 112-wide
// rows of large grids.  Its band (the group's 16 channels x 4*RBW + 2 input
// rows x 16*NBW + 8 columns from column ow0 - 4, in whole 16-byte pieces)
// goes straight from memory into LDS by buffer loads with the LDS bit (lane
// l of an instruction writes its 16 bytes at the instruction's LDS base +
// 16 l; pieces outside the image read zero), channels 0-7 first, then 8-15.  Each
// wave waits for its own first half (the loads count down in issue order),
// one barrier admits quads 0 and 1 while channels 8-15 land, a second one
// quads 2 and 3; every B operand is an LDS read at a compile-time offset
// from the lane's base.
//
// An earlier form staged the band through registers (48 of its 140 VGPRs),
// which held it to three waves per SIMD with 8-row tiles; with no register
// holding the band, 4-row tiles use 81 VGPRs and 32 KB of LDS, five
// workgroups per CU (measured on MI355X, cold buffers: N8 C256 112x112 86.1
// -> 83.3 us, 56x56 27.4 -> 25.0, N1 C64 56x56 8.5 -> 6.1; 8-row tiles in the
// same form, three per CU by LDS, were no faster than before).
constexpr int kG16RowsPerWave = 1;
constexpr long long kG16WideRowWorkgroups = 1024;

struct GlParams {
    int C, H, W, K, G;
    int n_seg;    // column segments (16*NBW columns) per row
    int n_rb;     // row blocks (4 * kG16RowsPerWave rows) per image
    int wgs;      // workgroups: N * G * n_rb * n_seg
};

template <int RBW, int NBW>
__global__ __launch_bounds__(kBlock) void grouped16_mfma_lds_kernel(const float *__restrict__ x,
                                                                    const float *__restrict__ w,
                                                                    const float *__restrict__ bias,
                                                                    float *__restrict__ y, GlParams p) {
    constexpr int TH = 4 * RBW;
    constexpr int LROWS = TH + 2;
    constexpr int PITCH = 16 * NBW + 8;                     // band row: columns ow0-4 .. ow0+16*NBW+3
    constexpr int P4 = PITCH / 4;                           // 16-byte pieces per band row
    constexpr int HPIECES = 8 * LROWS * P4;                 // pieces of a half band (8 channels)
    constexpr int HI = ((HPIECES + 63) / 64 + 3) / 4 * 4;  // DMA instructions per half, whole rounds of 4 waves
    constexpr int HIW = HI / 4;                             // per wave and half
    __shared__ float4 band4[2 * HI * 64];
    const float *band = reinterpret_cast<const float *>(band4);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    // workgroup -> (image, group, row block, column segment), segment
    // fastest, XCD-aware: the hardware deals consecutive workgroup ids to the
    // 8 XCDs in turn, so each XCD is given a contiguous run of tiles instead,
    // and vertically neighbouring tiles, whose bands share two halo rows,
    // run on one XCD close in time
    const int L = blockIdx.x;
    const int xcd = L & 7, slot = L >> 3;
    const int per = p.wgs >> 3, rem = p.wgs & 7;
    int t = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    const int seg = t % p.n_seg;
    t /= p.n_seg;
    const int rb = t % p.n_rb;
    t /= p.n_rb;
    const int g = t % p.G, n = t / p.G;
    const int oh0 = TH * rb, ow0 = 16 * NBW * seg;
    const int j = lane & 15, kq = lane >> 4;
    const int HW = p.H * p.W;

    // A operands and the bias first (waited for with the first half)
    float A[4][9];
    {
        const float *wl = w + ((size_t)(g * 16 + j) * 16 + kq) * 9;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int tp = 0; tp < 9; ++tp) A[q][tp] = wl[q * 36 + tp];
    }
    const __amdgpu_buffer_rsrc_t bs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(bias ? bias + g * 16 : w), (short)0, bias ? 16 * (int)sizeof(float) : 0, kBufferWord3);
    float bv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        bv[v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(bs, (4 * kq + v) * (int)sizeof(float), 0, 0));
    __builtin_amdgcn_sched_barrier(0);

    // ---- band: half hf holds channels 8hf..8hf+7; its piece f =
    //      (c * LROWS + lr) * P4 + c4 holds input columns ow0 - 4 + 4c4 .. +3
    //      of row oh0 - 1 + lr, channel 8hf + c
    const __amdgpu_buffer_rsrc_t xs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(x + ((size_t)n * p.C + (size_t)g * 16) * HW), (short)0, 16 * HW * (int)sizeof(float),
        kBufferWord3);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int ti = 0; ti < HIW; ++ti) {
            const int ii = ti * 4 + wv;
            const int f = ii * 64 + lane;
            const int c = f / (LROWS * P4), r2 = f - c * (LROWS * P4);
            const int lr = r2 / P4, c4 = r2 - lr * P4;
            const int ih = oh0 - 1 + lr, iw = ow0 - 4 + 4 * c4;
            const bool ok = f < HPIECES && ih >= 0 && ih < p.H && iw >= 0 && iw < p.W;
            const int off = ok ? ((8 * hf + c) * HW + ih * p.W + iw) * (int)sizeof(float) : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xs, (lds_void_t *)(band4 + (hf * HI + ii) * 64), 16, off, 0,
                                                     0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    floatx4 acc[RBW][NBW];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int rr = 0; rr < RBW; ++rr)
#pragma unroll
            for (int b = 0; b < NBW; ++b) acc[rr][b][v] = bv[v];

    // ---- MFMAs: B of (quad q, output row rr, tap (r, s), block b) is band
    //      half q/2, channel 4(q%2) + kq, row RBW*wave + rr + r, column
    //      16b + j + s - 1 + 4
    const float *bl = band + (kq * LROWS + RBW * wave) * PITCH + j + 3;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        // The waits and barriers are written out: a workgroup-scope release
        // fence before the barrier would make the compiler wait for every
        // load that writes LDS, the second half's too.  A load with the LDS bit
        // counts down once its data is in LDS, and the memory clobber keeps
        // the LDS reads below the barrier.
        if (q == 0) {
            // this wave's first half has landed (its second half's HIW loads
            // may still be in flight); after the barrier, every wave's has
            static_assert(HIW == 2 || HIW == 4 || HIW == 6, "a wait count for this tile");
            if constexpr (HIW == 2)
                asm volatile("s_waitcnt vmcnt(2)\n\ts_barrier" ::: "memory");
            else if constexpr (HIW == 4)
                asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
            else
                asm volatile("s_waitcnt vmcnt(6)\n\ts_barrier" ::: "memory");
        }
        if (q == 2) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        float B[RBW + 2][NBW][3];
#pragma unroll
        for (int i = 0; i < RBW + 2; ++i)
#pragma unroll
            for (int b = 0; b < NBW; ++b)
#pragma unroll
                for (int s = 0; s < 3; ++s)
                    B[i][b][s] = bl[(q >> 1) * HI * 256 + (4 * (q & 1) * LROWS + i) * PITCH + 16 * b + s];
#pragma unroll
        for (int r = 0; r < 3; ++r)
#pragma unroll
            for (int s = 0; s < 3; ++s)
#pragma unroll
                for (int rr = 0; rr < RBW; ++rr)
#pragma unroll
                    for (int b = 0; b < NBW; ++b)
                        acc[rr][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(A[q][r * 3 + s], B[rr + r][b][s],
                                                                          acc[rr][b], 0, 0, 0);
    }

    // ---- stores, as in grouped16_mfma_kernel
    const __amdgpu_buffer_rsrc_t ys = __builtin_amdgcn_make_buffer_rsrc(
        y + ((size_t)n * p.K + (size_t)g * 16) * HW, (short)0, 16 * HW * (int)sizeof(float), kBufferWord3);
#pragma unroll
    for (int rr = 0; rr < RBW; ++rr) {
        const int oh = oh0 + RBW * wave + rr;
#pragma unroll
        for (int b = 0; b < NBW; ++b) {
            const int ow = ow0 + 16 * b + j;
            const int vo = (oh < p.H && ow < p.W) ? ((4 * kq) * HW + oh * p.W + ow) * (int)sizeof(float)
                                                  : kRowOutOfRange;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float val = acc[rr][b][v];  // see grouped16_mfma_kernel
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, val), ys, vo,
                                                      v * HW * (int)sizeof(float), 0);
            }
        }
    }
}

template <int NB>
hipError_t launch_nb(const GmParams &p, const float *x, const float *w, const float *bias, float *y,
                     hipStream_t st) {
    const int grid = (p.units + kBlock / 64 - 1) / (kBlock / 64);
    clear_stale_launch_error();
    hipLaunchKernelGGL((grouped16_mfma_kernel<NB>), dim3(grid), dim3(kBlock), 0, st, x, w, bias, y, p);
    return hipGetLastError();
}

// blocks of 16 columns per wave: 4, or fewer when the row is narrow
int pick_nb(int W) { return W > 32 ? 4 : (W > 16 ? 2 : 1); }

bool plan(const gconv_desc *d, int NB, GmParams *p) {
    p->C = d->C; p->H = d->H; p->W = d->W; p->K = d->K; p->G = d->groups;
    p->n_seg = (d->W + 16 * NB - 1) / (16 * NB);
    p->n_rp = (d->H + kRB - 1) / kRB;
    const long long units = (long long)d->N * d->groups * p->n_rp * p->n_seg;
    if (units > 0x7fffffffLL - 64) return false;
    p->units = (int)units;
    return true;
}

}  // namespace

bool grouped16_mfma_applies(const gconv_desc *d) {
    if (!(d->R == 3 && d->S == 3 && d->stride == 1 && d->pad == 1 && d->dil == 1 && d->cin == 16 &&
          d->cout == 16 && d->groups > 1))
        return false;
    // 32-bit buffer offsets: a group's 16 planes stay below 1 GB
    if ((long long)16 * d->H * d->W * (long long)sizeof(float) >= kRowOutOfRange) return false;
    GmParams p;
    return plan(d, pick_nb(d->W), &p);
}

hipError_t launch_grouped16_mfma(const gconv_desc *d, const float *x, const float *w, const float *bias,
                                 float *y, hipStream_t st) {
    if (d->W % 4 == 0 && ((uintptr_t)x & 15u) == 0) {
        GlParams q;
        q.C = d->C; q.H = d->H; q.W = d->W; q.K = d->K; q.G = d->groups;
        // blocks of 16 columns per wave: 2 on rows at most 32 wide; 7 on rows
        // of 97-112 columns (one segment, not two of 64 with 16 idle) when
        // the grid still has kG16WideRowWorkgroups workgroups (measured: N8
        // C256 112x112 83.4 -> 77.6 us, while N1 C64 112x112, 112
        // workgroups, went 6.6 -> 8.5 us); else 4
        q.n_rb = (d->H + 4 * kG16RowsPerWave - 1) / (4 * kG16RowsPerWave);
        int nbw = d->W <= 32 ? 2 : 4;
        if (d->W > 96 && d->W <= 112 && (long long)d->N * d->groups * q.n_rb >= kG16WideRowWorkgroups) nbw = 7;
        q.n_seg = (d->W + 16 * nbw - 1) / (16 * nbw);
        const long long wgs = (long long)d->N * d->groups * q.n_rb * q.n_seg;
        if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        q.wgs = (int)wgs;
        clear_stale_launch_error();
        if (nbw == 7)
            hipLaunchKernelGGL((grouped16_mfma_lds_kernel<kG16RowsPerWave, 7>), dim3((unsigned)q.wgs), dim3(kBlock), 0,
                               st, x, w, bias, y, q);
        else if (nbw == 2)
            hipLaunchKernelGGL((grouped16_mfma_lds_kernel<kG16RowsPerWave, 2>), dim3((unsigned)q.wgs), dim3(kBlock), 0,
                               st, x, w, bias, y, q);
        else
            hipLaunchKernelGGL((grouped16_mfma_lds_kernel<kG16RowsPerWave, 4>), dim3((unsigned)q.wgs), dim3(kBlock), 0,
                               st, x, w, bias, y, q);
        return hipGetLastError();
    }
    const int NB = pick_nb(d->W);
    GmParams p;
    if (!plan(d, NB, &p)) return hipErrorInvalidConfiguration;
    if (NB == 4) return launch_nb<4>(p, x, w, bias, y, st);
    if (NB == 2) return launch_nb<2>(p, x, w, bias, y, st);
    return launch_nb<1>(p, x, w, bias, y, st);
}

}  // namespace gconv
