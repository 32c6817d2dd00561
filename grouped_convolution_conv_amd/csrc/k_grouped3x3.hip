// k_grouped3x3.hip -- grouped / depthwise 3x3, stride 1, pad 1, dilation 1,
// with 1, 2 or 4 input channels per group (the workload of the GroupConv
// Atlas page), and 8 or 16 on the register kernel.  VALU arithmetic,
// HBM-bound up to 4 channels per group, FMA-bound beyond.
//
// Two kernels:
//  - grouped3x3_rows_kernel (W a multiple of 4, W <= 256, 16-byte aligned
//    tensors): register streaming with no LDS and no barriers.  A lane owns
//    RB rows x 4 columns of one (n, group, block of up to 4 output channels)
//    plane, reads its 4-column piece of every input row it needs with one
//    16-byte load, and takes the columns to its left and right from the
//    neighbouring lanes.  This is the Atlas page's fourth kernel (several
//    neighbouring outputs per thread, sharing the overlapping input windows)
//    turned 2-D and widened over output channels, with the page's shared
//    halo tile left to the L2: on gfx950 the occupancy that no LDS
//    allocation buys is worth more than the reuse an LDS tile would add.
//  - grouped3x3_kernel (any other W or alignment): one workgroup stages a
//    band of input rows with a one-pixel zero halo in LDS (the cooperative
//    halo tile of the Atlas page's third kernel) using batches of
//    independent 128-bit loads, then each lane computes Q = 4 or 8
//    neighbouring outputs along W for up to 4 output channels, reading its
//    window of Q+2 inputs per row as b32 + Q/4 x b128 + b32 and the weights
//    as LDS broadcasts.  The W tail is masked.
#include "dev_common.h"
#include "internal.h"

namespace gconv {
namespace {

constexpr int kBlock = 256;
constexpr int kBatch = 8;   // global loads in flight per lane during staging
constexpr int kLead = 4;    // LDS index of interior column 0
// buffer resource descriptor word 3 for raw (untyped, unswizzled) 32-bit
// access on gfx9-family GPUs, and a byte offset no plane reaches (reads 0)
constexpr int kBufferWord3 = 0x00020000;
constexpr int kOutOfPlane = 0x7fffffff;
constexpr int kSmallWaves = 256;    // below this many waves at 2 rows per lane, use 1
constexpr int kLargeWaves = 8192;   // depthwise with at least this many waves at 4 rows per lane uses 4
constexpr int kWideWaves = 1536;    // halve the output channels per lane below this many waves
constexpr int kWideBlocks = 512;    // the same for the LDS band kernel's workgroups
constexpr size_t kWideBandLds = 64 * 1024;  // largest LDS band a wide group may stage

struct G3Params {
    int C, H, W, K;
    int cout;       // output channels per group
    int n_cob;      // output-channel blocks per group (cout / CO)
    int BH, TW;     // band height (rows) and width (columns, multiple of Q)
    int n_cb;       // column bands
    int pitch;      // LDS row pitch in floats (multiple of 4, >= TW + 5)
    int vec_load;   // W % 4 == 0 and x 16-byte aligned: 128-bit staging loads
    int vec_store;  // W % 4 == 0 and y 16-byte aligned
};

template <int CI, int CO, int Q>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void grouped3x3_kernel(const float *__restrict__ x,
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
    const int rows = p.BH + 2;                 // staged rows per channel
    const int nrows = CI * rows;               // staged rows in total
    const size_t HW = (size_t)p.H * p.W;
    const float *xg = x + ((size_t)n * p.C + (size_t)g * CI) * HW;
    const int k0 = g * p.cout + cob * CO;
    float *wl = lds + nrows * p.pitch;         // [CI][CO][9] weights of the block

    // ---- weights of the block (CO*CI*9 floats, contiguous in w)
    for (int e = tid; e < CO * CI * 9; e += kBlock) {
        const int co = e / (CI * 9), rem = e - co * (CI * 9);
        const int ci = rem / 9, t = rem - ci * 9;
        wl[(ci * CO + co) * 9 + t] = w[(size_t)k0 * CI * 9 + e];
    }

    // ---- interior columns [c0, c0 + TW) of every staged row
    const int tw = min(p.TW, p.W - c0);        // columns that exist
    if (p.vec_load) {
        const int per_row = p.TW >> 2;           // float4 slots per row
        const int total = nrows * per_row;
        for (int base = tid; base < total; base += kBatch * kBlock) {
            float4 v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int e = base + u * kBlock;
                v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (e < total) {
                    const int row = e / per_row, c4 = (e - row * per_row) << 2;
                    const int ci = row / rows, ih = oh0 - 1 + (row - ci * rows);
                    if (ih >= 0 && ih < p.H && c4 < tw)
                        v[u] = *reinterpret_cast<const float4 *>(xg + ci * HW + (size_t)ih * p.W + c0 + c4);
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int e = base + u * kBlock;
                if (e < total) {
                    const int row = e / per_row, c4 = (e - row * per_row) << 2;
                    *reinterpret_cast<float4 *>(lds + row * p.pitch + kLead + c4) = v[u];
                }
            }
        }
    } else {
        const int total = nrows * p.TW;
        for (int base = tid; base < total; base += kBatch * kBlock) {
            float v[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int e = base + u * kBlock;
                v[u] = 0.0f;
                if (e < total) {
                    const int row = e / p.TW, c = e - row * p.TW;
                    const int ci = row / rows, ih = oh0 - 1 + (row - ci * rows);
                    if (ih >= 0 && ih < p.H && c < tw) v[u] = xg[ci * HW + (size_t)ih * p.W + c0 + c];
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int e = base + u * kBlock;
                if (e < total) {
                    const int row = e / p.TW, c = e - row * p.TW;
                    lds[row * p.pitch + kLead + c] = v[u];
                }
            }
        }
    }
    // ---- halo columns c0 - 1 and c0 + TW (zero outside the image)
    for (int e = tid; e < 2 * nrows; e += kBlock) {
        const int row = e >> 1, right = e & 1;
        const int ci = row / rows, ih = oh0 - 1 + (row - ci * rows);
        const int iw = right ? c0 + p.TW : c0 - 1;
        float v = 0.0f;
        if (ih >= 0 && ih < p.H && iw >= 0 && iw < p.W) v = xg[ci * HW + (size_t)ih * p.W + iw];
        lds[row * p.pitch + (right ? kLead + p.TW : kLead - 1)] = v;
    }
    __syncthreads();

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

        // one input channel per iteration: unrolling this loop as well lets
        // the scheduler hoist every window and weight read of all channels
        // and run out of registers
#pragma unroll 1
        for (int ci = 0; ci < CI; ++ci) {
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                // window: input columns ow-1 .. ow+Q of row oh-1+r
                const float *src = lds + (ci * rows + lr + r) * p.pitch + kLead + jq;
                float win[Q + 2];
                win[0] = src[-1];
#pragma unroll
                for (int q = 0; q < Q; q += 4) {
                    const float4 v = *reinterpret_cast<const float4 *>(src + q);
                    win[q + 1] = v.x; win[q + 2] = v.y; win[q + 3] = v.z; win[q + 4] = v.w;
                }
                win[Q + 1] = src[Q];
                float wv[CO][3];
#pragma unroll
                for (int co = 0; co < CO; ++co)
#pragma unroll
                    for (int s = 0; s < 3; ++s) wv[co][s] = wl[(ci * CO + co) * 9 + r * 3 + s];
#pragma unroll
                for (int co = 0; co < CO; ++co)
#pragma unroll
                    for (int s = 0; s < 3; ++s)
#pragma unroll
                        for (int q = 0; q < Q; ++q) acc[co][q] = fmaf(win[q + s], wv[co][s], acc[co][q]);
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

// ---------------------------------------------------------------------------
// Register variant (W % 4 == 0, W <= 256, 16-byte aligned tensors): no LDS
// and no barriers.  Each wave owns a set of whole image rows of one
// (n, group, channel block) plane; a lane owns RB rows x 4 columns of the
// plane for the CO output channels of the block.  It reads its 4-column
// piece of each of the RB+2 input rows it needs straight from global memory
// into registers (one 16-byte load per row and input channel, coalesced
// along the row), takes the column to its left and right from the
// neighbouring lanes with cross-lane moves, and accumulates every 3x3 tap
// it touches.  The halo rows that neighbouring lanes and waves share come
// from the L2, so HBM sees each input byte about once.  With no LDS the
// occupancy is set by registers alone and every wave streams on its own.

struct G3Rows {
    int C, H, W, K, G;
    int cout, n_cob;
    int cg;       // 4-column groups per row (W / 4)
    int rpw;      // lane strips (of RB rows) per wave: 64 / cg
    int strips;   // strips per plane: ceil(H / RB)
    int wpp;      // waves per plane: ceil(strips / rpw)
    int waves;    // N * G * n_cob * wpp
};

template <int CI, int CO, int RB>
__global__ __launch_bounds__(kBlock) void grouped3x3_rows_kernel(const float *__restrict__ x,
                                                                 const float *__restrict__ w,
                                                                 const float *__restrict__ bias,
                                                                 float *__restrict__ y, G3Rows p) {
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)blockIdx.x * (kBlock / 64) + (int)(threadIdx.x >> 6));
    if (wv >= p.waves) return;  // whole waves only
    // wave -> (n, group, wave in plane, channel block), channel block
    // fastest: the blocks that read the same input rows are neighbouring
    // waves of one workgroup, so they run together on one XCD and share its
    // L2 instead of each fetching the rows from memory
    const int cob = wv % p.n_cob;
    const int t0 = wv / p.n_cob;
    const int wip = t0 % p.wpp;
    const int t = t0 / p.wpp;
    const int g = t % p.G, n = t / p.G;
    const int sl = lane / p.cg, cgi = lane - sl * p.cg;
    const int strip = wip * p.rpw + sl;
    const bool active = sl < p.rpw && strip < p.strips;
    const int r0 = strip * RB, c0 = cgi * 4;
    const bool has_left = cgi > 0, has_right = cgi < p.cg - 1;
    const size_t HW = (size_t)p.H * p.W;
    const float *xg = x + ((size_t)n * p.C + (size_t)g * CI) * HW + c0;
    const int k0 = g * p.cout + cob * CO;

    float acc[CO][RB][4];
#pragma unroll
    for (int co = 0; co < CO; ++co) {
        const float b = bias ? bias[k0 + co] : 0.0f;
#pragma unroll
        for (int rr = 0; rr < RB; ++rr)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[co][rr][q] = b;
    }
    // Input channels are processed in pairs with two row buffers: the rows
    // of channel ci+1 are loaded before the FMAs of channel ci and the rows
    // of ci+2 before those of ci+1, so every channel's loads are in flight
    // during the previous channel's arithmetic.
    float4 ra[RB + 2], rb[RB + 2];
    // Rows are read through a buffer resource spanning one input-channel
    // plane: rows above or below the image and idle lanes get an offset
    // outside the plane, for which the hardware returns zero.  The loads are
    // unconditional, so the code has no branches around them and the
    // compiler waits for exactly the loads it needs (a partial vmcnt).
    const int plane_bytes = (int)(HW * sizeof(float));
    auto load_rows = [&](float4 (&dst)[RB + 2], int ci) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(xg - c0 + (size_t)ci * HW), (short)0, plane_bytes, kBufferWord3);
#pragma unroll
        for (int i = 0; i < RB + 2; ++i) {
            const int ih = r0 - 1 + i;
            const int off = active ? (ih * p.W + c0) * (int)sizeof(float) : kOutOfPlane;
            dst[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
        }
    };
    auto accumulate = [&](const float4 (&rows)[RB + 2], int ci) __attribute__((always_inline)) {
        const float *wc = w + ((size_t)k0 * CI + ci) * 9;
#pragma unroll
        for (int i = 0; i < RB + 2; ++i) {
            float win[6];
            const float l = __shfl_up(rows[i].w, 1, 64);
            const float r = __shfl_down(rows[i].x, 1, 64);
            win[0] = has_left ? l : 0.0f;
            win[1] = rows[i].x; win[2] = rows[i].y; win[3] = rows[i].z; win[4] = rows[i].w;
            win[5] = has_right ? r : 0.0f;
#pragma unroll
            for (int kr = 0; kr < 3; ++kr) {
                const int rr = i - kr;  // output row fed by input row i through kernel row kr
                if (rr < 0 || rr >= RB) continue;
#pragma unroll
                for (int co = 0; co < CO; ++co) {
                    const float *wk = wc + (size_t)co * CI * 9 + kr * 3;
#pragma unroll
                    for (int s = 0; s < 3; ++s) {
                        const float wv_s = wk[s];
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[co][rr][q] = fmaf(win[q + s], wv_s, acc[co][rr][q]);
                    }
                }
            }
        }
    };
    load_rows(ra, 0);
#pragma unroll 1
    for (int ci = 0; ci < CI; ci += 2) {
        if (ci + 1 < CI) load_rows(rb, ci + 1);
        accumulate(ra, ci);
        if (ci + 1 < CI) {
            if (ci + 2 < CI) load_rows(ra, ci + 2);
            accumulate(rb, ci + 1);
        }
    }
    if (!active) return;
    float *yb = y + ((size_t)n * p.K + k0) * HW + c0;
#pragma unroll
    for (int co = 0; co < CO; ++co)
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
            const int oh = r0 + rr;
            if (oh < p.H)
                *reinterpret_cast<float4 *>(yb + (size_t)co * HW + (size_t)oh * p.W) =
                    make_float4(acc[co][rr][0], acc[co][rr][1], acc[co][rr][2], acc[co][rr][3]);
        }
}

template <int CI, int CO, int RB>
hipError_t launch_rows_t(const G3Rows &p, const float *x, const float *w, const float *bias, float *y,
                         hipStream_t st) {
    const int grid = (p.waves + kBlock / 64 - 1) / (kBlock / 64);
    clear_stale_launch_error();
    hipLaunchKernelGGL((grouped3x3_rows_kernel<CI, CO, RB>), dim3(grid), dim3(kBlock), 0, st, x, w, bias, y, p);
    return hipGetLastError();
}

template <int RB>
hipError_t launch_rows(int CI, int CO, const G3Rows &p, const float *x, const float *w, const float *bias,
                       float *y, hipStream_t st) {
    if constexpr (RB <= 2) {
        // 8 or 16 channels per group: blocks of 8 (or 4) output channels
        if (CI == 16) {
            if (CO == 4) return launch_rows_t<16, 4, RB>(p, x, w, bias, y, st);
            if (CO == 2) return launch_rows_t<16, 2, RB>(p, x, w, bias, y, st);
            return launch_rows_t<16, 1, RB>(p, x, w, bias, y, st);
        }
        if (CI == 8) {
            if (CO == 4) return launch_rows_t<8, 4, RB>(p, x, w, bias, y, st);
            if (CO == 2) return launch_rows_t<8, 2, RB>(p, x, w, bias, y, st);
            return launch_rows_t<8, 1, RB>(p, x, w, bias, y, st);
        }
    }
    if (CI == 4) {
        if (CO == 4) return launch_rows_t<4, 4, RB>(p, x, w, bias, y, st);
        if (CO == 2) return launch_rows_t<4, 2, RB>(p, x, w, bias, y, st);
        return launch_rows_t<4, 1, RB>(p, x, w, bias, y, st);
    }
    if (CI == 2) {
        if (CO == 4) return launch_rows_t<2, 4, RB>(p, x, w, bias, y, st);
        if (CO == 2) return launch_rows_t<2, 2, RB>(p, x, w, bias, y, st);
        return launch_rows_t<2, 1, RB>(p, x, w, bias, y, st);
    }
    if (CO == 4) return launch_rows_t<1, 4, RB>(p, x, w, bias, y, st);
    if (CO == 2) return launch_rows_t<1, 2, RB>(p, x, w, bias, y, st);
    return launch_rows_t<1, 1, RB>(p, x, w, bias, y, st);
}

// Output channels per lane: up to 4 (the most that divides the group's).
int rows_co(const gconv_desc *d) { return d->cout % 4 == 0 ? 4 : (d->cout % 2 == 0 ? 2 : 1); }

// The LDS band kernel's geometry for CO output channels per workgroup: Q
// outputs per lane along W, the band (BH rows x TW columns), the number of
// bands (*gx) and the dynamic LDS bytes (staged rows with halo + weights).
size_t band_plan(const gconv_desc *d, int CO, G3Params *p, int *Q, long long *gx) {
    *Q = d->W >= 32 ? 8 : 4;
    p->C = d->C; p->H = d->H; p->W = d->W; p->K = d->K;
    p->cout = d->cout;
    p->n_cob = d->cout / CO;
    // band width: the whole row when it fits 32 lanes, else 32*Q columns
    const int wq = (d->W + *Q - 1) / *Q;
    const int tasks_per_row = wq < 32 ? wq : 32;
    p->TW = tasks_per_row * *Q;
    p->n_cb = (d->W + p->TW - 1) / p->TW;
    // band height: fill 256 lanes, then even out the bands over H
    int bh = kBlock / tasks_per_row;
    if (bh > d->H) bh = d->H;
    const int n_rb = (d->H + bh - 1) / bh;
    p->BH = (d->H + n_rb - 1) / n_rb;
    p->pitch = (p->TW + kLead + 1 + 3) & ~3;
    p->vec_load = p->vec_store = 0;
    *gx = (long long)n_rb * p->n_cb;
    return sizeof(float) * ((size_t)d->cin * (p->BH + 2) * p->pitch + (size_t)CO * d->cin * 9);
}

// Wide groups: 8 or 16 input channels per group and up to 16 output
// channels (a multiple of 4).  They run on the register kernel when W allows
// it, else on the LDS band kernel when its band fits kWideBandLds; the
// register kernel's alignment limit is checked at launch.
bool wide_geometry(const gconv_desc *d) {
    if (!((d->cin == 8 || d->cin == 16) && d->groups > 1 && d->cout % 4 == 0 && d->cout <= 16)) return false;
    if (d->W % 4 == 0 && d->W <= 256 && (long long)(d->H + 2) * d->W * (long long)sizeof(float) < 0x7fffffffLL)
        return true;
    G3Params p;
    int Q;
    long long gx;
    return band_plan(d, 4, &p, &Q, &gx) <= kWideBandLds;
}

// The register variant's geometry for RB rows per lane, or false.
bool rows_plan(const gconv_desc *d, const float *x, const float *y, int RB, int CO, G3Rows *p) {
    if (d->W % 4 != 0 || d->W > 256) return false;
    // byte offsets within one plane, including one row before and after it,
    // must fit a signed 32-bit buffer offset
    if ((long long)(d->H + 2) * d->W * (long long)sizeof(float) >= 0x7fffffffLL) return false;
    if (((uintptr_t)x | (uintptr_t)y) & 15u) return false;
    p->C = d->C; p->H = d->H; p->W = d->W; p->K = d->K; p->G = d->groups;
    p->cout = d->cout;
    p->n_cob = d->cout / CO;
    p->cg = d->W / 4;
    p->rpw = 64 / p->cg;
    p->strips = (d->H + RB - 1) / RB;
    p->wpp = (p->strips + p->rpw - 1) / p->rpw;
    const long long waves = (long long)d->N * d->groups * p->n_cob * p->wpp;
    if (waves > 0x7fffffffLL - 64) return false;
    p->waves = (int)waves;
    return true;
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
        case 16: return launch_co<16, Q>(CO, p, grid, lds, x, w, bias, y, st);
        case 8: return launch_co<8, Q>(CO, p, grid, lds, x, w, bias, y, st);
        case 4: return launch_co<4, Q>(CO, p, grid, lds, x, w, bias, y, st);
        case 2: return launch_co<2, Q>(CO, p, grid, lds, x, w, bias, y, st);
        default: return launch_co<1, Q>(CO, p, grid, lds, x, w, bias, y, st);
    }
}

}  // namespace

bool grouped3x3_supported(const gconv_desc *d) {
    return d->R == 3 && d->S == 3 && d->stride == 1 && d->pad == 1 && d->dil == 1 &&
           (d->cin == 1 || d->cin == 2 || d->cin == 4 || wide_geometry(d) || grouped16_mfma_applies(d));
}

hipError_t launch_grouped3x3(const gconv_desc *d, const float *x, const float *w, const float *bias,
                             float *y, hipStream_t st) {
    if (!grouped3x3_supported(d)) return hipErrorInvalidValue;
    // 16 input and 16 output channels per group with enough waves: the FP32
    // matrix cores (k_grouped_mfma.hip)
    if (grouped16_mfma_applies(d)) return launch_grouped16_mfma(d, x, w, bias, y, st);
    {
        // rows per lane: 2 in general; 4 for large depthwise problems (less
        // halo traffic through the L2, and registers to spare); 1 when the
        // problem is so small that the critical path of one wave dominates
        G3Rows rp;
        int CO = rows_co(d);
        {
            // a lane runs 9 * cin FMAs per output it owns, so on small
            // problems one wave's chain of channels sets the time; fewer
            // output channels per lane then buy more waves
            while (CO > 1) {
                if (!rows_plan(d, x, y, 2, CO, &rp)) break;
                if (rp.waves < kSmallWaves) rows_plan(d, x, y, 1, CO, &rp);
                if (rp.waves >= kWideWaves) break;
                CO /= 2;
            }
        }
        if (rows_plan(d, x, y, 2, CO, &rp)) {
            if (rp.waves < kSmallWaves && rows_plan(d, x, y, 1, CO, &rp))
                return launch_rows<1>(d->cin, CO, rp, x, w, bias, y, st);
            if (d->cin == 1 && rows_plan(d, x, y, 4, CO, &rp) && rp.waves >= kLargeWaves)
                return launch_rows<4>(d->cin, CO, rp, x, w, bias, y, st);
            rows_plan(d, x, y, 2, CO, &rp);
            return launch_rows<2>(d->cin, CO, rp, x, w, bias, y, st);
        }
    }
    int CO = rows_co(d);
    G3Params p;
    int Q;
    long long gx = 0;
    size_t lds = band_plan(d, CO, &p, &Q, &gx);
    if (d->cin > 4 && lds > kWideBandLds) {
        // wide groups on a band that does not fit (wide rows that are not
        // 16-byte aligned): the implicit GEMM or the direct kernel
        if (igemm_supported(d)) return launch_igemm(d, x, w, bias, y, st);
        return launch_direct(d, x, w, bias, y, st);
    }
    // fewer output channels per workgroup buy more workgroups on small grids
    while (CO > 1 && gx * d->groups * (d->cout / CO) * d->N < kWideBlocks) {
        CO /= 2;
        lds = band_plan(d, CO, &p, &Q, &gx);
    }
    p.vec_load = (d->W % 4 == 0) && (((uintptr_t)x & 15u) == 0);
    p.vec_store = (d->W % 4 == 0) && (((uintptr_t)y & 15u) == 0);
    const long long gy = (long long)d->groups * p.n_cob;
    // the band kernel's grid is (tiles, group x channel block, n): beyond
    // the hardware's 65535 limit on y and z the direct kernel takes over
    if (gx > 0x7fffffffLL || gy > 65535 || d->N > 65535) return launch_direct(d, x, w, bias, y, st);
    dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)d->N);
    if (Q == 8) return launch_ci<8>(d->cin, CO, p, grid, lds, x, w, bias, y, st);
    return launch_ci<4>(d->cin, CO, p, grid, lds, x, w, bias, y, st);
}

}  // namespace gconv
