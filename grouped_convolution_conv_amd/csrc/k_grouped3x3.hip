// k_grouped3x3.hip -- grouped / depthwise 3x3, stride 1, pad 1, dilation 1,
// with 1, 2 or 4 input channels per group (the workload of the GroupConv
// Atlas page).
//
// Design for gfx950 (VALU, HBM-bound):
//  - One workgroup (256 lanes = 4 wave64) owns one (n, group, block of up
//    to 4 output channels, band of BH rows x TW columns).  It stages the
//    band's input rows for the group's channels, with a one-pixel zero halo,
//    in LDS, so every input byte comes from HBM once per output-channel
//    block (the cooperative shared halo of the Atlas page's third kernel).
//  - The staging issues its global loads in batches of kBatch independent
//    128-bit loads per lane before writing any of them to LDS, so a lane
//    keeps several loads in flight instead of waiting on each one.
//  - LDS row layout: [3 pad][left halo][TW interior columns][right halo][pad]
//    so interior columns land 16-byte aligned (128-bit LDS writes) and a
//    lane's window of Q+2 inputs is read as b32 + Q/4 x b128 + b32.
//  - Each lane computes Q adjacent outputs along W for every output channel
//    of the block (the Atlas page's fourth kernel gives each thread four
//    neighbouring outputs; here Q is 4 or 8 and the lane also covers up to four
//    output channels): per input channel and kernel row, Q+2 LDS reads feed
//    CO*3*Q FMAs.  The block's weights sit in LDS and are read as broadcasts.
//  - Results leave as 128-bit stores; the W tail is masked.
#include "dev_common.h"
#include "internal.h"

namespace gconv {
namespace {

constexpr int kBlock = 256;
constexpr int kBatch = 8;   // global loads in flight per lane during staging
constexpr int kLead = 4;    // LDS index of interior column 0

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
// Streaming variant for full-row bands (W % 4 == 0, W <= 256, 16-byte aligned
// tensors): a persistent grid walks the units (n, group, channel block, band)
// and double-buffers them in LDS.  A band of one input channel is a single
// contiguous run of global memory, copied straight into LDS with
// global_load_lds_dwordx4 (lane l of a wave writes 16 bytes at M0 + 16*l),
// so the next unit's loads are in flight, without using registers, while the
// current unit is computed.  Rows above and below the image are zero-filled
// with LDS stores; the left/right zero padding is applied when a lane reads
// its window.  The weights of a unit are uniform over the workgroup and come
// through the scalar cache.

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

struct G3Stream {
    int C, H, W, K, G;
    int cout, n_cob;
    int BH, n_rb;      // band height and bands per plane
    int units;         // N * G * n_cob * n_rb
    int buf_floats;    // floats of one staged band (CI * (BH + 2) * W)
};

__device__ __forceinline__ void wait_async_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int CI, int CO>
__device__ __forceinline__ void stream_stage(const float *__restrict__ x, const float *__restrict__ w,
                                             const G3Stream &p, int u, float *buf) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rb = u % p.n_rb;
    int t = u / p.n_rb;
    const int cob = t % p.n_cob;
    t /= p.n_cob;
    const int g = t % p.G, n = t / p.G;
    const int oh0 = rb * p.BH;
    const int rows = p.BH + 2;
    const int ih_lo = max(oh0 - 1, 0), ih_hi = min(oh0 + p.BH + 1, p.H);
    const int lr_lo = ih_lo - (oh0 - 1);                  // first staged row that exists
    const int n16 = (ih_hi - ih_lo) * p.W / 4;            // 16-byte pieces per channel
    const size_t HW = (size_t)p.H * p.W;
    const float *xg = x + ((size_t)n * p.C + (size_t)g * CI) * HW + (size_t)ih_lo * p.W;
    // rows outside the image read zero: staged rows [0, lr_lo) and
    // [lr_hi, rows) of every channel
    const int lr_hi = lr_lo + (ih_hi - ih_lo);
    const int nz = lr_lo + (rows - lr_hi);                 // zero rows per channel
    if (nz > 0) {
        const int w4 = p.W >> 2;
        for (int e = tid; e < CI * nz * w4; e += kBlock) {
            const int zr = e / w4, c4 = (e - zr * w4) << 2;
            const int ci = zr / nz, k = zr - ci * nz;
            const int lr = k < lr_lo ? k : lr_hi + (k - lr_lo);
            *reinterpret_cast<float4 *>(buf + (ci * rows + lr) * p.W + c4) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    // the rows that exist, one contiguous run of global memory per channel,
    // straight into LDS (after the zero rows: an LDS store issued after the
    // DMA would make the compiler wait for the DMA)
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
        float *dst = buf + (ci * rows + lr_lo) * p.W;
        const float *src = xg + ci * HW;
        for (int q = wave; q * 64 < n16; q += 4) {
            const int e = q * 64 + lane;
            if (e < n16)
                __builtin_amdgcn_global_load_lds((glb_void_t *)(src + 4 * e), (lds_void_t *)(dst + q * 256), 16, 0, 0);
        }
    }
}

// One unit's compute from band buffer `buf`: every lane's CI*3 windows feed
// CO*CI*9*Q FMAs; the results stay in `outv` and are stored by the caller
// after the next barrier (see the kernel below).
template <int CI, int CO, int Q>
__device__ __forceinline__ void stream_compute(const float *buf, const float *__restrict__ w,
                                               const float *__restrict__ bias, const G3Stream &p,
                                               int k0, int lr, int jq, float (&outv)[CO][Q]) {
    const int rows = p.BH + 2;
#pragma unroll
    for (int co = 0; co < CO; ++co) {
        const float b = bias ? bias[k0 + co] : 0.0f;
#pragma unroll
        for (int q = 0; q < Q; ++q) outv[co][q] = b;
    }
#pragma unroll 1
    for (int ci = 0; ci < CI; ++ci) {
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const int base = (ci * rows + lr + r) * p.W + jq;
            float win[Q + 2];
            const float left = buf[jq > 0 ? base - 1 : base];
            const float right = buf[jq + Q < p.W ? base + Q : base];
            win[0] = jq > 0 ? left : 0.0f;
            win[Q + 1] = jq + Q < p.W ? right : 0.0f;
#pragma unroll
            for (int q = 0; q < Q; q += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(buf + base + q);
                win[q + 1] = v.x; win[q + 2] = v.y; win[q + 3] = v.z; win[q + 4] = v.w;
            }
#pragma unroll
            for (int co = 0; co < CO; ++co) {
                // readfirstlane keeps the weight offset uniform (scalar loads,
                // which never wait on the band DMA) and opaque, so the loads
                // of different channels are not merged into one long batch
                const int off = __builtin_amdgcn_readfirstlane(((k0 + co) * CI + ci) * 9 + r * 3);
                const float *wg = w + off;
#pragma unroll
                for (int s = 0; s < 3; ++s) {
                    const float wv = wg[s];
#pragma unroll
                    for (int q = 0; q < Q; ++q) outv[co][q] = fmaf(win[q + s], wv, outv[co][q]);
                }
            }
        }
    }
}

// Static LDS double buffer: two distinct LDS objects, so the compiler can
// tell that reads of one buffer never alias the DMA into the other and does
// not wait for the DMA before them.  CAP floats per buffer (a size class
// chosen on the host).
template <int CI, int CO, int Q, int CAP>
__global__ __launch_bounds__(kBlock) void grouped3x3_stream_kernel(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ y, G3Stream p) {
    __shared__ float4 bufA4[CAP / 4];
    __shared__ float4 bufB4[CAP / 4];
    float *bufA = reinterpret_cast<float *>(bufA4);
    float *bufB = reinterpret_cast<float *>(bufB4);
    const int tid = threadIdx.x;
    const int tasks_per_row = p.W / Q;
    const int lr = tid / tasks_per_row;                 // this lane's output row in the band
    const int jq = (tid - lr * tasks_per_row) * Q;      // and its first column
    const size_t HW = (size_t)p.H * p.W;

    // Per unit: wait for its band, store the previous unit's outputs, start
    // the next unit's DMA, compute.  The vector-memory counter covers stores
    // as well as loads and retires them in order, so stores issued before
    // the next DMA are older than it: the wait at the top of the next unit
    // finds them long done instead of stalling on freshly issued ones.
    float outv[CO][Q];
    float *out_dst = nullptr;  // row start of channel k0 for outv; null: nothing pending
    auto flush = [&]() __attribute__((always_inline)) {
        if (out_dst) {
#pragma unroll
            for (int co = 0; co < CO; ++co)
#pragma unroll
                for (int q = 0; q < Q; q += 4)
                    *reinterpret_cast<float4 *>(out_dst + co * HW + q) =
                        make_float4(outv[co][q], outv[co][q + 1], outv[co][q + 2], outv[co][q + 3]);
            out_dst = nullptr;
        }
    };
    auto unit = [&](int u, const float *cur, float *nxt) __attribute__((always_inline)) {
        wait_async_loads();
        __syncthreads();  // unit u staged in cur; every lane is done with nxt
        flush();
        const int un = u + (int)gridDim.x;
        if (un < p.units) stream_stage<CI, CO>(x, w, p, un, nxt);
        const int rb = u % p.n_rb;
        int t = u / p.n_rb;
        const int cob = t % p.n_cob;
        t /= p.n_cob;
        const int g = t % p.G, n = t / p.G;
        const int oh = rb * p.BH + lr;
        if (lr < p.BH && oh < p.H) {
            const int k0 = g * p.cout + cob * CO;
            stream_compute<CI, CO, Q>(cur, w, bias, p, k0, lr, jq, outv);
            out_dst = y + ((size_t)n * p.K + k0) * HW + (size_t)oh * p.W + jq;
        }
    };
    int u = blockIdx.x;
    if (u < p.units) stream_stage<CI, CO>(x, w, p, u, bufA);
    while (u < p.units) {
        unit(u, bufA, bufB);
        u += gridDim.x;
        if (u >= p.units) break;
        unit(u, bufB, bufA);
        u += gridDim.x;
    }
    flush();
}

template <int CI, int CO, int Q, int CAP>
hipError_t launch_stream_t(const G3Stream &p, const float *x, const float *w, const float *bias,
                           float *y, hipStream_t st) {
    auto kern = grouped3x3_stream_kernel<CI, CO, Q, CAP>;
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return hipErrorInvalidDevice;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBlock, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    const long long want = (long long)cus * per_cu;
    const int grid = (int)(p.units < want ? p.units : want);
    clear_stale_launch_error();
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlock), 0, st, x, w, bias, y, p);
    return hipGetLastError();
}

// buffer size classes (floats per band buffer)
constexpr int kCapS = 2304, kCapM = 4608, kCapL = 9216;

template <int CI, int CO, int Q>
hipError_t launch_stream_cap(int cap, const G3Stream &p, const float *x, const float *w,
                             const float *bias, float *y, hipStream_t st) {
    if (cap == kCapS) return launch_stream_t<CI, CO, Q, kCapS>(p, x, w, bias, y, st);
    if (cap == kCapM) return launch_stream_t<CI, CO, Q, kCapM>(p, x, w, bias, y, st);
    return launch_stream_t<CI, CO, Q, kCapL>(p, x, w, bias, y, st);
}

template <int CI, int Q>
hipError_t launch_stream_co(int CO, int cap, const G3Stream &p, const float *x, const float *w,
                            const float *bias, float *y, hipStream_t st) {
    switch (CO) {
        case 4: return launch_stream_cap<CI, 4, Q>(cap, p, x, w, bias, y, st);
        case 2: return launch_stream_cap<CI, 2, Q>(cap, p, x, w, bias, y, st);
        default: return launch_stream_cap<CI, 1, Q>(cap, p, x, w, bias, y, st);
    }
}

template <int Q>
hipError_t launch_stream_ci(int CI, int CO, int cap, const G3Stream &p, const float *x,
                            const float *w, const float *bias, float *y, hipStream_t st) {
    switch (CI) {
        case 4:
            if constexpr (Q == 8) return hipErrorInvalidValue;  // never planned: Q = 4 for 4-channel groups
            else return launch_stream_co<4, Q>(CO, cap, p, x, w, bias, y, st);
        case 2: return launch_stream_co<2, Q>(CO, cap, p, x, w, bias, y, st);
        default: return launch_stream_co<1, Q>(CO, cap, p, x, w, bias, y, st);
    }
}

// The streaming variant's geometry, or false when it does not apply.
bool stream_plan(const gconv_desc *d, const float *x, const float *y, int *Qout, G3Stream *p, int *cap) {
    if (d->W % 4 != 0 || d->W > 256) return false;
    if (((uintptr_t)x | (uintptr_t)y) & 15u) return false;
    // Q = 8 halves the LDS reads per output, but a lane then holds 3*CI
    // windows of 10 inputs; 4-channel groups take Q = 4 (fewer registers,
    // half-height bands, four workgroups per CU).
    const int Q = (d->W % 8 == 0 && d->cin < 4) ? 8 : 4;
    const int tpr = d->W / Q;
    if (tpr > 64) return false;
    const int CO = d->cout % 4 == 0 ? 4 : (d->cout % 2 == 0 ? 2 : 1);
    int bh = kBlock / tpr;
    if (bh > d->H) bh = d->H;
    const int n_rb = (d->H + bh - 1) / bh;
    p->C = d->C; p->H = d->H; p->W = d->W; p->K = d->K; p->G = d->groups;
    p->cout = d->cout;
    p->n_cob = d->cout / CO;
    p->BH = (d->H + n_rb - 1) / n_rb;
    p->n_rb = n_rb;
    const long long units = (long long)d->N * d->groups * p->n_cob * n_rb;
    if (units > 0x7fffffffLL) return false;
    p->units = (int)units;
    p->buf_floats = d->cin * (p->BH + 2) * d->W;
    if (p->buf_floats <= kCapS) *cap = kCapS;
    else if (p->buf_floats <= kCapM) *cap = kCapM;
    else if (p->buf_floats <= kCapL) *cap = kCapL;
    else return false;
    *Qout = Q;
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
    {
        G3Stream sp;
        int cap = 0, sq = 0;
        if (stream_plan(d, x, y, &sq, &sp, &cap)) {
            const int CO = d->cout % 4 == 0 ? 4 : (d->cout % 2 == 0 ? 2 : 1);
            if (sq == 8) return launch_stream_ci<8>(d->cin, CO, cap, sp, x, w, bias, y, st);
            return launch_stream_ci<4>(d->cin, CO, cap, sp, x, w, bias, y, st);
        }
    }
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
    p.pitch = (p.TW + kLead + 1 + 3) & ~3;
    p.vec_load = (d->W % 4 == 0) && (((uintptr_t)x & 15u) == 0);
    p.vec_store = (d->W % 4 == 0) && (((uintptr_t)y & 15u) == 0);
    const long long gx = (long long)n_rb * p.n_cb;
    const long long gy = (long long)d->groups * p.n_cob;
    if (gx > 0x7fffffffLL || gy > 65535 || d->N > 65535) return hipErrorInvalidConfiguration;
    const size_t lds = sizeof(float) * ((size_t)d->cin * (p.BH + 2) * p.pitch + (size_t)CO * d->cin * 9);
    dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)d->N);
    if (Q == 8) return launch_ci<8>(d->cin, CO, p, grid, lds, x, w, bias, y, st);
    return launch_ci<4>(d->cin, CO, p, grid, lds, x, w, bias, y, st);
}

}  // namespace gconv
