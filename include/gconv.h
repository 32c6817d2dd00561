/*
 * gconv.h -- C ABI of the MI355X (gfx950) FP32 NCHW convolution library.
 *
 * What it computes
 * ----------------
 * conv_fwd: the forward pass of 2-D convolution (cross-correlation, no
 * kernel flip) on contiguous NCHW FP32 tensors:
 *
 *   y[n,k,oh,ow] = bias[k] + sum_{c < C/G} sum_{r < R} sum_{s < S}
 *                  x[n, g*(C/G) + c, oh*stride - pad + r*dil, ow*stride - pad + s*dil]
 *                  * w[k, c, r, s]          with g = k / (K/G),
 *
 * where taps that fall outside the input read zero.  The sum over the input
 * channels and the window is the direct-convolution definition of the
 * POPCORNBENCH trace "Kimi-K2.6 l2_p21" (tiled direct conv design); the
 * weight layout [K][C/G][R][S], the output size
 * Ho = (H + 2*pad - dil*(R-1) - 1)/stride + 1 (likewise Wo) and the
 * input coordinate out*stride - pad + tap*dil are those of the POPCORNBENCH
 * trace "Kimi-K2.6 l1_p62" (dense 5x9 conv, tile and host-wrapper
 * discussion).  Grouped 3x3 stride-1 pad-1 convolution with 1, 2 or 4
 * channels per group up to depthwise is the workload of the GroupConv Atlas
 * page ("Source / Method / Records", first step).  Output channels form G
 * contiguous groups, each reading its own contiguous block of C/G input
 * channels.
 *
 * conv_fused_gn_fwd: the chain of the "Kimi-K2.6 l2_p21" trace, in module
 * order (parameter discussion of that trace):
 *
 *   t   = (conv(x, w)[n,k,oh,ow] + bias[k]) * scale[k]
 *   v   = 1 / (1 + exp(-t))
 *   out = (v - mu[n,gg]) / sqrt(var[n,gg] + eps) * gamma[k] + beta[k]
 *
 * where gg = k / (K/gn_groups) is the GroupNorm group of channel k and
 * mu, var are the mean and the population variance of v over the
 * (K/gn_groups) x Ho x Wo elements of group gg of sample n.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Every tensor argument is a device pointer to contiguous FP32 data
 *    owned by the caller (x [N][C][H][W], w [K][C/G][R][S], y [N][K][Ho][Wo],
 *    per-channel vectors [K]).  Pointers must be 4-byte aligned; faster
 *    kernels are picked when they are 16-byte aligned.  y must not overlap
 *    any input.
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *    The compute calls only enqueue kernels on it: they never allocate,
 *    free, memset or synchronize, so they may be captured into a hipGraph.
 *    A device fault shows up at the caller's next synchronization.
 *  - The descriptor is an opaque host object.  Its geometry is fixed at
 *    creation; the only mutable setting is the algorithm choice.  A
 *    descriptor may be used from several host threads only if none of them
 *    changes the algorithm concurrently.
 *  - Every function returns a status code and never throws across the ABI.
 *  - Arithmetic is FP32 with FP32 accumulation.  Most kernels reorder the
 *    direct sum; plain convs 3 wide at stride 1 on the implicit GEMM's
 *    64-column tiles, and the fused chain's 3x3 passes, use Winograd forms
 *    (F(2, 3) along the columns, F(2x2, 3x3); Lavin and Gray, "Fast
 *    Algorithms for Convolutional Neural Networks"), exact in exact
 *    arithmetic and rounded differently.  Results are repeatable bit for
 *    bit for a given descriptor and algorithm; integer-valued inputs of
 *    small magnitude give exact results on every path of conv_fwd.
 */
#ifndef GCONV_H
#define GCONV_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define GCONV_OK 0
#define GCONV_ERR_INVALID_ARG 1 /* null pointer, non-positive size, bad groups, empty output, ... */
#define GCONV_ERR_WORKSPACE 2   /* workspace missing or smaller than required                  */
#define GCONV_ERR_UNSUPPORTED 3 /* a forced algorithm does not cover this geometry             */
#define GCONV_ERR_LAUNCH 4      /* the HIP runtime refused a kernel launch                     */
#define GCONV_ERR_SCRATCH_LIMIT 5 /* conv_fused_gn_fwd_noalloc: the problem needs more scratch
                                     than the library's static buffer holds                     */

/* Algorithm choices for conv_desc_set_algo.  AUTO lets the dispatcher pick. */
#define GCONV_ALGO_AUTO 0
#define GCONV_ALGO_DIRECT 1     /* one output per lane, any geometry                           */
#define GCONV_ALGO_GROUPED3X3 2 /* 3x3 stride 1 pad 1 dil 1: 1, 2 or 4 input channels per
                                   group; 8 or 16 (groups > 1, <= 16 output channels per group
                                   in multiples of 4) when W % 4 == 0 and W <= 256 or the band
                                   fits 64 KB; 16 in / 16 out per group at any W (run on the
                                   FP32 matrix cores)                                          */
#define GCONV_ALGO_IGEMM 3      /* FP32 MFMA implicit GEMM, >= 4 input and >= 8 output channels
                                   per group, dilation 1, stride 1 (R x S in {1x1, 3x3, 5x5,
                                   5x9, 7x7}) or stride 2 on both axes at 1x1 and 3x3         */
#define GCONV_ALGO_DEPTHWISE 4  /* KxK with padding dil*(K/2), (K, stride, dil) = (5,1,1),
                                   (7,1,1), (3,2,1), (5,2,1), (3,1,2), and (3,1,1) for one input
                                   channel per group on planes of at most 32 lanes (4-column
                                   groups x 2-row strips, x below 2 GB): one input channel per
                                   group (depthwise, any channel multiplier) or groups > 1 of
                                   2, 4, 8 or 16 input channels, any output channels per group;
                                   output width up to 256                                      */

/* How conv_fused_gn_fwd organizes its passes (conv_desc_set_fused_variant). */
#define GCONV_FUSED_AUTO 0
#define GCONV_FUSED_STORE 1     /* conv+epilogue+stats storing v, then normalize v in place    */
#define GCONV_FUSED_RECOMPUTE 2 /* conv+epilogue+stats, merge, then conv again + normalize     */
#define GCONV_FUSED_ONEPASS 3   /* one conv pass: v held in registers until its image's
                                   statistics are merged, then normalized and stored           */

typedef struct gconv_desc *gconv_desc_t;

/* Creates a descriptor for x[N][C][H][W] * w[K][C/groups][R][S] with a
 * symmetric stride, zero padding and dilation.  Requires N,C,H,W,K,R,S >= 1,
 * stride >= 1, dilation >= 1, pad >= 0, groups >= 1 dividing both C and K,
 * Ho >= 1 and Wo >= 1, and every tensor below 2^31 elements.  On success
 * *out owns a host allocation released by conv_desc_destroy; on failure
 * *out is set to NULL. */
int conv_desc_create(gconv_desc_t *out, int N, int C, int H, int W, int K, int R, int S,
                     int stride, int pad, int dilation, int groups);

/* The same with stride, zero padding and dilation given per axis (h along
 * H and R, w along W and S), as in the per-axis conv2d host wrapper of the
 * POPCORNBENCH trace "Kimi-K2.6 l1_p62" (host-wrapper discussion):
 *   Ho = (H + 2*pad_h - dil_h*(R-1) - 1)/stride_h + 1, likewise Wo,
 *   input row oh*stride_h - pad_h + r*dil_h, column ow*stride_w - pad_w + s*dil_w.
 * The fast paths take unit stride and dilation on both axes (the implicit
 * GEMM kernels accept different paddings per axis; the grouped 3x3 kernels
 * need pad 1 on both); any other geometry runs on the direct kernel.
 * conv_desc_create(..., stride, pad, dil, ...) is this call with equal
 * values on both axes. */
int conv_desc_create_2d(gconv_desc_t *out, int N, int C, int H, int W, int K, int R, int S,
                        int stride_h, int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                        int groups);

/* Releases a descriptor.  NULL is accepted and ignored. */
int conv_desc_destroy(gconv_desc_t desc);

/* Output height and width of the descriptor's convolution. */
int conv_desc_get_output_dims(gconv_desc_t desc, int *Ho, int *Wo);

/* Forces an algorithm (GCONV_ALGO_*).  Returns GCONV_ERR_UNSUPPORTED, and
 * leaves the setting unchanged, when the algorithm cannot run this
 * geometry. */
int conv_desc_set_algo(gconv_desc_t desc, int algo);

/* The algorithm conv_fwd and conv_fused_gn_fwd will run (never AUTO). */
int conv_desc_get_algo(gconv_desc_t desc, int *algo);

/* Forces how conv_fused_gn_fwd organizes its passes (GCONV_FUSED_*).
 * GCONV_FUSED_RECOMPUTE needs the MFMA kernel with LDS-resident weights
 * (stride 1, dilation 1, 3x3 or 1x1, 4..8 input and 8..64 output channels,
 * groups 1, 4 channels per GroupNorm group); GCONV_FUSED_ONEPASS needs the
 * same kernel with exactly 32 output channels (8 GroupNorm groups of 4).
 * Otherwise the fused call returns GCONV_ERR_UNSUPPORTED.  All variants
 * compute the same function; they trade HBM traffic (storing and re-reading
 * v) against a second convolution pass, or (one-pass) against holding v in
 * registers while the image's statistics are merged. */
int conv_desc_set_fused_variant(gconv_desc_t desc, int variant);

/* One-pass variant only: the longest time, in microseconds, a wave waits
 * for its image's merged GroupNorm statistics before it stores v as is and
 * leaves that part of the tile to a trailing in-place pass.  0 = do not
 * wait; -1 = leave every tile to the trailing pass; at most 10,000,000.
 * The default is 200.  The output is bit-for-bit the same for every
 * setting; only the time differs.  Because no wave waits past this bound,
 * the call completes whether or not the GPU runs all of its workgroups at
 * once (other work on other streams, say). */
int conv_desc_set_fused_wait(gconv_desc_t desc, int wait_us);

/* The variant conv_fused_gn_fwd will run for gn_groups groups (never AUTO). */
int conv_desc_get_fused_variant(gconv_desc_t desc, int gn_groups, int *variant);

/* y = conv(x, w) (+ bias[k] when bias is not NULL).  See the conventions
 * above. */
int conv_fwd(gconv_desc_t desc, const float *x, const float *w, const float *bias,
             float *y, void *stream);

/* Bytes of device workspace conv_fused_gn_fwd needs for gn_groups groups
 * (gn_groups >= 1 dividing K), for the variant the descriptor resolves to. */
int conv_fused_gn_workspace_size(gconv_desc_t desc, int gn_groups, size_t *bytes);

/* The fused chain above.  bias and scale are required [K] vectors; gamma
 * and beta are [K] vectors or NULL for 1 and 0; eps > 0.  y receives the
 * normalized output.  workspace is caller-owned device memory of at least
 * conv_fused_gn_workspace_size bytes, 16-byte aligned; its contents on
 * entry do not matter and are overwritten.  Kernels run back to back on
 * `stream`: GCONV_FUSED_STORE runs the conv with the elementwise epilogue
 * and per-tile group statistics (storing v in y), then merges the
 * statistics and normalizes y in place; GCONV_FUSED_RECOMPUTE runs the conv
 * with the epilogue for the statistics only, merges them, then runs the
 * conv again and writes the normalized output; GCONV_FUSED_ONEPASS clears
 * its counters, runs the conv once (each image's statistics are merged by
 * the wave that completes them, in a fixed order, and tiles are normalized
 * from registers), then normalizes in place whatever the conv pass left
 * (see conv_desc_set_fused_wait).  On the resident-weight kernel, a 3x3 conv
 * with 32 output channels runs its STORE and RECOMPUTE conv passes in the
 * Winograd form F(2x2, 3x3) (Lavin and Gray, "Fast Algorithms for
 * Convolutional Neural Networks"): the same function, rounded differently
 * from the direct sum (the variants then differ by a few units in the last
 * place of the conv; every variant stays within 1e-4 of the exact chain on
 * the inputs the tests draw). */
int conv_fused_gn_fwd(gconv_desc_t desc, const float *x, const float *w, const float *bias,
                      const float *scale, const float *gamma, const float *beta, int gn_groups,
                      float eps, float *y, void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * chain and arguments as conv_fused_gn_fwd, without the workspace.  The
 * chain's scratch memory (per-tile GroupNorm partials and merged
 * statistics) is a static device array inside the library,
 * conv_fused_gn_noalloc_limit() bytes (16 MiB) on every GPU the library
 * runs on, held until the process ends.  The call allocates and frees
 * nothing.  Its first call on a device looks up that device's copy of the
 * array (hipGetSymbolAddress); make that first call outside stream capture.
 * Returns GCONV_ERR_SCRATCH_LIMIT, before enqueuing anything, when
 * conv_fused_gn_workspace_size exceeds the limit (the fused 8 -> 32 chain
 * on 64 images of 256 x 256 needs 4 MiB).  Every call on one GPU shares that
 * GPU's array, so calls that overlap on one GPU (concurrent streams or host
 * threads) race: serialize them.  Nothing in the array needs to start at
 * zero; every value is written by the call before it is read. */
int conv_fused_gn_fwd_noalloc(gconv_desc_t desc, const float *x, const float *w, const float *bias,
                              const float *scale, const float *gamma, const float *beta, int gn_groups,
                              float eps, float *y, void *stream);

/* Bytes of the static scratch array behind conv_fused_gn_fwd_noalloc. */
size_t conv_fused_gn_noalloc_limit(void);

/* Timing harness for the graph boundary of the GroupConv Atlas page
 * ("Method": device events around launches captured in a CUDA graph).
 * Captures `launches` back-to-back calls into one hipGraph on `stream` and
 * replays it `replays` times between device events; ms_per_launch (host
 * array of `replays` floats) receives each replay's elapsed time divided by
 * `launches`.
 *  - fused = 0: the calls are conv_fwd(desc, xs[i % nsets], w, bias,
 *    ys[i % nsets]); scale, gamma, beta, gn_groups, eps and the workspace
 *    are ignored.
 *  - fused = 1: the calls are conv_fused_gn_fwd with the same rotation.
 * xs and ys are host arrays of nsets device pointers (rotating buffer sets
 * keep the inputs out of the caches between launches).  stream must not be
 * NULL (the null stream cannot be captured).  One eager call runs first
 * and its status is returned if it fails, so a bad argument never leaves a
 * capture open.  Unlike the compute calls this one synchronizes: it
 * returns after the last replay has finished.  The outputs hold the result
 * of the last launch of each buffer set. */
int gconv_time_graph(gconv_desc_t desc, int fused, const float *const *xs, float *const *ys, int nsets,
                     const float *w, const float *bias, const float *scale, const float *gamma,
                     const float *beta, int gn_groups, float eps, void *workspace, size_t workspace_bytes,
                     int launches, int replays, float *ms_per_launch, void *stream);

/* Measured compute peaks of the current device, for roofline fractions
 * against what the chip sustains rather than its datasheet: *mfma_tflops
 * from back-to-back FP32 MFMA (v_mfma_f32_32x32x2f32) chains, *fma_tflops
 * from non-packed FP32 FMA chains, each one timed launch (after a warm-up
 * launch) over four workgroups per CU on `stream` (a hipStream_t; NULL is the
 * default stream).  sink: a caller-owned device buffer of at least 4 bytes that
 * the probes never write in practice (it keeps their arithmetic alive).
 * Synchronizes on the stream.  Returns GCONV_ERR_INVALID_ARG for a null
 * argument, GCONV_ERR_LAUNCH if the runtime refuses a call. */
int gconv_probe_peaks(float *mfma_tflops, float *fma_tflops, float *sink, void *stream);

/* Measured vector-ALU peaks of the current device: *fp32_tflops from
 * chains of non-packed FP32 FMAs (v_fma_f32), *fp64_tflops from the same
 * loop in FP64 (v_fma_f64), sixteen independent chains per lane and eight
 * workgroups of 256 lanes per CU, one timed launch each after a warm-up
 * launch on `stream`.  The FP64 figure is the control for the loop: on
 * MI355X its datasheet peak is one FMA per lane per clock (78.6 TFLOP/s).
 * sink: a caller-owned device buffer of at least 4 bytes the probes never
 * write in practice.  Synchronizes on the stream.  Returns
 * GCONV_ERR_INVALID_ARG for a null argument, GCONV_ERR_LAUNCH if the runtime
 * refuses a call. */
int gconv_probe_vector_peaks(float *fp32_tflops, float *fp64_tflops, float *sink, void *stream);

/* Measured streaming rate of the device memory: copies `bytes` from src to
 * dst (caller-owned device buffers, 16-byte aligned, not overlapping, bytes
 * a positive multiple of 16) with the library's own copy kernel (16-byte
 * non-temporal loads and stores, four pieces in flight per lane), one
 * warm-up launch and five timed launches on `stream`; *gbs receives the
 * fastest launch's rate, counting the bytes read and the bytes written
 * (2 * bytes per launch).  Use buffers well beyond the last-level cache
 * (256 MB) to measure HBM.  Synchronizes on the stream.  dst receives a copy
 * of src. */
int gconv_probe_copy(float *gbs, float *dst, const float *src, size_t bytes, void *stream);

/* Static text for a status code. */
const char *gconv_status_string(int status);

/* Text of the HIP runtime error behind the calling thread's most recent
 * GCONV_ERR_LAUNCH, or "none". */
const char *gconv_last_launch_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GCONV_H */
