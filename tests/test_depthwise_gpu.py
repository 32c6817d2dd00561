"""GPU parity of the depthwise kernel (5x5 and 7x7 at stride 1, 3x3 and 5x5
at stride 2, 3x3 at dilation 2; padding dil * (R // 2)) through the C ABI
against the CPU oracle.

Same bars as the other parity tests: |y_gpu - y_oracle| <= 1e-4 * A + 1e-6
with A = sum |x * w| over the receptive field; bit-for-bit equality for
integer-valued inputs.  Outputs are pre-filled with NaN.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
import grouped_convolution_conv_amd as gc

pytestmark = pytest.mark.gpu

CONV_RTOL, CONV_ATOL = 1e-4, 1e-6


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _dw(name, N, C, H, W, R, stride, seed, dil=1):
    return synth.Workload(name, N, C, H, W, C, R, R, stride, dil * (R // 2), dil, C, seed,
                          ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0))


def _grp(name, N, C, H, W, K, R, stride, G, seed, dil=1):
    return synth.Workload(name, N, C, H, W, K, R, R, stride, dil * (R // 2), dil, G, seed,
                          ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0))


# Small cases: the oracle computes every output.  They cover one 4-column
# group per row (a wave holds 64 row strips), a full 256-column output row
# per wave (one strip per wave), row counts that leave part of the last
# strip and part of the last wave idle, a single input row, and output rows
# whose lanes do not fill a wave.
SMALL = [
    _dw("dw5_h13_w20", 2, 6, 13, 20, 5, 1, 201),
    _dw("dw5_h1_w8", 3, 4, 1, 8, 5, 1, 202),
    _dw("dw5_h14_w28_planes", 8, 64, 14, 28, 5, 1, 203),
    _dw("dw7_h9_w256", 1, 3, 9, 256, 7, 1, 204),
    _dw("dw7_h3_w4", 2, 4, 3, 4, 7, 1, 205),
    _dw("dw7_h31_w60", 2, 5, 31, 60, 7, 1, 206),
    _dw("dw3s2_h7_w8", 2, 5, 7, 8, 3, 2, 207),
    _dw("dw3s2_h33_w512", 1, 2, 33, 512, 3, 2, 208),
    _dw("dw3s2_h2_w16", 4, 3, 2, 16, 3, 2, 209),
    _dw("dw3s2_h30_w56_planes", 4, 48, 30, 56, 3, 2, 210),
    _dw("dw5s2_h9_w8", 2, 5, 9, 8, 5, 2, 216),
    _dw("dw5s2_h27_w512", 1, 3, 27, 512, 5, 2, 217),
    _dw("dw5s2_h2_w24_planes", 8, 40, 2, 24, 5, 2, 218),
    _dw("dw3d2_h11_w12", 2, 5, 11, 12, 3, 1, 219, dil=2),
    _dw("dw3d2_h3_w256", 1, 3, 3, 256, 3, 1, 220, dil=2),
    _dw("dw3d2_h17_w4_planes", 8, 36, 17, 4, 3, 1, 221, dil=2),
    # groups of 2 or 4 input channels: 4, 2 or 1 output channels per lane,
    # several blocks per group, ragged rows, a whole 256-column row per wave
    _grp("grp3s2_cpg4", 2, 16, 14, 16, 16, 3, 2, 4, 222),
    _grp("grp3s2_cpg2_cout3", 2, 8, 9, 24, 12, 3, 2, 4, 223),
    _grp("grp5_cpg4_cout8", 1, 8, 11, 20, 16, 5, 1, 2, 224),
    _grp("grp7_cpg2", 2, 4, 9, 12, 4, 7, 1, 2, 225),
    _grp("grp3d2_cpg4", 2, 8, 13, 16, 8, 3, 1, 2, 226, dil=2),
    _grp("grp5s2_cpg2_cout4", 1, 4, 10, 40, 8, 5, 2, 2, 227),
    _grp("grp3s2_cpg4_w512", 1, 8, 9, 512, 8, 3, 2, 2, 228),
    # groups of 8 or 16 input channels
    _grp("grp3s2_cpg8", 2, 32, 15, 24, 32, 3, 2, 4, 229),
    _grp("grp3s2_cpg16_cout8", 1, 32, 10, 32, 16, 3, 2, 2, 230),
    _grp("grp5_cpg8_cout4", 2, 16, 7, 12, 8, 5, 1, 2, 231),
    _grp("grp3d2_cpg16", 1, 32, 11, 20, 32, 3, 1, 2, 232, dil=2),
    _grp("grp7_cpg8_cout6", 1, 16, 9, 8, 12, 7, 1, 2, 233),
    # one input channel per group with a channel multiplier of 2, 3, 4, 6
    # and 8 (4, 2 or 1 output channels per lane), also with groups = 1
    _grp("dwm5_cout2", 2, 6, 13, 20, 12, 5, 1, 6, 234),
    _grp("dwm3s2_cout4", 2, 4, 14, 16, 16, 3, 2, 4, 235),
    _grp("dwm7_cout3", 1, 3, 9, 12, 9, 7, 1, 3, 236),
    _grp("dwm3d2_cout6", 2, 4, 11, 16, 24, 3, 1, 4, 237, dil=2),
    _grp("dwm5s2_c1_k8", 2, 1, 10, 40, 8, 5, 2, 1, 238),
    _grp("dwm3s2_cout2_w512", 1, 3, 9, 512, 6, 3, 2, 3, 239),
    # ragged rows: output widths that are not a multiple of 4 (one lane
    # partly past the row end), odd input widths at stride 2, one partial
    # lane, the widest row (64 lanes, the last one partial), 256 outputs
    # from an odd 511-column input
    _dw("rag_dw5_h14_w14", 2, 6, 14, 14, 5, 1, 240),
    _dw("rag_dw7_h7_w7", 2, 5, 7, 7, 7, 1, 241),
    _dw("rag_dw3s2_h14_w14", 2, 6, 14, 14, 3, 2, 242),
    _dw("rag_dw3s2_h13_w13", 2, 5, 13, 13, 3, 2, 243),
    _dw("rag_dw5s2_h11_w21", 1, 4, 11, 21, 5, 2, 244),
    _dw("rag_dw3d2_h10_w10", 2, 4, 10, 10, 3, 1, 245, dil=2),
    _dw("rag_dw7_h5_w3", 3, 4, 5, 3, 7, 1, 246),
    _dw("rag_dw5_h9_w254", 1, 3, 9, 254, 5, 1, 247),
    _dw("rag_dw3s2_h5_w511", 1, 2, 5, 511, 3, 2, 248),
    _dw("rag_dw5s2_h1_w9", 2, 3, 1, 9, 5, 2, 249),
    _grp("rag_grp5_cpg4_w14", 2, 8, 14, 14, 8, 5, 1, 2, 250),
    _grp("rag_grp3s2_cpg8_w13", 1, 16, 13, 13, 16, 3, 2, 2, 251),
    _grp("rag_grp3d2_cpg16_cout4_w6", 1, 32, 7, 6, 8, 3, 1, 2, 252, dil=2),
    _grp("rag_dwm7_cout2_w7", 2, 4, 7, 7, 8, 7, 1, 4, 253),
    # small planes packed several to a wave (one input channel per group,
    # a plane filling at most 32 lanes): many waves, a multiplier of 3, a
    # whole-row-aligned 8x8 plane
    _dw("pk_dw5_h14_w14_planes", 4, 40, 14, 14, 5, 1, 254),
    _grp("pk_dwm5_cout3_h3_w3", 3, 7, 3, 3, 21, 5, 1, 7, 255),
    _dw("pk_dw3d2_h8_w8", 2, 6, 8, 8, 3, 1, 256, dil=2),
    _dw("pk_dw3s2_h28_w28_planes", 2, 70, 28, 28, 3, 2, 257),
    # 3x3 stride 1 on small depthwise planes (packed, chosen over the grouped
    # 3x3 kernels): 7x7, 14x14 with many waves, a whole-row-aligned 16x16,
    # a channel multiplier, a single 3-column row
    _dw("pk_dw3_h7_w7", 2, 5, 7, 7, 3, 1, 258),
    _dw("pk_dw3_h14_w14_planes", 4, 40, 14, 14, 3, 1, 259),
    _dw("pk_dw3_h16_w16", 2, 6, 16, 16, 3, 1, 260),
    _grp("pk_dwm3_cout2_h9_w9", 2, 4, 9, 9, 8, 3, 1, 4, 261),
    _dw("pk_dw3_h1_w3", 3, 4, 1, 3, 3, 1, 262),
]

# The depthwise layers of MobileNet-, EfficientNet- and ConvNeXt-style
# networks at batch 16 (the shapes the benchmark can time beside the five
# workloads): compared on sampled outputs (random ones plus every border pixel
# of a few planes).
FULL = list(synth.EXTRA_WORKLOADS.values())


def _dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _run(wl, inp, bias=None, algo=gc.ALGO_AUTO, y_offset=0, x_offset=0):
    """Offsets (in floats) place x or y 4 bytes past a 16-byte boundary."""
    d = gc.conv_desc_create(wl.N, wl.C, wl.H, wl.W, wl.K, wl.R, wl.S, wl.stride, wl.pad, wl.dil, wl.groups)
    gc.conv_desc_set_algo(d, algo)
    ho, wo = gc.conv_desc_get_output_dims(d)
    n_out = wl.N * wl.K * ho * wo
    ybuf = torch.full((n_out + y_offset,), float("nan"), device="cuda")
    y = ybuf[y_offset:]
    x = _dev(inp["x"])
    if x_offset:
        xbuf = torch.empty((x.numel() + x_offset,), device="cuda")
        xbuf[x_offset:] = x.reshape(-1)
        x = xbuf[x_offset:].data_ptr()
    gc.conv_fwd(d, x, _dev(inp["w"]), _dev(bias), y.data_ptr() if y_offset else y)
    torch.cuda.synchronize()
    return y.view(wl.N, wl.K, ho, wo).cpu().numpy(), gc.conv_desc_get_algo(d)


def _check(y_gpu, y_ref, A, what):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bound = CONV_RTOL * A + CONV_ATOL
    ok = err <= bound
    if not np.all(ok):
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError("%s: %d of %d outputs outside 1e-4*A+1e-6; first at %s: gpu %r oracle %r"
                             % (what, len(bad), err.size, i, y_gpu[i], y_ref[i]))
    return float(np.max(err / bound))


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_depthwise_small(wl):
    inp = synth.make_inputs(wl)
    bias = synth.normal((wl.K,), 0.5, wl.seed, 7)
    for b in (None, bias):
        _say("[parity] depthwise", wl.name, "bias" if b is not None else "")
        y_ref, A = oracle.conv2d(inp["x"], inp["w"], b, wl.stride, wl.pad, wl.dil, wl.groups)
        # forced: the dispatcher gives a few small 3x3 planes to the grouped
        # kernels
        y, used = _run(wl, inp, b, algo=gc.ALGO_DEPTHWISE)
        assert used == gc.ALGO_DEPTHWISE
        _check(y, y_ref, A, wl.name)
        # 4-byte aligned output or input: the kernel's ragged-row form
        y1, used = _run(wl, inp, b, algo=gc.ALGO_DEPTHWISE, y_offset=1)
        assert used == gc.ALGO_DEPTHWISE
        _check(y1, y_ref, A, wl.name + " misaligned y")
        y1, _ = _run(wl, inp, b, algo=gc.ALGO_DEPTHWISE, x_offset=1)
        _check(y1, y_ref, A, wl.name + " misaligned x")


@pytest.mark.parametrize("wl", SMALL[::3], ids=lambda w: w.name)
def test_depthwise_integer_inputs_bit_exact(wl):
    wl = wl.with_(x_dist=("int", -3, 3), w_dist=("int", -2, 2), seed=wl.seed + 500)
    _say("[parity] depthwise int", wl.name)
    inp = synth.make_inputs(wl)
    y, used = _run(wl, inp, algo=gc.ALGO_DEPTHWISE)
    assert used == gc.ALGO_DEPTHWISE
    y_ref, _ = oracle.conv2d(inp["x"], inp["w"], None, wl.stride, wl.pad, wl.dil, wl.groups)
    assert np.array_equal(y.astype(np.float64), y_ref)


def _sample_indices(shape, n_random, seed):
    N, K, Ho, Wo = shape
    rng = np.random.default_rng(seed)
    idx = [rng.integers(0, N * K * Ho * Wo, n_random)]
    for (n, k) in [(0, 0), (N - 1, K - 1), (N // 2, K // 3)]:
        base = (n * K + k) * Ho * Wo
        cols = np.arange(Wo)
        rows = np.arange(Ho) * Wo
        idx += [base + cols, base + (Ho - 1) * Wo + cols, base + rows, base + rows + Wo - 1]
    return np.unique(np.concatenate(idx))


@pytest.mark.parametrize("wl", FULL, ids=lambda w: w.name)
def test_depthwise_full_size_sampled(wl):
    _say("[parity] depthwise full-size sampled", wl.name)
    inp = synth.make_inputs(wl)
    bias = synth.normal((wl.K,), 0.5, wl.seed, 7)
    y, used = _run(wl, inp, bias)
    assert used == gc.ALGO_DEPTHWISE
    assert not np.isnan(y).any(), "unwritten outputs"
    idx = _sample_indices(y.shape, 6000, wl.seed)
    y_ref, A = oracle.conv2d_points(inp["x"], inp["w"], idx, bias, wl.stride, wl.pad, wl.dil, wl.groups)
    _check(y.ravel()[idx], y_ref, A, wl.name + " sampled")
