"""GPU parity over the 80-shape grouped 3x3 grid (the GroupConv Atlas's fixed
experiment: FP32, contiguous NCHW, 3x3, stride and dilation 1, padding 1, no
bias), through the C ABI, against the CPU oracle.

The Atlas checks complete outputs before it times anything ("Method":
verify before timing); this is that check for the grid the benchmark's sweep
times.  Every shape runs under AUTO (the dispatcher's choice) and under the
forced DIRECT kernel (the one-output-per-lane baseline the sweep compares
against), and every output element is compared.

Bar: |y_gpu - y_oracle| <= 1e-4 * A + 1e-6 per output, A = sum |x * w| over
the output's receptive field.  Outputs start as NaN, so an element no kernel
writes fails.
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


def _expected_algo(wl):
    """The grid's largest depthwise 14x14 shape (2048 planes, two per wave)
    runs on the packed depthwise kernel; every other shape on the grouped
    kernels: the register kernel when W is a multiple of 4, else the LDS band
    kernel (its band fits at these widths for 16 channels per group too)."""
    if wl.C // wl.groups == 1 and wl.H == 14 and wl.N * wl.C >= 2048:
        return gc.ALGO_DEPTHWISE
    return gc.ALGO_GROUPED3X3


def _run(d, x, w, ho, wo, wl):
    y = torch.full((wl.N, wl.K, ho, wo), float("nan"), device="cuda")
    gc.conv_fwd(d, x, w, None, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("name", list(synth.ATLAS_GRID))
def test_grid_shape_full_output(name):
    wl = synth.ATLAS_GRID[name]
    print("[grid] %s" % name, file=sys.stderr, flush=True)
    inp = synth.make_inputs(wl)
    ref, A = oracle.conv2d(inp["x"], inp["w"], None, wl.stride, wl.pad, wl.dil, wl.groups)
    x = torch.from_numpy(inp["x"]).cuda()
    w = torch.from_numpy(inp["w"]).cuda()
    bound = CONV_RTOL * A + CONV_ATOL
    for algo in (gc.ALGO_AUTO, gc.ALGO_DIRECT):
        d = gc.conv_desc_create(wl.N, wl.C, wl.H, wl.W, wl.K, wl.R, wl.S, wl.stride, wl.pad, wl.dil, wl.groups)
        gc.conv_desc_set_algo(d, algo)
        chosen = gc.conv_desc_get_algo(d)
        if algo == gc.ALGO_AUTO:
            assert chosen == _expected_algo(wl), "AUTO chose %s" % gc.ALGO_NAMES[chosen]
        ho, wo = gc.conv_desc_get_output_dims(d)
        y = _run(d, x, w, ho, wo, wl)
        err = np.abs(y.astype(np.float64) - ref)
        bad = ~(err <= bound)
        assert not bad.any(), "%s (%s): %d outputs over the bar, max err %r" % (
            name, gc.ALGO_NAMES[chosen], int(bad.sum()), float(np.nanmax(err)))
