"""GPU parity of the implicit GEMM on dense and 32-channel-group layers at
full size (ResNet- and ResNeXt-style shapes at batch 16: 3x3 at stride 1 and
2, a 1x1 reduction; a dilated 3x3, dense 5x5 and 7x7 at stride 2), through
the C ABI, against the CPU oracle on sampled outputs: random ones plus every
border pixel of three planes.

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


@pytest.mark.parametrize("name", list(synth.IGEMM_WORKLOADS))
def test_igemm_layer_full_size_sampled(name):
    wl = synth.IGEMM_WORKLOADS[name]
    print("[parity] implicit GEMM full-size sampled %s" % name, file=sys.stderr, flush=True)
    inp = synth.make_inputs(wl)
    bias = synth.normal((wl.K,), 0.5, wl.seed, 7)
    d = gc.conv_desc_create(wl.N, wl.C, wl.H, wl.W, wl.K, wl.R, wl.S, wl.stride, wl.pad, wl.dil, wl.groups)
    assert gc.conv_desc_get_algo(d) == gc.ALGO_IGEMM
    ho, wo = gc.conv_desc_get_output_dims(d)
    y = torch.full((wl.N, wl.K, ho, wo), float("nan"), device="cuda")
    gc.conv_fwd(d, torch.from_numpy(inp["x"]).cuda(), torch.from_numpy(inp["w"]).cuda(),
                torch.from_numpy(bias).cuda(), y)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert not np.isnan(y).any(), "unwritten outputs"
    idx = _sample_indices(y.shape, 6000, wl.seed)
    y_ref, A = oracle.conv2d_points(inp["x"], inp["w"], idx, bias, wl.stride, wl.pad, wl.dil, wl.groups)
    err = np.abs(y.ravel()[idx].astype(np.float64) - y_ref)
    bad = ~(err <= CONV_RTOL * A + CONV_ATOL)
    assert not bad.any(), "%s: %d sampled outputs over the bar, max err %r" % (name, int(bad.sum()), float(err.max()))
