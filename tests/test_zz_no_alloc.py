"""The allocation-free fused entry point (conv_fused_gn_fwd_noalloc) against
conv_fused_gn_fwd with a caller workspace, through the C ABI.

Both run the same kernels in the same order, so their outputs must agree to
the GroupNorm bar (|difference| <= 1e-4) and in fact bit for bit.  Two calls
in a row, the second on a smaller problem, show that the static scratch
array carries nothing from one call into the next."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
import grouped_convolution_conv_amd as gc

pytestmark = pytest.mark.gpu

GN_ATOL = 1e-4


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _run_both(wl, algo=gc.ALGO_AUTO, variant=gc.FUSED_AUTO):
    inp = synth.make_inputs(wl)
    t = {k: (torch.from_numpy(v).cuda() if v is not None else None) for k, v in inp.items()}
    d = gc.conv_desc_create(wl.N, wl.C, wl.H, wl.W, wl.K, wl.R, wl.S, wl.stride, wl.pad, wl.dil, wl.groups)
    gc.conv_desc_set_algo(d, algo)
    gc.conv_desc_set_fused_variant(d, variant)
    ho, wo = gc.conv_desc_get_output_dims(d)
    nbytes = gc.conv_fused_gn_workspace_size(d, wl.gn_groups)
    assert nbytes <= gc.conv_fused_gn_noalloc_limit()
    ws = torch.full((max(nbytes, 16),), 0xFF, dtype=torch.uint8, device="cuda")
    y_ref = torch.full((wl.N, wl.K, ho, wo), float("nan"), device="cuda")
    gc.conv_fused_gn_fwd(d, t["x"], t["w"], t["bias"], t["scale"], t["gamma"], t["beta"], wl.gn_groups, wl.eps,
                         y_ref, ws)
    y = torch.full_like(y_ref, float("nan"))
    gc.conv_fused_gn_fwd_noalloc(d, t["x"], t["w"], t["bias"], t["scale"], t["gamma"], t["beta"], wl.gn_groups,
                                 wl.eps, y)
    torch.cuda.synchronize()
    return y.cpu().numpy(), y_ref.cpu().numpy()


def _check(y, y_ref, what):
    assert not np.isnan(y).any(), what + ": unwritten outputs"
    err = float(np.max(np.abs(y.astype(np.float64) - y_ref.astype(np.float64))))
    assert err <= GN_ATOL, "%s: max |noalloc - workspace| %r > 1e-4" % (what, err)
    assert np.array_equal(y, y_ref), "%s: not bitwise equal (max diff %r)" % (what, err)


C5 = synth.WORKLOADS["c5_fused_gn"]


@pytest.mark.parametrize("algo,variant", [(gc.ALGO_AUTO, gc.FUSED_AUTO), (gc.ALGO_AUTO, gc.FUSED_STORE),
                                          (gc.ALGO_AUTO, gc.FUSED_ONEPASS), (gc.ALGO_DIRECT, gc.FUSED_AUTO)])
def test_noalloc_matches_workspace_entry_point_twice(algo, variant):
    """A larger call, then a smaller one on the same scratch array."""
    big = C5.with_(N=8, H=130, W=132)
    small = C5.with_(N=2, H=42, W=70, seed=C5.seed + 1)
    for wl in (big, small):
        _say("[noalloc]", gc.ALGO_NAMES[algo], gc.FUSED_NAMES[variant], "N=%d %dx%d" % (wl.N, wl.H, wl.W))
        y, y_ref = _run_both(wl, algo, variant)
        _check(y, y_ref, "%s %s N=%d %dx%d" % (gc.ALGO_NAMES[algo], gc.FUSED_NAMES[variant], wl.N, wl.H, wl.W))


@pytest.mark.parametrize("variant", [gc.FUSED_AUTO, gc.FUSED_STORE])
def test_noalloc_full_size_fused_workload(variant):
    """The full fused workload (64 images, 4 MiB of statistics) fits the
    scratch array, in the recompute organisation (the default there) and in
    the store organisation (batch slices)."""
    _say("[noalloc] full-size fused workload", gc.FUSED_NAMES[variant])
    y, y_ref = _run_both(C5, variant=variant)
    _check(y, y_ref, "full fused workload " + gc.FUSED_NAMES[variant])


def test_noalloc_refuses_problems_beyond_the_scratch_limit():
    wl = C5.with_(N=1024)
    d = gc.conv_desc_create(wl.N, wl.C, wl.H, wl.W, wl.K, wl.R, wl.S, wl.stride, wl.pad, wl.dil, wl.groups)
    assert gc.conv_fused_gn_workspace_size(d, wl.gn_groups) > gc.conv_fused_gn_noalloc_limit()
    fake = 1 << 20  # never dereferenced: the call refuses before enqueuing anything
    with pytest.raises(gc.GconvError) as ei:
        gc.conv_fused_gn_fwd_noalloc(d, fake, fake, fake, fake, None, None, wl.gn_groups, wl.eps, fake)
    assert ei.value.status == gc.GCONV_ERR_SCRATCH_LIMIT
