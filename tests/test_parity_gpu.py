"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars (written into every check below):
  conv:      |y_gpu - y_oracle| <= 1e-4 * A + 1e-6 at every compared output,
             A = sum |x * w| over the output's receptive field;
  GroupNorm: |out_gpu - out_oracle| <= 1e-4 at every compared output;
  integer-valued inputs: bit-for-bit equality (every partial sum is an
             exactly representable integer, so any summation order is exact).
Outputs are pre-filled with NaN so that an element a kernel fails to write
fails the comparison.
"""
import math
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import synth
import grouped_convolution_conv_amd as gc

pytestmark = pytest.mark.gpu

CONV_RTOL, CONV_ATOL, GN_ATOL = 1e-4, 1e-6, 1e-4


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _desc(wl):
    return gc.conv_desc_create(wl.N, wl.C, wl.H, wl.W, wl.K, wl.R, wl.S, wl.stride, wl.pad, wl.dil, wl.groups)


def gpu_conv(wl, inp, algo=gc.ALGO_AUTO, bias=None, y_offset=0):
    d = _desc(wl)
    gc.conv_desc_set_algo(d, algo)
    ho, wo = gc.conv_desc_get_output_dims(d)
    x, w, b = _dev(inp["x"]), _dev(inp["w"]), _dev(bias)
    n_out = wl.N * wl.K * ho * wo
    ybuf = torch.full((n_out + y_offset,), float("nan"), device="cuda")
    y = ybuf[y_offset:]
    gc.conv_fwd(d, x, w, b, y.data_ptr() if y_offset else y)
    torch.cuda.synchronize()
    return y.view(wl.N, wl.K, ho, wo).cpu().numpy(), gc.conv_desc_get_algo(d)


def gpu_fused(wl, inp, algo=gc.ALGO_AUTO, gn_groups=None, variant=gc.FUSED_AUTO, wait_us=None, y_offset=0):
    gn_groups = gn_groups or wl.gn_groups
    d = _desc(wl)
    gc.conv_desc_set_algo(d, algo)
    gc.conv_desc_set_fused_variant(d, variant)
    if wait_us is not None:
        gc.conv_desc_set_fused_wait(d, wait_us)
    ho, wo = gc.conv_desc_get_output_dims(d)
    ws = torch.empty(max(1, gc.conv_fused_gn_workspace_size(d, gn_groups)), dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)  # the kernels must not rely on its contents
    # y_offset floats into a larger buffer: an output that is not 8- or
    # 16-byte aligned
    ybuf = torch.full((wl.N * wl.K * ho * wo + y_offset,), float("nan"), device="cuda")
    y = ybuf[y_offset:].view(wl.N, wl.K, ho, wo)
    gc.conv_fused_gn_fwd(d, _dev(inp["x"]), _dev(inp["w"]), _dev(inp["bias"]), _dev(inp["scale"]),
                         _dev(inp.get("gamma")), _dev(inp.get("beta")), gn_groups, wl.eps, y, ws)
    torch.cuda.synchronize()
    assert y_offset == 0 or bool(torch.isnan(ybuf[:y_offset]).all()), "write before the output"
    return y.cpu().numpy()


def check_conv(y_gpu, y_ref, A, what):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bound = CONV_RTOL * A + CONV_ATOL
    ok = err <= bound
    if not np.all(ok):
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError("%s: %d of %d outputs outside 1e-4*A+1e-6; first at %s: gpu %r oracle %r A %r"
                             % (what, len(bad), err.size, i, y_gpu[i], y_ref[i], A[i]))
    return float(np.max(err / bound))


def oracle_conv(wl, inp, bias=None):
    return oracle.conv2d(inp["x"], inp["w"], bias, wl.stride, wl.pad, wl.dil, wl.groups)


# Reduced versions of the workloads: the oracle finishes them in seconds, and
# they still span several tiles and ragged tails.
W = synth.WORKLOADS
SMALL = {
    "c1_grouped_cpg4": W["c1_grouped_cpg4"],
    "c2_depthwise_144": W["c2_depthwise_144"],
    "c3a_grouped_g64": W["c3a_grouped_g64"].with_(N=2),
    "c3b_grouped_g128": W["c3b_grouped_g128"].with_(N=2),
    "c3c_depthwise_g256": W["c3c_depthwise_g256"].with_(N=2),
    "c4_dense_5x9": W["c4_dense_5x9"].with_(N=1, H=44, W=75),        # out 40 x 67: 5 x 2 tiles
    "c5_fused_gn": W["c5_fused_gn"].with_(N=2, H=42, W=70),          # out 40 x 68
}
AUTO_ALGO = {"c1_grouped_cpg4": gc.ALGO_GROUPED3X3, "c2_depthwise_144": gc.ALGO_GROUPED3X3,
             "c3a_grouped_g64": gc.ALGO_GROUPED3X3, "c3b_grouped_g128": gc.ALGO_GROUPED3X3,
             "c3c_depthwise_g256": gc.ALGO_GROUPED3X3, "c4_dense_5x9": gc.ALGO_IGEMM,
             "c5_fused_gn": gc.ALGO_IGEMM}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("algo", [gc.ALGO_AUTO, gc.ALGO_DIRECT])
def test_conv_small_workloads(name, algo):
    wl = SMALL[name]
    _say("[parity] conv", name, gc.ALGO_NAMES[algo], wl)
    inp = synth.make_inputs(wl)
    y, used = gpu_conv(wl, inp, algo)
    assert used == (AUTO_ALGO[name] if algo == gc.ALGO_AUTO else algo)
    y_ref, A = oracle_conv(wl, inp)
    r = check_conv(y, y_ref, A, name)
    _say("   max err/bound %.3g" % r)


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("algo", [gc.ALGO_AUTO, gc.ALGO_DIRECT])
def test_conv_integer_inputs_bit_exact(name, algo):
    wl = SMALL[name].with_(x_dist=("int", -2, 2), w_dist=("int", -2, 2), seed=SMALL[name].seed + 500)
    _say("[parity] int", name, gc.ALGO_NAMES[algo])
    inp = synth.make_inputs(wl)
    y, _ = gpu_conv(wl, inp, algo)
    y_ref, _ = oracle_conv(wl, inp)
    assert np.array_equal(y.astype(np.float64), y_ref)


@pytest.mark.parametrize("name", list(SMALL))
def test_conv_with_bias(name):
    wl = SMALL[name]
    inp = synth.make_inputs(wl)
    bias = synth.normal((wl.K,), 0.5, wl.seed, 7)
    _say("[parity] bias", name)
    for algo in (gc.ALGO_AUTO, gc.ALGO_DIRECT):
        y, _ = gpu_conv(wl, inp, algo, bias=bias)
        y_ref, A = oracle_conv(wl, inp, bias)
        check_conv(y, y_ref, A, name + " bias")


def _sample_indices(shape, n_random, seed):
    """Random flat indices plus every border pixel of a few planes."""
    N, K, Ho, Wo = shape
    rng = np.random.default_rng(seed)
    idx = [rng.integers(0, N * K * Ho * Wo, n_random)]
    for (n, k) in [(0, 0), (N - 1, K - 1), (N // 2, K // 3)]:
        base = (n * K + k) * Ho * Wo
        rows = np.arange(Wo)
        cols = np.arange(Ho) * Wo
        idx += [base + rows, base + (Ho - 1) * Wo + rows, base + cols, base + cols + Wo - 1]
    return np.unique(np.concatenate(idx))


def check_conv_whole(wl, inp, y, chunk):
    """Every output of y against the oracle, `chunk` images at a time (the
    oracle's FP64 output and bound of a whole full-size batch would hold
    several GB of host memory at once)."""
    worst = 0.0
    for n0 in range(0, wl.N, chunk):
        n1 = min(wl.N, n0 + chunk)
        y_ref, A = oracle.conv2d(inp["x"][n0:n1], inp["w"], None, wl.stride, wl.pad, wl.dil, wl.groups)
        worst = max(worst, check_conv(y[n0:n1], y_ref, A, "%s images %d..%d" % (wl.name, n0, n1 - 1)))
        del y_ref, A
    return worst


CONV_ROWS = [n for n in synth.ROW_ORDER if not W[n].fused]


@pytest.mark.parametrize("name", CONV_ROWS)
def test_conv_full_size_whole_output(name):
    """The full workload in the launch configuration the benchmark times,
    every output element against the oracle."""
    wl = W[name]
    _say("[parity] full-size whole output", name)
    inp = synth.make_inputs(wl)
    y, used = gpu_conv(wl, inp)
    assert used == AUTO_ALGO[name]
    r = check_conv_whole(wl, inp, y, chunk=max(1, (1 << 22) // (wl.K * y.shape[2] * y.shape[3])))
    _say("   max err/bound %.3g" % r)


# Mid-size cases that take the same kernel instances as the full-size rows.
MID = {
    # dense 5x9 with W and the padding multiples of 4 and a 16-byte aligned
    # x (16-byte band loads), more than 32 output columns (two 32-column
    # blocks per wave row) and 4 x 64 x 17 x 4 = 544 >= 512 workgroups
    # (8-row tiles): the instance the benchmark times on the dense row;
    # 129 x 252 outputs leave a ragged last tile row and column
    "c4_mid_vec_8row": W["c4_dense_5x9"].with_(N=4, H=133, W=260),
    # 3x3, 8 -> 32 and 8 -> 64 channels, pad 0, W a multiple of 4: the
    # resident-weight MFMA kernel with 16-byte band loads (the fused
    # workload's instance), ragged rows and columns
    "res_vec_k32": W["c5_fused_gn"].with_(N=2, H=42, W=68, bias_dist=None, scale_dist=None, gn_groups=0),
    "res_vec_k64": W["c5_fused_gn"].with_(N=2, K=64, H=45, W=132, bias_dist=None, scale_dist=None, gn_groups=0),
}


@pytest.mark.parametrize("name", list(MID))
def test_conv_mid_size_whole_output(name):
    wl = MID[name]
    _say("[parity] mid-size whole output", name, wl)
    inp = synth.make_inputs(wl)
    y, used = gpu_conv(wl, inp)
    assert used == gc.ALGO_IGEMM
    y_ref, A = oracle_conv(wl, inp)
    r = check_conv(y, y_ref, A, name)
    wi = wl.with_(x_dist=("int", -2, 2), w_dist=("int", -2, 2), seed=wl.seed + 500)
    inp = synth.make_inputs(wi)
    y, _ = gpu_conv(wi, inp)
    y_ref, _ = oracle_conv(wi, inp)
    assert np.array_equal(y.astype(np.float64), y_ref), name + " integer inputs"
    _say("   max err/bound %.3g, integer inputs bit-exact" % r)


# ------------------------------------------------------------------ fused chain


def check_gn(out_gpu, out_ref, what):
    err = np.abs(out_gpu.astype(np.float64) - out_ref)
    if not np.all(err <= GN_ATOL):
        i = np.unravel_index(np.nanargmax(np.where(np.isnan(err), np.inf, err)), err.shape)
        raise AssertionError("%s: max |err| %r > 1e-4 at %s (gpu %r oracle %r)"
                             % (what, float(np.nanmax(err)) if not np.isnan(err).all() else float("nan"),
                                i, out_gpu[i], out_ref[i]))
    return float(err.max())


def oracle_fused(wl, inp, gn_groups=None):
    return oracle.fused_gn(inp["x"], inp["w"], inp["bias"], inp["scale"], inp.get("gamma"), inp.get("beta"),
                           gn_groups or wl.gn_groups, wl.eps, wl.stride, wl.pad, wl.dil, wl.groups)


@pytest.mark.parametrize("algo,variant", [(gc.ALGO_AUTO, gc.FUSED_RECOMPUTE), (gc.ALGO_AUTO, gc.FUSED_STORE),
                                           (gc.ALGO_AUTO, gc.FUSED_ONEPASS), (gc.ALGO_DIRECT, gc.FUSED_AUTO)])
def test_fused_small(algo, variant):
    wl = SMALL["c5_fused_gn"]
    _say("[parity] fused small", gc.ALGO_NAMES[algo], gc.FUSED_NAMES[variant])
    inp = synth.make_inputs(wl)
    out = gpu_fused(wl, inp, algo, variant=variant)
    e = check_gn(out, oracle_fused(wl, inp), "fused c5 small")
    _say("   max |err| %.3g" % e)


@pytest.mark.parametrize("gn_groups", [1, 2, 4, 8, 16, 32])
def test_fused_group_counts(gn_groups):
    wl = SMALL["c5_fused_gn"].with_(N=1, H=23, W=37)
    inp = synth.make_inputs(wl)
    inp["gamma"] = synth.uniform((wl.K,), 0.5, 1.5, 5, 0)
    inp["beta"] = synth.uniform((wl.K,), -0.5, 0.5, 5, 1)
    _say("[parity] fused gn_groups", gn_groups)
    out = gpu_fused(wl, inp, gn_groups=gn_groups)
    check_gn(out, oracle_fused(wl, inp, gn_groups), "gn_groups=%d" % gn_groups)


def test_fused_other_geometries():
    # padded, stride 2, wider channel counts: stage A takes the direct kernel,
    # the chunked MFMA kernel or the resident-weight MFMA kernel (both
    # variants) according to the geometry
    cases = [W["c5_fused_gn"].with_(N=1, H=19, W=21, pad=1),
             W["c5_fused_gn"].with_(N=1, H=19, W=21, stride=2),
             W["c5_fused_gn"].with_(N=2, C=16, K=64, H=17, W=33, gn_groups=16),
             W["c5_fused_gn"].with_(N=2, C=8, K=64, H=17, W=70, gn_groups=16),
             W["c5_fused_gn"].with_(N=2, C=5, K=32, H=21, W=67, pad=1),
             W["c5_fused_gn"].with_(N=1, C=4, K=32, H=12, W=140, R=1, S=1),
             W["c5_fused_gn"].with_(N=1, C=6, K=12, H=9, W=9, groups=3, gn_groups=3)]
    for wl in cases:
        inp = synth.make_inputs(wl)
        ref = oracle_fused(wl, inp)
        for variant in (gc.FUSED_AUTO, gc.FUSED_STORE, gc.FUSED_RECOMPUTE, gc.FUSED_ONEPASS):
            d = _desc(wl)
            gc.conv_desc_set_fused_variant(d, variant)
            try:
                gc.conv_desc_get_fused_variant(d, wl.gn_groups)
                out = gpu_fused(wl, inp, variant=variant)
            except gc.GconvError as e:
                assert variant in (gc.FUSED_RECOMPUTE, gc.FUSED_ONEPASS) and e.status == gc.GCONV_ERR_UNSUPPORTED
                continue
            _say("[parity] fused geometry", wl, gc.FUSED_NAMES[variant])
            check_gn(out, ref, "%s %s" % (wl, gc.FUSED_NAMES[variant]))


def test_fused_winograd_geometries():
    """The fused 3x3 passes with 32 output channels multiply in the Winograd
    form F(2x2, 3x3): 4- and 8-channel chunks (4, 5 and 8 input channels),
    16-byte and 4-byte band loads, ragged tiles, a random GroupNorm affine and
    wider value ranges, in the recompute and store organisations, compared
    whole with the oracle (the implicit GEMM forced: with 4 input channels and
    padding AUTO takes the register kernel)."""
    base = W["c5_fused_gn"]
    cases = [base.with_(N=2, C=4, H=30, W=68),
             base.with_(N=2, C=4, H=27, W=45, pad=1),
             base.with_(N=1, C=5, H=70, W=133),
             base.with_(N=2, C=8, H=35, W=36, x_dist=("uniform", -4.0, 4.0), w_dist=("uniform", -0.3, 0.3)),
             base.with_(N=1, C=7, H=66, W=20, pad=1, seed=base.seed + 7),
             # one output pixel; exactly one 64-column tile; a single output row
             base.with_(N=2, C=8, H=3, W=3, seed=base.seed + 8),
             base.with_(N=3, C=6, H=4, W=66, seed=base.seed + 9),
             base.with_(N=2, C=8, H=1, W=90, pad=1, seed=base.seed + 10),
             base.with_(N=1, C=8, H=3, W=68, seed=base.seed + 11)]
    for wl in cases:
        inp = synth.make_inputs(wl)
        inp["gamma"] = synth.uniform((wl.K,), 0.5, 1.5, wl.seed, 16)
        inp["beta"] = synth.uniform((wl.K,), -0.5, 0.5, wl.seed, 17)
        ref = oracle_fused(wl, inp)
        for variant in (gc.FUSED_RECOMPUTE, gc.FUSED_STORE):
            _say("[parity] fused Winograd form", wl, gc.FUSED_NAMES[variant])
            check_gn(gpu_fused(wl, inp, gc.ALGO_IGEMM, variant=variant), ref, "%s %s" % (wl, gc.FUSED_NAMES[variant]))


_FUSED_FULL_REF = {}


def _fused_full_reference(wl, inp, chunk=8):
    """Oracle output of the whole fused workload, computed once per session
    (float64, in image chunks)."""
    if wl not in _FUSED_FULL_REF:
        parts = []
        for n0 in range(0, wl.N, chunk):
            sl = dict(inp)
            sl["x"] = inp["x"][n0:n0 + chunk]
            parts.append(oracle_fused(wl.with_(N=sl["x"].shape[0]), sl))
        _FUSED_FULL_REF.clear()
        _FUSED_FULL_REF[wl] = np.concatenate(parts)
    return _FUSED_FULL_REF[wl]


@pytest.mark.parametrize("variant", [gc.FUSED_AUTO, gc.FUSED_STORE, gc.FUSED_RECOMPUTE, gc.FUSED_ONEPASS])
def test_fused_full_size_whole_output(variant):
    """The full fused workload in the benchmark's launch configuration
    (AUTO is the recompute organisation there), all 64 images compared
    whole with the oracle."""
    wl = W["c5_fused_gn"]
    _say("[parity] fused full size, whole output,", gc.FUSED_NAMES[variant])
    inp = synth.make_inputs(wl)
    out = gpu_fused(wl, inp, variant=variant)
    ref = _fused_full_reference(wl, inp)
    worst = 0.0
    for n0 in range(0, wl.N, 8):
        worst = max(worst, check_gn(out[n0:n0 + 8], ref[n0:n0 + 8], "c5 full, images %d..%d" % (n0, n0 + 7)))
    _say("   max |err| %.3g" % worst)


def test_fused_mid_size_vec_resident():
    """The fused chain on the resident-weight kernel with 16-byte band loads
    (W a multiple of 4), every organisation, with a random GroupNorm affine,
    compared whole."""
    wl = W["c5_fused_gn"].with_(N=3, H=42, W=68)
    inp = synth.make_inputs(wl)
    inp["gamma"] = synth.uniform((wl.K,), 0.5, 1.5, wl.seed, 14)
    inp["beta"] = synth.uniform((wl.K,), -0.5, 0.5, wl.seed, 15)
    ref = oracle_fused(wl, inp)
    for variant in (gc.FUSED_RECOMPUTE, gc.FUSED_STORE, gc.FUSED_ONEPASS):
        _say("[parity] fused mid-size vec", gc.FUSED_NAMES[variant])
        check_gn(gpu_fused(wl, inp, variant=variant), ref, "fused vec " + gc.FUSED_NAMES[variant])


@pytest.mark.parametrize("y_offset", [1, 2, 3])
def test_fused_output_alignment(y_offset):
    """The Winograd passes store a lane's two neighbouring columns with one
    8-byte store only when y is 8-byte aligned; an output 4 or 12 bytes off
    (odd offsets) takes the 4-byte stores, 8 bytes off the paired ones.  Every
    organisation, compared whole, and nothing written before the output."""
    wl = W["c5_fused_gn"].with_(N=2, H=42, W=68)
    inp = synth.make_inputs(wl)
    ref = oracle_fused(wl, inp)
    for variant in (gc.FUSED_RECOMPUTE, gc.FUSED_STORE, gc.FUSED_ONEPASS):
        _say("[parity] fused, y offset %d floats," % y_offset, gc.FUSED_NAMES[variant])
        check_gn(gpu_fused(wl, inp, variant=variant, y_offset=y_offset), ref,
                 "fused y+%d %s" % (y_offset, gc.FUSED_NAMES[variant]))


@pytest.mark.parametrize("case", ["small", "mid vec", "mid ragged", "full"])
def test_onepass_normalizes_the_same_bits_on_every_path(case):
    """The one-pass variant normalizes a tile in the conv pass once its
    image's statistics are ready, or leaves v for the trailing in-place pass
    after its bounded wait.  Forcing every tile onto the trailing pass (wait
    -1) or never waiting (wait 0, a mix of both paths) gives the same bits as
    the default, and the result matches the oracle."""
    wl = {"small": SMALL["c5_fused_gn"], "mid vec": W["c5_fused_gn"].with_(N=3, H=42, W=68),
          "mid ragged": W["c5_fused_gn"].with_(N=5, H=37, W=70), "full": W["c5_fused_gn"]}[case]
    inp = synth.make_inputs(wl)
    _say("[parity] one-pass paths,", case)
    base = gpu_fused(wl, inp, variant=gc.FUSED_ONEPASS)
    for wait in (0, -1):
        other = gpu_fused(wl, inp, variant=gc.FUSED_ONEPASS, wait_us=wait)
        assert np.array_equal(base, other), "%s: wait %d differs from the default" % (case, wait)
    n = min(wl.N, 4)
    sl = dict(inp)
    sl["x"] = inp["x"][:n]
    check_gn(base[:n], oracle_fused(wl.with_(N=n), sl), "one-pass %s, first %d images" % (case, n))


@pytest.mark.parametrize("affine", ["random", "none"])
def test_onepass_group_norm_affine(affine):
    """The one-pass variant applies gamma and beta (random, or absent: 1
    and 0) the same way on both of its paths: in the conv pass and in the
    trailing pass."""
    wl = W["c5_fused_gn"].with_(N=3, H=42, W=68)
    inp = synth.make_inputs(wl)
    if affine == "random":
        inp["gamma"] = synth.uniform((wl.K,), 0.5, 1.5, wl.seed, 12)
        inp["beta"] = synth.uniform((wl.K,), -0.5, 0.5, wl.seed, 13)
    else:
        inp["gamma"] = inp["beta"] = None
    _say("[parity] one-pass affine", affine)
    base = gpu_fused(wl, inp, variant=gc.FUSED_ONEPASS)
    assert np.array_equal(base, gpu_fused(wl, inp, variant=gc.FUSED_ONEPASS, wait_us=-1))
    check_gn(base, oracle_fused(wl, inp), "one-pass affine " + affine)


def test_onepass_images_larger_than_a_round():
    """Images of more tiles than the grid holds (1030 x 1030: 2193 tiles
    against at most a few hundred resident workgroups), so an image spans
    rounds of the grid and tiles wait for, or leave to the trailing pass,
    statistics that complete rounds later: every output matches the oracle
    and equals the all-trailing-pass result."""
    wl = W["c5_fused_gn"].with_(N=2, H=1030, W=1030)
    inp = synth.make_inputs(wl)
    _say("[parity] one-pass, images larger than a round")
    base = gpu_fused(wl, inp, variant=gc.FUSED_ONEPASS)
    assert np.array_equal(base, gpu_fused(wl, inp, variant=gc.FUSED_ONEPASS, wait_us=-1))
    check_gn(base, oracle_fused(wl, inp), "one-pass 2 x 1030 x 1030")


def test_fused_store_batch_slices_direct_stage():
    """The store variant runs over slices of the batch (v of a slice sized
    for the last-level cache): 66 images of 32 x 128 x 128 outputs make a
    slice of 64 and one of 2.  The direct kernel runs stage A here; the
    images at both slice edges are compared whole."""
    wl = W["c5_fused_gn"].with_(N=66, H=130, W=130)
    inp = synth.make_inputs(wl)
    _say("[parity] fused store slices, direct stage A")
    out = gpu_fused(wl, inp, algo=gc.ALGO_DIRECT, variant=gc.FUSED_STORE)
    for n in (0, 63, 64, 65):
        sl = dict(inp)
        sl["x"] = inp["x"][n:n + 1]
        ref = oracle_fused(wl.with_(N=1), sl)
        check_gn(out[n:n + 1], ref, "store slices, sample %d" % n)


# ------------------------------------------------------------------ geometry fuzz and edges


def _fuzz_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        groups = int(rng.choice([1, 1, 2, 3, 4]))
        cin = int(rng.choice([1, 2, 3, 4, 5, 8, 9]))
        cout = int(rng.choice([1, 2, 4, 8, 33, 40]))
        R, S = int(rng.integers(1, 10)), int(rng.integers(1, 10))
        st, pad, dil = int(rng.integers(1, 4)), int(rng.integers(0, 3)), int(rng.integers(1, 3))
        H, W_ = int(rng.integers(1, 40)), int(rng.integers(1, 80))
        if H + 2 * pad - dil * (R - 1) - 1 < 0 or W_ + 2 * pad - dil * (S - 1) - 1 < 0:
            continue
        out.append(synth.Workload("fuzz%d" % len(out), int(rng.integers(1, 3)), groups * cin, H, W_,
                                  groups * cout, R, S, st, pad, dil, groups, 3000 + len(out),
                                  ("uniform", -1.0, 1.0), ("uniform", -0.5, 0.5)))
    return out


@pytest.mark.parametrize("wl", _fuzz_cases(40, 11), ids=lambda w: w.name)
def test_conv_geometry_fuzz(wl):
    inp = synth.make_inputs(wl)
    y_ref, A = oracle_conv(wl, inp)
    for algo in (gc.ALGO_AUTO, gc.ALGO_DIRECT, gc.ALGO_IGEMM, gc.ALGO_GROUPED3X3, gc.ALGO_DEPTHWISE):
        d = _desc(wl)
        try:
            gc.conv_desc_set_algo(d, algo)
        except gc.GconvError:
            continue
        y, _ = gpu_conv(wl, inp, algo)
        check_conv(y, y_ref, A, "%s %s" % (wl, gc.ALGO_NAMES[algo]))



def _flat_cases(n, seed):
    """Geometries for the flattened-pixel implicit GEMM: square 1x1-7x7
    kernels, stride 1 and 2, dilation 1 and 2 (3x3), any padding up to 3,
    small ragged images whose 128-pixel tiles span rows and images, 4-12
    input and 8-40 output channels per group."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        R = int(rng.choice([1, 3, 3, 5, 7]))
        st = int(rng.integers(1, 3))
        dil = int(rng.choice([1, 2])) if R == 3 else 1
        pad = int(rng.integers(0, 4))
        H, W_ = int(rng.integers(5, 41)), int(rng.integers(5, 41))
        if H + 2 * pad - dil * (R - 1) - 1 < 0 or W_ + 2 * pad - dil * (R - 1) - 1 < 0:
            continue
        groups = int(rng.choice([1, 1, 2, 3]))
        cin, cout = int(rng.integers(4, 13)), int(rng.choice([8, 16, 33, 40]))
        out.append(synth.Workload("flat%d_r%d_s%d_d%d" % (len(out), R, st, dil), int(rng.integers(1, 6)), groups * cin,
                                  H, W_, groups * cout, R, R, st, pad, dil, groups, 7000 + len(out),
                                  ("uniform", -1.0, 1.0), ("uniform", -0.5, 0.5)))
    return out


@pytest.mark.parametrize("wl", _flat_cases(30, 17), ids=lambda w: w.name)
def test_flattened_implicit_gemm_fuzz(wl):
    inp = synth.make_inputs(wl)
    y_ref, A = oracle_conv(wl, inp)
    for algo in (gc.ALGO_AUTO, gc.ALGO_IGEMM):
        d = _desc(wl)
        try:
            gc.conv_desc_set_algo(d, algo)
        except gc.GconvError:
            continue
        y, _ = gpu_conv(wl, inp, algo)
        check_conv(y, y_ref, A, "%s %s" % (wl.name, gc.ALGO_NAMES[algo]))

def _factorized_cases(n, seed):
    """Factorized kernels (1x3, 3x1, 1x7, 7x1) at stride 1: padding chosen per
    axis up to 4, small ragged images (either the row x column tiles or the
    flattened-pixel tiles), 3-12 input and 8-40 output channels per group."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        R, S = [(1, 3), (3, 1), (1, 7), (7, 1)][int(rng.integers(0, 4))]
        ph, pw = int(rng.integers(0, 5)), int(rng.integers(0, 5))
        H, W_ = int(rng.integers(3, 41)), int(rng.integers(3, 72))
        if H + 2 * ph - R < 0 or W_ + 2 * pw - S < 0:
            continue
        groups = int(rng.choice([1, 1, 2]))
        cin, cout = int(rng.integers(3, 13)), int(rng.choice([8, 16, 33, 40]))
        out.append(synth.Workload("fact%d_%dx%d_p%d%d" % (len(out), R, S, ph, pw), int(rng.integers(1, 5)),
                                  groups * cin, H, W_, groups * cout, R, S, 1, (ph, pw), 1, groups, 7500 + len(out),
                                  ("uniform", -1.0, 1.0), ("uniform", -0.5, 0.5)))
    return out


@pytest.mark.parametrize("wl", _factorized_cases(16, 29), ids=lambda w: w.name)
def test_factorized_implicit_gemm_fuzz(wl):
    inp = synth.make_inputs(wl)
    y_ref, A = oracle_conv(wl, inp)
    for algo in (gc.ALGO_AUTO, gc.ALGO_IGEMM):
        y, _ = gpu_conv(wl, inp, algo)
        check_conv(y, y_ref, A, "%s %s" % (wl.name, gc.ALGO_NAMES[algo]))


WINO_COLUMNS = [
    # kernels 3 wide at stride 1 on 64-column tiles: Winograd columns
    synth.Workload("wgcol_3x3_p1", 2, 20, 12, 64, 40, 3, 3, 1, 1, 1, 1, 131, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("wgcol_3x3_vec", 2, 16, 10, 64, 32, 3, 3, 1, 0, 1, 1, 132, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("wgcol_3x3_odd_w", 1, 12, 9, 63, 33, 3, 3, 1, 0, 1, 1, 133, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("wgcol_1x3", 2, 12, 8, 64, 32, 1, 3, 1, (0, 1), 1, 1, 134, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("wgcol_cpg32", 1, 64, 16, 128, 64, 3, 3, 1, 1, 1, 2, 135, ("uniform", -1, 1), ("uniform", -1, 1)),
]


@pytest.mark.parametrize("wl", WINO_COLUMNS, ids=lambda w: w.name)
def test_winograd_columns_whole_output(wl):
    """Plain convs 3 wide at stride 1 on 64-column tiles run the implicit
    GEMM with Winograd columns: every output against the oracle, and integer
    inputs bit for bit (the transforms' halves are exact there)."""
    inp = synth.make_inputs(wl)
    y_ref, A = oracle_conv(wl, inp)
    y, algo = gpu_conv(wl, inp)
    assert algo == gc.ALGO_IGEMM, gc.ALGO_NAMES[algo]
    check_conv(y, y_ref, A, wl.name)
    wi = wl.with_(x_dist=("int", -2, 2), w_dist=("int", -2, 2), seed=wl.seed + 500)
    inp = synth.make_inputs(wi)
    y, _ = gpu_conv(wi, inp)
    y_ref, _ = oracle_conv(wi, inp)
    assert np.array_equal(y.astype(np.float64), y_ref), wl.name + " integer inputs"
    # an output 4 bytes off 8-byte alignment: the 4-byte stores
    y1, _ = gpu_conv(wi, inp, y_offset=1)
    assert np.array_equal(y1.astype(np.float64), y_ref), wl.name + " integer inputs, y offset 1 float"


EDGE = [
    synth.Workload("one_pixel", 2, 4, 1, 1, 4, 3, 3, 1, 1, 1, 4, 41, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("w5_tail", 1, 8, 7, 5, 8, 3, 3, 1, 1, 1, 2, 42, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("w33_tail", 1, 4, 9, 33, 8, 3, 3, 1, 1, 1, 4, 43, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("wide_300", 1, 2, 5, 300, 2, 3, 3, 1, 1, 1, 2, 44, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("cout3", 1, 8, 10, 10, 6, 3, 3, 1, 1, 1, 2, 45, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("rows_h37_cob2", 2, 8, 37, 64, 16, 3, 3, 1, 1, 1, 2, 51, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("rows_w252", 1, 4, 9, 252, 4, 3, 3, 1, 1, 1, 4, 52, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("rows_w20_cpg2", 3, 6, 11, 20, 6, 3, 3, 1, 1, 1, 3, 53, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("rows_h1", 2, 8, 1, 8, 8, 3, 3, 1, 1, 1, 8, 54, ("uniform", -1, 1), ("uniform", -1, 1)),
    # depthwise with enough waves for 4 rows per lane, H not a multiple of 4
    synth.Workload("rows_rb4_h30", 64, 128, 30, 16, 128, 3, 3, 1, 1, 1, 128, 58, ("uniform", -1, 1), ("uniform", -1, 1)),
    # a whole 256-column row per wave, one lane strip per wave
    synth.Workload("rows_w256_cpg4", 1, 8, 5, 256, 8, 3, 3, 1, 1, 1, 2, 59, ("uniform", -1, 1), ("uniform", -1, 1)),
    # tiny: one row per lane
    synth.Workload("rows_rb1_w4", 1, 2, 3, 4, 2, 3, 3, 1, 1, 1, 1, 60, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("res_cin5_pad1", 2, 5, 13, 70, 32, 3, 3, 1, 1, 1, 1, 55, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("res_cin4_k40", 1, 4, 19, 131, 40, 3, 3, 1, 0, 1, 1, 56, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("res_1x1_k64", 2, 8, 9, 66, 64, 1, 1, 1, 0, 1, 1, 57, ("uniform", -1, 1), ("uniform", -1, 1)),
    # wide groups on the register kernel: 8 and 16 input channels per group,
    # blocks of 4, 2 or 1 output channels, one or two rows per lane, ragged H;
    # the misaligned-y pass takes the implicit GEMM or the direct kernel
    synth.Workload("rows_cpg8_cob8", 2, 32, 13, 36, 32, 3, 3, 1, 1, 1, 4, 61, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("rows_cpg16_h9", 3, 64, 9, 20, 64, 3, 3, 1, 1, 1, 4, 62, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("rows_cpg8_cout4", 1, 16, 11, 8, 8, 3, 3, 1, 1, 1, 2, 63, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("rows_cpg16_cout12", 2, 32, 7, 64, 24, 3, 3, 1, 1, 1, 2, 64, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("rows_cpg8_w256_rb2", 8, 64, 37, 256, 64, 3, 3, 1, 1, 1, 8, 65, ("uniform", -1, 1), ("uniform", -1, 1)),
    # wide groups with W not a multiple of 4: the LDS band kernel (and wider
    # than 256 with a band over 64 KB: the implicit GEMM)
    synth.Workload("band_cpg16_w14", 2, 64, 14, 14, 64, 3, 3, 1, 1, 1, 4, 67, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("band_cpg16_cout8_w14", 2, 32, 14, 14, 16, 3, 3, 1, 1, 1, 2, 74, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("band_cpg8_w30", 8, 256, 9, 30, 256, 3, 3, 1, 1, 1, 32, 68, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("wide_w260_igemm", 1, 32, 6, 260, 32, 3, 3, 1, 1, 1, 4, 69, ("uniform", -1, 1), ("uniform", -1, 1)),
    # 16 input and 16 output channels per group with enough waves: the FP32
    # matrix-core kernel (blocks of 16 columns: 4, 2 or 1 per wave; ragged
    # rows, partial blocks, three column segments)
    synth.Workload("mfma16_h97_w40", 4, 128, 97, 40, 128, 3, 3, 1, 1, 1, 8, 70, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("mfma16_h193_w20", 2, 128, 193, 20, 128, 3, 3, 1, 1, 1, 8, 71, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("mfma16_h100_w9", 4, 128, 100, 9, 128, 3, 3, 1, 1, 1, 8, 72, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("mfma16_h200_w150", 2, 64, 200, 150, 64, 3, 3, 1, 1, 1, 4, 73, ("uniform", -1, 1), ("uniform", -1, 1)),
    # enough waves for 2 output channels per lane, not for 4 (16 in / 16 out
    # per group takes the matrix cores; 16 in / 8 out the register kernel)
    synth.Workload("rows_cpg16_co2", 4, 64, 37, 256, 64, 3, 3, 1, 1, 1, 4, 66, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("rows_cpg16_cout8_co2", 6, 64, 37, 256, 32, 3, 3, 1, 1, 1, 4, 75, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_k8", 1, 16, 12, 40, 8, 3, 3, 1, 0, 1, 1, 46, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_cin5_pad2", 2, 5, 13, 70, 40, 5, 5, 1, 2, 1, 1, 47, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_k96_1x1", 1, 12, 9, 65, 96, 1, 1, 1, 0, 1, 1, 48, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_groups2", 1, 16, 11, 35, 128, 7, 7, 1, 3, 1, 2, 49, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_5x9_K130", 1, 6, 12, 40, 130, 5, 9, 1, 1, 1, 1, 50, ("uniform", -1, 1), ("uniform", -1, 1)),
    # stride 2 on the implicit GEMM (1x1 and 3x3): ragged row and column
    # tiles, a partial channel chunk, a partial 32-channel block, no padding,
    # 32 channels per group, and a grouped layer too wide for the register
    # kernel
    synth.Workload("igemm_s2_dense3", 2, 8, 19, 70, 40, 3, 3, 2, 1, 1, 1, 76, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_s2_1x1", 2, 6, 17, 131, 16, 1, 1, 2, 0, 1, 1, 77, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_s2_cpg32", 1, 64, 14, 14, 64, 3, 3, 2, 1, 1, 2, 78, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_s2_p0", 1, 16, 20, 20, 32, 3, 3, 2, 0, 1, 1, 79, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_s2_tall", 1, 4, 40, 9, 8, 3, 3, 2, 1, 1, 1, 80, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_s2_grouped_w600", 1, 8, 5, 600, 16, 3, 3, 2, 1, 1, 2, 81, ("uniform", -1, 1), ("uniform", -1, 1)),
    # exactly 32 output columns (the one-block-wide tile), 3 channel chunks,
    # a partial third 32-channel block
    synth.Workload("igemm_s2_w32_k72", 1, 12, 10, 64, 72, 3, 3, 2, 1, 1, 1, 82, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_s2_1x1_w32", 2, 9, 9, 64, 40, 1, 1, 2, 0, 1, 1, 83, ("uniform", -1, 1), ("uniform", -1, 1)),
    # stride 1 on outputs at most 32 wide (the one-block-wide tile): with
    # the 16-byte band loads (W and padding multiples of 4) and without
    synth.Workload("igemm_n_w32_1x1_vec", 2, 16, 10, 32, 40, 1, 1, 1, 0, 1, 1, 84, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_n_w12_5x5_vec", 1, 8, 16, 16, 32, 5, 5, 1, 0, 1, 1, 85, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_n_w28_cpg32", 2, 64, 28, 28, 64, 3, 3, 1, 1, 1, 2, 86, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_n_w15_7x7", 1, 6, 9, 15, 16, 7, 7, 1, 3, 1, 1, 87, ("uniform", -1, 1), ("uniform", -1, 1)),
    # 1x1 with 16-channel chunks on 8x64 tiles (512 workgroups; 70 KB of
    # LDS, beyond the 64 KB a workgroup's static LDS took before), with the
    # 16-byte band loads and without
    synth.Workload("igemm_n_1x1_c16_tile8x64_vec", 16, 16, 64, 124, 64, 1, 1, 1, 0, 1, 1, 109,
                   ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_n_1x1_c16_tile8x64", 16, 16, 64, 126, 64, 1, 1, 1, 0, 1, 1, 110,
                   ("uniform", -1, 1), ("uniform", -1, 1)),
    # flattened-pixel tiles (1x1 and 3x3 outputs that fill under 80 % of the
    # row x column tiles): blocks of 32 pixels running over rows and images,
    # 4-byte and 16-byte bands (a column shift of 3 for padding 1), stride 1
    # and 2, partial channel chunks and 32-channel blocks, 5x5 images whose
    # tiles span six of them, and two blocks per wave on a grid of 1664 and
    # 2048 workgroups
    synth.Workload("igemm_flat_w28_cpg32", 3, 64, 28, 28, 64, 3, 3, 1, 1, 1, 2, 88, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_vec_p0_k40", 2, 16, 16, 16, 40, 3, 3, 1, 0, 1, 1, 89, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_vec_shift3", 2, 16, 20, 20, 40, 3, 3, 1, 1, 1, 1, 90, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_s2_c10", 3, 10, 15, 15, 40, 3, 3, 2, 1, 1, 1, 91, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_s2_1x1_k33", 2, 12, 13, 13, 33, 1, 1, 2, 0, 1, 1, 92, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_1x1_vec_c20", 4, 20, 12, 12, 64, 1, 1, 1, 0, 1, 1, 93, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_5x5_images", 9, 32, 5, 5, 32, 3, 3, 1, 1, 1, 1, 94, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_s2_vec", 3, 24, 28, 28, 32, 3, 3, 2, 1, 1, 1, 95, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_s2_vec_1x1", 2, 16, 24, 24, 32, 1, 1, 2, 0, 1, 1, 96, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_nb2_1x1", 16, 512, 14, 14, 1024, 1, 1, 1, 0, 1, 128, 97, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_nb2_vec_1x1", 16, 512, 16, 16, 1024, 1, 1, 1, 0, 1, 128, 98, ("uniform", -1, 1), ("uniform", -1, 1)),
    # geometries only the flattened-pixel kernel takes: 3x3 at dilation 2
    # (stride 1 and 2, "same" and narrower padding, 16-byte and 4-byte
    # bands, 32 channels per group), 5x5 and 7x7 at stride 2 (partial
    # chunks, 7x7's 98-weight chunks on 4-byte weight loads)
    synth.Workload("igemm_flat_dil2_vec", 2, 32, 20, 20, 40, 3, 3, 1, 2, 2, 1, 99, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_dil2_s2_vec", 3, 16, 32, 32, 32, 3, 3, 2, 2, 2, 1, 100, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_dil2_p1", 2, 8, 15, 15, 16, 3, 3, 1, 1, 2, 1, 101, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_dil2_cpg32", 2, 64, 14, 14, 64, 3, 3, 1, 2, 2, 2, 102, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_dil2_s2", 2, 8, 29, 29, 16, 3, 3, 2, 2, 2, 1, 108, ("uniform", -1, 1), ("uniform", -1, 1)),
    # dilation 3 and 4 at stride 1: 4-channel chunks, 16-byte and 4-byte
    # bands, a ragged last chunk, grouped, tiles over image boundaries
    synth.Workload("igemm_flat_dil3_vec", 2, 16, 20, 20, 40, 3, 3, 1, 3, 3, 1, 126, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_dil3_p1", 3, 10, 17, 19, 33, 3, 3, 1, 1, 3, 1, 127, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_dil4_vec", 2, 12, 24, 24, 32, 3, 3, 1, 4, 4, 1, 128, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_dil4_cpg32", 2, 64, 14, 14, 64, 3, 3, 1, 4, 4, 2, 129, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_dil4_p2", 4, 9, 13, 22, 16, 3, 3, 1, 2, 4, 1, 130, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_5x5_s2", 2, 12, 23, 23, 40, 5, 5, 2, 2, 1, 1, 103, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_5x5_s2_vec", 2, 16, 24, 24, 32, 5, 5, 2, 2, 1, 1, 104, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_7x7_s2", 2, 6, 29, 29, 64, 7, 7, 2, 3, 1, 1, 105, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_7x7_s2_vec", 1, 4, 40, 40, 32, 7, 7, 2, 3, 1, 1, 106, ("uniform", -1, 1), ("uniform", -1, 1)),
    # the tile kernel at 5x5 and 7x7 stride 2 (wide outputs, 64-column
    # tiles), and with fewer than 4 input channels: a 3-channel stem (7x7
    # stride 2), a 3-channel 3x3 stride-2 first layer, 2 and 3 channels at
    # stride 1 (partial chunks only)
    synth.Workload("igemm_s2_5x5_tile", 2, 8, 70, 140, 40, 5, 5, 2, 2, 1, 1, 111, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_s2_7x7_tile", 1, 6, 40, 150, 32, 7, 7, 2, 3, 1, 1, 112, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_s2_7x7_stem_c3", 2, 3, 64, 160, 64, 7, 7, 2, 3, 1, 1, 113, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_s2_3x3_c3", 2, 3, 40, 144, 32, 3, 3, 2, 1, 1, 1, 114, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_n_5x5_c2", 2, 2, 20, 70, 16, 5, 5, 1, 2, 1, 1, 115, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_n_7x7_c3", 1, 3, 18, 90, 40, 7, 7, 1, 3, 1, 1, 116, ("uniform", -1, 1), ("uniform", -1, 1)),
    # the factorized kernels of Inception-style blocks at stride 1, with
    # per-axis padding: 1x7 and 1x3 (4-byte bands: padding 3 and 1 across),
    # 7x1 and 3x1 (16-byte bands), a partial chunk and two output blocks
    synth.Workload("igemm_n_1x7_p03", 2, 12, 13, 40, 40, 1, 7, 1, (0, 3), 1, 1, 117, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_n_7x1_p30_vec", 2, 16, 30, 36, 32, 7, 1, 1, (3, 0), 1, 1, 118, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_n_1x3_p01", 3, 8, 9, 70, 16, 1, 3, 1, (0, 1), 1, 1, 119, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_n_3x1_p10_vec", 1, 20, 33, 64, 64, 3, 1, 1, (1, 0), 1, 1, 120, ("uniform", -1, 1), ("uniform", -1, 1)),
    # factorized kernels whose row x column tiles are at least 80 % full stay
    # on the tile kernel (the cases above take flattened-pixel tiles)
    synth.Workload("igemm_t_1x7_p03_full", 2, 12, 16, 64, 40, 1, 7, 1, (0, 3), 1, 1, 121, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_t_7x1_p30_full", 1, 16, 16, 32, 32, 7, 1, 1, (3, 0), 1, 1, 122, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_t_1x3_p01_full", 2, 9, 8, 30, 24, 1, 3, 1, (0, 1), 1, 1, 123, ("uniform", -1, 1), ("uniform", -1, 1)),
    # factorized kernels on flattened-pixel tiles with two blocks per wave
    # (grids of 2432 and 4096 workgroups): 16-row and 22-row bands, 4-byte loads
    synth.Workload("igemm_flat_nb2_1x7", 16, 512, 17, 17, 1024, 1, 7, 1, (0, 3), 1, 128, 124, ("uniform", -1, 1), ("uniform", -1, 1)),
    synth.Workload("igemm_flat_nb2_7x1_w30", 16, 512, 17, 30, 1024, 7, 1, 1, (3, 0), 1, 128, 125, ("uniform", -1, 1), ("uniform", -1, 1)),
]


@pytest.mark.parametrize("wl", EDGE, ids=lambda w: w.name)
def test_conv_edge_cases(wl):
    inp = synth.make_inputs(wl)
    y_ref, A = oracle_conv(wl, inp)
    y, algo = gpu_conv(wl, inp)
    _say("[parity] edge", wl.name, gc.ALGO_NAMES[algo])
    if wl.name.startswith(("igemm_s2", "igemm_n_", "igemm_t_", "igemm_flat")):
        assert algo == gc.ALGO_IGEMM, gc.ALGO_NAMES[algo]
    check_conv(y, y_ref, A, wl.name)
    # an output pointer that is only 4-byte aligned takes the scalar stores
    y1, _ = gpu_conv(wl, inp, y_offset=1)
    check_conv(y1, y_ref, A, wl.name + " misaligned y")


WIDE = [wl for wl in EDGE if wl.name.startswith(("rows_cpg", "band_cpg", "mfma16"))]


@pytest.mark.parametrize("wl", WIDE, ids=lambda w: w.name)
def test_wide_groups_register_kernel(wl):
    """8 and 16 channels per group on the register kernel: integer inputs
    bit-exact, and a bias."""
    assert gc.conv_desc_get_algo(_desc(wl)) == gc.ALGO_GROUPED3X3
    wi = wl.with_(x_dist=("int", -2, 2), w_dist=("int", -2, 2), seed=wl.seed + 500)
    inp = synth.make_inputs(wi)
    y, _ = gpu_conv(wi, inp)
    y_ref, _ = oracle_conv(wi, inp)
    assert np.array_equal(y.astype(np.float64), y_ref), wl.name
    inp = synth.make_inputs(wl)
    bias = synth.normal((wl.K,), 0.5, wl.seed, 7)
    y, _ = gpu_conv(wl, inp, bias=bias)
    y_ref, A = oracle_conv(wl, inp, bias)
    check_conv(y, y_ref, A, wl.name + " bias")


def _fast_path_cases(n, seed):
    """Random shapes aimed at the register, band, general-geometry and
    matrix-core paths: channels per group in {1, 2, 4, 8, 16}, output
    channels per group a multiple of 4 (or equal to the input), the five
    (K, stride, dilation) geometries with "same" padding and 3x3 stride 1."""
    rng = np.random.default_rng(seed)
    geoms = [(3, 1, 1)] * 5 + [(5, 1, 1), (7, 1, 1), (3, 2, 1), (5, 2, 1), (3, 1, 2)]
    out = []
    while len(out) < n:
        cin = int(rng.choice([1, 2, 4, 8, 16]))
        R, st, dil = geoms[int(rng.integers(len(geoms)))]
        if (R, st, dil) != (3, 1, 1) and cin > 4:
            continue
        cout = cin if cin == 1 and (R, st, dil) != (3, 1, 1) else int(rng.choice([cin, 4, 8, 16]))
        if (R, st, dil) == (3, 1, 1) and cin > 4 and cout > 16:
            continue
        groups = int(rng.integers(2, 5))
        wo = 4 * int(rng.integers(1, 20)) if rng.random() < 0.8 else int(rng.integers(3, 70))
        W = st * wo
        H = int(rng.integers(1, 30))
        out.append(synth.Workload("fast%d_c%d_k%d_r%ds%dd%d" % (len(out), cin, cout, R, st, dil), int(rng.integers(1, 4)),
                                  groups * cin, H, W, groups * cout, R, R, st, dil * (R // 2), dil, groups,
                                  4000 + len(out), ("uniform", -1.0, 1.0), ("uniform", -0.5, 0.5)))
    return out


@pytest.mark.parametrize("wl", _fast_path_cases(30, 23), ids=lambda w: w.name)
def test_fast_path_fuzz(wl):
    inp = synth.make_inputs(wl)
    y_ref, A = oracle_conv(wl, inp)
    y, algo = gpu_conv(wl, inp)
    check_conv(y, y_ref, A, "%s %s" % (wl.name, gc.ALGO_NAMES[algo]))


def _wide_path_cases(n, seed):
    """Random shapes aimed at the depthwise channel multiplier, ragged and
    packed small planes (any output width, odd stride-2 inputs, 3x3 stride 1
    forced onto the depthwise kernel), and the implicit GEMM at stride 2 and
    on narrow or small grids (1x1 and 3x3, dense or grouped)."""
    rng = np.random.default_rng(seed)
    geoms = [(3, 1, 1), (5, 1, 1), (7, 1, 1), (3, 2, 1), (5, 2, 1), (3, 1, 2)]
    out = []
    while len(out) < n:
        N = int(rng.integers(1, 4))
        H = int(rng.integers(1, 24))
        if rng.random() < 0.5:
            # one input channel per group, 1-8 outputs per group, any width
            R, st, dil = geoms[int(rng.integers(len(geoms)))]
            groups = int(rng.integers(1, 9))
            cout = int(rng.integers(1, 9))
            W = int(rng.integers(1, 80))
            pad = dil * (R // 2)
            if (W + 2 * pad - dil * (R - 1) - 1) // st + 1 < 1 or (H + 2 * pad - dil * (R - 1) - 1) // st + 1 < 1:
                continue
            # 3x3 stride 1 runs on the depthwise kernel only on small planes
            # (at most 32 lanes: 4-column groups x 2-row strips)
            if (R, st, dil) == (3, 1, 1) and -(-W // 4) * -(-H // 2) > 32:
                continue
            algo = gc.ALGO_DEPTHWISE
            out.append((synth.Workload("wide%d_dw_m%d_r%ds%dd%d_w%d" % (len(out), cout, R, st, dil, W), N, groups, H, W,
                                       groups * cout, R, R, st, pad, dil, groups, 5000 + len(out),
                                       ("uniform", -1.0, 1.0), ("uniform", -0.5, 0.5)), algo))
        else:
            # implicit GEMM: 1x1 or 3x3, stride 1 or 2, dense or grouped
            R = int(rng.choice([1, 3]))
            st = int(rng.choice([1, 2]))
            pad = int(rng.integers(0, R // 2 + 1))
            groups = int(rng.choice([1, 1, 2]))
            cin = int(rng.integers(4, 41))
            cout = int(rng.integers(8, 73))
            W = int(rng.integers(R, 140))
            H = max(H, R)
            out.append((synth.Workload("wide%d_ig_c%d_k%d_r%ds%dp%d_w%d" % (len(out), cin, cout, R, st, pad, W), N,
                                       groups * cin, H, W, groups * cout, R, R, st, pad, 1, groups, 5000 + len(out),
                                       ("uniform", -1.0, 1.0), ("uniform", -0.5, 0.5)), gc.ALGO_IGEMM))
    return out


@pytest.mark.parametrize("case", _wide_path_cases(30, 29), ids=lambda c: c[0].name)
def test_wide_path_fuzz(case):
    wl, algo = case
    inp = synth.make_inputs(wl)
    y_ref, A = oracle_conv(wl, inp)
    _say("[parity] fuzz", wl.name, gc.ALGO_NAMES[algo])
    y, used = gpu_conv(wl, inp, algo=algo)
    assert used == algo
    check_conv(y, y_ref, A, "%s %s" % (wl.name, gc.ALGO_NAMES[used]))


def test_repeatable_bitwise():
    for name in ("c4_dense_5x9", "c3a_grouped_g64"):
        wl = SMALL[name]
        inp = synth.make_inputs(wl)
        a, _ = gpu_conv(wl, inp)
        b, _ = gpu_conv(wl, inp)
        assert np.array_equal(a, b), name
    wl = SMALL["c5_fused_gn"]
    inp = synth.make_inputs(wl)
    assert np.array_equal(gpu_fused(wl, inp), gpu_fused(wl, inp))
    wl = W["c5_fused_gn"].with_(N=8, H=130, W=132)
    inp = synth.make_inputs(wl)
    assert np.array_equal(gpu_fused(wl, inp, variant=gc.FUSED_ONEPASS), gpu_fused(wl, inp, variant=gc.FUSED_ONEPASS))


def test_graph_capture_replays_match_eager():
    """Both entry points captured in a HIP graph; every replay equals the eager run."""
    wl = SMALL["c4_dense_5x9"]
    inp = synth.make_inputs(wl)
    d = _desc(wl)
    ho, wo = gc.conv_desc_get_output_dims(d)
    x, w = _dev(inp["x"]), _dev(inp["w"])
    y_eager = torch.empty((wl.N, wl.K, ho, wo), device="cuda")
    gc.conv_fwd(d, x, w, None, y_eager)

    wf = SMALL["c5_fused_gn"]
    fi = synth.make_inputs(wf)
    df = _desc(wf)
    hf, wfo = gc.conv_desc_get_output_dims(df)
    fx, fw, fb, fs = _dev(fi["x"]), _dev(fi["w"]), _dev(fi["bias"]), _dev(fi["scale"])
    ws = torch.empty(gc.conv_fused_gn_workspace_size(df, wf.gn_groups), dtype=torch.uint8, device="cuda")
    f_eager = torch.empty((wf.N, wf.K, hf, wfo), device="cuda")
    gc.conv_fused_gn_fwd(df, fx, fw, fb, fs, None, None, wf.gn_groups, wf.eps, f_eager, ws)
    torch.cuda.synchronize()

    y_g = torch.zeros_like(y_eager)
    f_g = torch.zeros_like(f_eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            gc.conv_fwd(d, x, w, None, y_g)
            gc.conv_fused_gn_fwd(df, fx, fw, fb, fs, None, None, wf.gn_groups, wf.eps, f_g, ws)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        y_g.fill_(float("nan"))
        f_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_eager), rep
        assert torch.equal(f_g, f_eager), rep
        # unrelated eager work between replays
        y_eager.add_(0.0)
        torch.cuda.synchronize()


def test_graph_capture_of_store_variant_slices():
    """The store variant runs its conv and in-place normalize over batch
    slices (16 full-size images: slices of 15 and 1): captured in a HIP
    graph, every replay equals the eager run, and the eager run matches the
    oracle on the images at the slice edges."""
    wl = W["c5_fused_gn"].with_(N=16)
    inp = synth.make_inputs(wl)
    d = _desc(wl)
    gc.conv_desc_set_fused_variant(d, gc.FUSED_STORE)
    ho, wo = gc.conv_desc_get_output_dims(d)
    t = {k: _dev(v) for k, v in inp.items()}
    ws = torch.empty(gc.conv_fused_gn_workspace_size(d, wl.gn_groups), dtype=torch.uint8, device="cuda")
    f_eager = torch.full((wl.N, wl.K, ho, wo), float("nan"), device="cuda")
    gc.conv_fused_gn_fwd(d, t["x"], t["w"], t["bias"], t["scale"], t["gamma"], t["beta"], wl.gn_groups, wl.eps,
                         f_eager, ws)
    torch.cuda.synchronize()
    out = f_eager.cpu().numpy()
    for n in (0, 14, 15):
        sl = dict(inp)
        sl["x"] = inp["x"][n:n + 1]
        check_gn(out[n:n + 1], oracle_fused(wl.with_(N=1), sl), "store variant slices, image %d" % n)
    f_g = torch.zeros_like(f_eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            gc.conv_fused_gn_fwd(d, t["x"], t["w"], t["bias"], t["scale"], t["gamma"], t["beta"], wl.gn_groups,
                                 wl.eps, f_g, ws)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        f_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(f_g, f_eager), rep
        f_eager.add_(0.0)  # unrelated eager work between replays
        torch.cuda.synchronize()


def test_graph_capture_of_onepass_variant():
    """The one-pass variant (counter clear, conv pass, trailing pass) captured
    twice in one HIP graph: every replay equals the eager run, so the counters
    start from zero on every replay."""
    wl = W["c5_fused_gn"].with_(N=8, H=130, W=132)
    inp = synth.make_inputs(wl)
    d = _desc(wl)
    gc.conv_desc_set_fused_variant(d, gc.FUSED_ONEPASS)
    ho, wo = gc.conv_desc_get_output_dims(d)
    t = {k: _dev(v) for k, v in inp.items()}
    ws = torch.empty(gc.conv_fused_gn_workspace_size(d, wl.gn_groups), dtype=torch.uint8, device="cuda")
    f_eager = torch.full((wl.N, wl.K, ho, wo), float("nan"), device="cuda")
    gc.conv_fused_gn_fwd(d, t["x"], t["w"], t["bias"], t["scale"], t["gamma"], t["beta"], wl.gn_groups, wl.eps,
                         f_eager, ws)
    torch.cuda.synchronize()
    check_gn(f_eager.cpu().numpy()[:2], oracle_fused(wl.with_(N=2), dict(inp, x=inp["x"][:2])), "one-pass eager")
    f_g = torch.zeros_like(f_eager)
    f_g2 = torch.zeros_like(f_eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for out in (f_g, f_g2):
                gc.conv_fused_gn_fwd(d, t["x"], t["w"], t["bias"], t["scale"], t["gamma"], t["beta"], wl.gn_groups,
                                     wl.eps, out, ws)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        f_g.fill_(float("nan"))
        f_g2.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(f_g, f_eager), rep
        assert torch.equal(f_g2, f_eager), rep
        f_eager.add_(0.0)  # unrelated eager work between replays
        torch.cuda.synchronize()


def test_graph_capture_of_every_kernel_family():
    """One conv per kernel family captured in a single HIP graph (grouped
    register and band kernels, matrix-core 16/16 groups at 64- and 32-column
    segments, depthwise aligned, ragged and packed, implicit GEMM at stride 1
    and 2 and on flattened pixels (narrow, dilated, 7x7 stride 2), the direct
    kernel); every replay equals the eager runs."""
    shapes = [  # (N, C, H, W, K, R, stride, pad, dil, groups)
        (2, 16, 20, 32, 16, 3, 1, 1, 1, 4),       # grouped register kernel
        (2, 16, 13, 30, 16, 3, 1, 1, 1, 4),       # grouped band kernel (W % 4 != 0)
        (2, 64, 24, 40, 64, 3, 1, 1, 1, 4),       # 16 in / 16 out: matrix cores
        (2, 8, 20, 40, 8, 5, 1, 2, 1, 8),         # depthwise, aligned rows
        (2, 8, 21, 21, 16, 3, 2, 1, 1, 8),        # depthwise multiplier, ragged stride-2 rows
        (16, 1024, 7, 7, 1024, 3, 1, 1, 1, 1024), # depthwise 3x3 small planes, packed
        (2, 8, 20, 70, 40, 3, 1, 1, 1, 1),        # implicit GEMM, stride 1
        (2, 8, 19, 70, 40, 3, 2, 1, 1, 1),        # implicit GEMM, stride 2
        (1, 64, 14, 14, 64, 3, 1, 1, 1, 2),       # implicit GEMM, flattened pixels (narrow output)
        (2, 16, 20, 20, 32, 3, 1, 2, 2, 1),       # implicit GEMM, flattened, dilation 2
        (2, 6, 29, 29, 64, 7, 2, 3, 1, 1),        # implicit GEMM, flattened, 7x7 stride 2
        (2, 64, 16, 28, 64, 3, 1, 1, 1, 4),       # 16 in / 16 out, 32-column segments
        (2, 6, 11, 13, 9, 3, 2, 1, 2, 3),         # direct kernel
    ]
    runs = []
    for i, (N, C, H, W, K, R, st, pad, dil, G) in enumerate(shapes):
        wl = synth.Workload("graph%d" % i, N, C, H, W, K, R, R, st, pad, dil, G, 6000 + i,
                            ("uniform", -1.0, 1.0), ("uniform", -0.5, 0.5))
        inp = synth.make_inputs(wl)
        d = _desc(wl)
        ho, wo = gc.conv_desc_get_output_dims(d)
        x, w = _dev(inp["x"]), _dev(inp["w"])
        y_eager = torch.empty((N, K, ho, wo), device="cuda")
        gc.conv_fwd(d, x, w, None, y_eager)
        runs.append((d, x, w, y_eager, torch.zeros_like(y_eager), gc.ALGO_NAMES[gc.conv_desc_get_algo(d)]))
    torch.cuda.synchronize()
    assert {r[5] for r in runs} == {"grouped3x3", "depthwise", "igemm", "direct"}
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for d, x, w, _, y_g, _ in runs:
                gc.conv_fwd(d, x, w, None, y_g)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for r in runs:
            r[4].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, r in enumerate(runs):
            assert torch.equal(r[4], r[3]), (rep, i, r[5])
        runs[0][3].add_(0.0)  # unrelated eager work between replays
        torch.cuda.synchronize()


def test_time_graph_helper_outputs_match_eager():
    """gconv_time_graph: positive per-launch times, and the rotated outputs
    equal eager calls on the same buffers (conv and fused entry points)."""
    wl = SMALL["c3a_grouped_g64"]
    inp = synth.make_inputs(wl)
    d = _desc(wl)
    ho, wo = gc.conv_desc_get_output_dims(d)
    w = _dev(inp["w"])
    xs = [_dev(inp["x"]), _dev(inp["x"] * 0.5 - 0.25)]
    ys = [torch.full((wl.N, wl.K, ho, wo), float("nan"), device="cuda") for _ in xs]
    ref = []
    for x in xs:
        r = torch.empty((wl.N, wl.K, ho, wo), device="cuda")
        gc.conv_fwd(d, x, w, None, r)
        ref.append(r)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    ms = gc.gconv_time_graph(d, xs, ys, w, None, launches=3, replays=5, stream=s)
    torch.cuda.synchronize()
    assert len(ms) == 5 and all(m > 0 for m in ms), ms
    for a, b in zip(ys, ref):
        assert torch.equal(a, b)

    wf = SMALL["c5_fused_gn"]
    fi = synth.make_inputs(wf)
    df = _desc(wf)
    hf, wfo = gc.conv_desc_get_output_dims(df)
    fx, fw, fb, fs = _dev(fi["x"]), _dev(fi["w"]), _dev(fi["bias"]), _dev(fi["scale"])
    ws = torch.empty(gc.conv_fused_gn_workspace_size(df, wf.gn_groups), dtype=torch.uint8, device="cuda")
    f_eager = torch.empty((wf.N, wf.K, hf, wfo), device="cuda")
    gc.conv_fused_gn_fwd(df, fx, fw, fb, fs, None, None, wf.gn_groups, wf.eps, f_eager, ws)
    torch.cuda.synchronize()
    f_g = torch.full_like(f_eager, float("nan"))
    ms = gc.gconv_time_graph(df, [fx], [f_g], fw, fb, launches=2, replays=3, stream=s,
                             fused=dict(scale=fs, gamma=None, beta=None, gn_groups=wf.gn_groups, eps=wf.eps,
                                        workspace=ws))
    torch.cuda.synchronize()
    assert len(ms) == 3 and all(m > 0 for m in ms), ms
    assert torch.equal(f_g, f_eager)


# ---- per-axis stride, padding and dilation

PER_AXIS = [
    # (N, C, H, W, K, R, S, stride, pad, dil, groups)
    (2, 8, 19, 23, 8, 3, 3, (1, 2), (1, 1), (1, 1), 8),     # depthwise, stride along W only
    (1, 6, 17, 15, 9, 3, 5, (2, 1), (1, 2), (1, 2), 3),     # grouped, everything per axis
    (2, 16, 21, 30, 32, 5, 5, (1, 1), (0, 2), (1, 1), 1),   # implicit GEMM, padding per axis
    (1, 8, 14, 66, 32, 3, 3, (1, 1), (2, 1), (1, 1), 1),    # resident-weight MFMA, padding per axis
    (1, 12, 25, 11, 24, 5, 3, (2, 2), (2, 1), (2, 1), 4),   # dilation per axis
    (3, 4, 9, 40, 8, 1, 7, (1, 3), (0, 3), (1, 1), 2),      # 1x7, stride 3 along W
]


@pytest.mark.parametrize("geom", PER_AXIS)
def test_per_axis_conv_matches_oracle(geom):
    N, C, H, W, K, R, S, stride, pad, dil, groups = geom
    x = synth.uniform((N, C, H, W), -1, 1, 91, 0)
    w = synth.uniform((K, C // groups, R, S), -1, 1, 91, 1)
    b = synth.uniform((K,), -1, 1, 91, 2)
    y_ref, A = oracle.conv2d(x, w, b, stride, pad, dil, groups)
    d = gc.conv_desc_create_2d(N, C, H, W, K, R, S, stride, pad, dil, groups)
    ho, wo = gc.conv_desc_get_output_dims(d)
    assert (ho, wo) == y_ref.shape[2:]
    for algo in (gc.ALGO_AUTO, gc.ALGO_DIRECT):
        gc.conv_desc_set_algo(d, algo)
        y = torch.full((N, K, ho, wo), float("nan"), device="cuda")
        gc.conv_fwd(d, _dev(x), _dev(w), _dev(b), y)
        torch.cuda.synchronize()
        _say("[parity] per-axis", geom, gc.ALGO_NAMES[gc.conv_desc_get_algo(d)])
        check_conv(y.cpu().numpy(), y_ref, A, "per-axis %s %s" % (geom, gc.ALGO_NAMES[algo]))


def test_per_axis_fused_matches_oracle():
    N, C, H, W, K, R, S = 2, 8, 15, 33, 32, 3, 3
    stride, pad, dil = (1, 1), (2, 1), (1, 1)
    x = synth.uniform((N, C, H, W), 0, 1, 92, 0)
    w = synth.uniform((K, C, R, S), -0.3, 0.3, 92, 1)
    bias = synth.normal((K,), 0.1, 92, 2)
    scale = synth.normal((K,), 0.1, 92, 3)
    ref = oracle.fused_gn(x, w, bias, scale, None, None, 8, 1e-5, stride, pad, dil, 1)
    d = gc.conv_desc_create_2d(N, C, H, W, K, R, S, stride, pad, dil, 1)
    ho, wo = gc.conv_desc_get_output_dims(d)
    for variant in (gc.FUSED_STORE, gc.FUSED_RECOMPUTE):
        gc.conv_desc_set_fused_variant(d, variant)
        ws = torch.empty(gc.conv_fused_gn_workspace_size(d, 8), dtype=torch.uint8, device="cuda")
        y = torch.full((N, K, ho, wo), float("nan"), device="cuda")
        gc.conv_fused_gn_fwd(d, _dev(x), _dev(w), _dev(bias), _dev(scale), None, None, 8, 1e-5, y, ws)
        torch.cuda.synchronize()
        err = np.abs(y.cpu().numpy() - ref).max()
        assert err <= GN_ATOL, (variant, err)


def test_probe_peaks_are_plausible():
    """The measured FP32 MFMA and FMA peaks are positive and below the
    datasheet's 157.3 TFLOP/s (FP32 matrix, and FP32 vector with packed
    instructions: the ceiling for any FP32 vector code) with a little margin.
    Non-packed FMA chains measure above half of it on gfx950."""
    sink = torch.zeros(4, device="cuda")
    mfma, fma = gc.gconv_probe_peaks(sink)
    _say("[parity] measured peaks: MFMA %.1f TFLOP/s, FMA %.1f TFLOP/s" % (mfma, fma))
    assert 20.0 < mfma < 170.0, mfma
    assert 10.0 < fma < 165.0, fma
    assert float(sink[0]) == 0.0


def test_vector_and_copy_probes_are_plausible():
    """The measured FP64 FMA rate stays at or below its datasheet peak of one
    FMA per lane per clock (78.6 TFLOP/s) with a little margin; the FP32 FMA
    rate stays below the FP32 vector datasheet peak (157.3 TFLOP/s); the
    library's copy moves the buffer exactly and reports a rate below the
    8 TB/s HBM peak (read + write over 2 x 256 MiB, beyond the last-level
    cache)."""
    sink = torch.zeros(4, device="cuda")
    f32, f64 = gc.gconv_probe_vector_peaks(sink)
    _say("[parity] measured vector peaks: FP32 FMA %.1f TFLOP/s, FP64 FMA %.1f TFLOP/s" % (f32, f64))
    assert 10.0 < f64 < 82.0, f64
    assert 10.0 < f32 < 165.0, f32
    assert float(sink[0]) == 0.0
    src = torch.empty(64 << 20, device="cuda").uniform_()
    dst = torch.zeros_like(src)
    gbs = gc.gconv_probe_copy(dst, src)
    torch.cuda.synchronize()
    _say("[parity] library copy: %.1f GB/s" % gbs)
    assert torch.equal(dst, src)
    assert 500.0 < gbs < 8400.0, gbs


def test_grids_beyond_65535_planes_or_images():
    """More than 65535 output channels or images: the direct kernel and the
    in-place GroupNorm normalize run one-dimensional grids, and the band
    kernel hands such batches to the direct kernel, instead of refusing the
    launch."""
    cases = [  # (N, C, H, W, K, R, pad, groups)
        (1, 1, 1, 1, 70000, 1, 0, 1),     # 70000 output planes, direct kernel
        (70000, 1, 2, 2, 1, 3, 1, 1),     # 70000 images, grouped 3x3 band path -> direct
        (66000, 2, 3, 5, 2, 3, 1, 2),     # the same, two groups
    ]
    for i, (N, C, H, W, K, R, pad, G) in enumerate(cases):
        wl = synth.Workload("grid%d" % i, N, C, H, W, K, R, R, 1, pad, 1, G, 7000 + i, ("uniform", -1.0, 1.0),
                            ("uniform", -0.5, 0.5))
        _say("[parity] grid limits", wl)
        inp = synth.make_inputs(wl)
        y, _ = gpu_conv(wl, inp)
        y_ref, A = oracle_conv(wl, inp)
        check_conv(y, y_ref, A, wl.name)
    # the fused chain on 70000 images: stage A on the direct kernel, then the
    # normalize over 70000 (image, group) pairs
    wl = synth.WORKLOADS["c5_fused_gn"].with_(N=70000, C=4, K=4, H=2, W=2, pad=1, gn_groups=1)
    _say("[parity] grid limits, fused", wl)
    inp = synth.make_inputs(wl)
    check_gn(gpu_fused(wl, inp), oracle_fused(wl, inp), "fused 70000 images")
