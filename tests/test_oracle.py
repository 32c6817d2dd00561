"""Pins for the CPU oracle, independent of the oracle's own code.

Each test checks the oracle against something fixed from outside it: the
pages' printed geometry (tests/golden), closed forms (delta kernel, all-ones
tap counts, GroupNorm moments), textbook/library routines (scipy 2-D
correlation, an explicit im2col x matmul, torch float64 conv2d and
group_norm on the CPU, scipy's logistic function) and a scatter-form brute
force on tiny integer inputs.  A dropped term, a wrong sign or index, a
transposed weight or a wrong group mapping fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal
import scipy.special
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_geometry.json")


def _torch_conv(x, w, bias, stride, pad, dil, groups):
    xt = torch.from_numpy(np.asarray(x, np.float64))
    wt = torch.from_numpy(np.asarray(w, np.float64))
    bt = None if bias is None else torch.from_numpy(np.asarray(bias, np.float64))
    return F.conv2d(xt, wt, bt, stride, pad, dil, groups).numpy()


def _rand(shape, seed, slot=0, lo=-1.0, hi=1.0):
    return synth.uniform(shape, lo, hi, seed, slot)


# ---------------------------------------------------------------- golden


def test_golden_page_geometry():
    cases = json.load(open(GOLDEN))["cases"]
    assert cases
    for c in cases:
        assert oracle.out_dim(c["H"], c["R"], c["stride"], c["pad"], c["dil"]) == c["Ho"], c["cite"]
        assert oracle.out_dim(c["W"], c["S"], c["stride"], c["pad"], c["dil"]) == c["Wo"], c["cite"]
        assert c["K"] * (c["C"] // c["groups"]) * c["R"] * c["S"] == c["weight_count"]
        # all-ones input and weights: every output of a padding-free window
        # sums exactly macs_per_output ones.
        x = np.ones((1, c["C"], c["H"], c["W"]), np.float32)
        w = np.ones((1, c["C"] // c["groups"], c["R"], c["S"]), np.float32)
        rng = np.random.default_rng(7)
        idx = np.concatenate([[0, c["Ho"] * c["Wo"] - 1], rng.integers(0, c["Ho"] * c["Wo"], 30)])
        y, A = oracle.conv2d_points(x, w, idx, None, c["stride"], c["pad"], c["dil"], c["groups"])
        assert np.all(y == c["macs_per_output"]), c["cite"]
        assert np.all(A == c["macs_per_output"])


# ---------------------------------------------------------------- closed forms

DELTA_CASES = [
    # (N, C, H, W, R, dil, groups)
    (2, 4, 9, 11, 3, 1, 1),
    (1, 6, 7, 5, 3, 2, 3),
    (2, 8, 12, 10, 5, 1, 8),
    (1, 4, 6, 13, 1, 1, 2),
    (1, 3, 10, 10, 5, 2, 1),
]


@pytest.mark.parametrize("N,C,H,W,R,dil,groups", DELTA_CASES)
def test_delta_kernel_reproduces_input(N, C, H, W, R, dil, groups):
    x = _rand((N, C, H, W), 11)
    cin = C // groups
    w = np.zeros((C, cin, R, R), np.float32)
    for k in range(C):
        w[k, k % cin, (R - 1) // 2, (R - 1) // 2] = 1.0
    pad = dil * (R - 1) // 2
    y, _ = oracle.conv2d(x, w, None, 1, pad, dil, groups)
    assert y.shape == x.shape
    assert np.array_equal(y, x.astype(np.float64))


def _count_taps(o, k, stride, pad, dil, n):
    # number of taps t in [0, k) with 0 <= o*stride - pad + t*dil <= n-1,
    # from the two inequalities solved for t
    lo = max(0, -((o * stride - pad) // dil))  # ceil((pad - o*stride)/dil)
    hi = min(k - 1, (n - 1 + pad - o * stride) // dil)
    return max(0, hi - lo + 1)


ONES_CASES = [
    # (C, H, W, K, R, S, stride, pad, dil, groups)
    (4, 16, 16, 8, 3, 3, 1, 1, 1, 2),
    (3, 11, 9, 3, 3, 3, 2, 1, 1, 3),
    (2, 13, 17, 4, 5, 9, 1, 0, 1, 1),
    (6, 10, 12, 6, 3, 5, 3, 2, 2, 2),
    (2, 7, 7, 2, 4, 2, 2, 3, 2, 1),
    (8, 9, 9, 8, 7, 7, 1, 3, 1, 8),
]


@pytest.mark.parametrize("C,H,W,K,R,S,stride,pad,dil,groups", ONES_CASES)
def test_all_ones_gives_tap_counts(C, H, W, K, R, S, stride, pad, dil, groups):
    x = np.ones((2, C, H, W), np.float32)
    w = np.ones((K, C // groups, R, S), np.float32)
    y, A = oracle.conv2d(x, w, None, stride, pad, dil, groups)
    Ho, Wo = y.shape[2:]
    cr = np.array([_count_taps(o, R, stride, pad, dil, H) for o in range(Ho)])
    cs = np.array([_count_taps(o, S, stride, pad, dil, W) for o in range(Wo)])
    expect = (C // groups) * cr[:, None] * cs[None, :]
    assert np.array_equal(y, np.broadcast_to(expect, y.shape))
    assert np.array_equal(A, y)
    if (stride, pad, dil, R) == (1, 1, 1, 3):
        # interior 9*cpg, edges 6*cpg, corners 4*cpg
        cpg = C // groups
        assert y[0, 0, 1, 1] == 9 * cpg and y[0, 0, 0, 1] == 6 * cpg and y[0, 0, 0, 0] == 4 * cpg


# ---------------------------------------------------------------- library routines


@pytest.mark.parametrize("pad", [0, 1, 2])
def test_depthwise_equals_per_channel_correlate2d(pad):
    N, C, H, W, R, S = 2, 5, 12, 9, 3, 3
    x = _rand((N, C, H, W), 21)
    w = _rand((C, 1, R, S), 21, 1)
    y, _ = oracle.conv2d(x, w, None, 1, pad, 1, C)
    for n in range(N):
        for c in range(C):
            ref = scipy.signal.correlate2d(np.pad(x[n, c].astype(np.float64), pad),
                                           w[c, 0].astype(np.float64), mode="valid")
            np.testing.assert_allclose(y[n, c], ref, rtol=1e-12, atol=1e-14)


def _im2col_matmul(x, w, stride, pad, dil):
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    xp = np.pad(x.astype(np.float64), ((0, 0), (0, 0), (pad, pad), (pad, pad)))
    Ho = (H + 2 * pad - dil * (R - 1) - 1) // stride + 1
    Wo = (W + 2 * pad - dil * (S - 1) - 1) // stride + 1
    cols = np.empty((N, C * R * S, Ho * Wo))
    row = 0
    for c in range(C):
        for r in range(R):
            for s in range(S):
                patch = xp[:, c, r * dil: r * dil + stride * (Ho - 1) + 1: stride,
                           s * dil: s * dil + stride * (Wo - 1) + 1: stride]
                cols[:, row, :] = patch.reshape(N, -1)
                row += 1
    out = np.einsum("kq,nqp->nkp", w.reshape(K, -1).astype(np.float64), cols)
    return out.reshape(N, K, Ho, Wo)


@pytest.mark.parametrize("stride,pad,dil,R,S", [(1, 0, 1, 5, 9), (2, 1, 1, 3, 3), (1, 2, 2, 3, 5), (3, 0, 1, 2, 4)])
def test_groups1_equals_im2col_matmul(stride, pad, dil, R, S):
    x = _rand((2, 3, 17, 19), 31)
    w = _rand((4, 3, R, S), 31, 1)
    y, _ = oracle.conv2d(x, w, None, stride, pad, dil, 1)
    np.testing.assert_allclose(y, _im2col_matmul(x, w, stride, pad, dil), rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("groups,cin,cout", [(2, 4, 4), (3, 1, 2), (4, 2, 1), (2, 3, 5)])
def test_grouped_equals_concatenated_dense_convs(groups, cin, cout):
    C, K = groups * cin, groups * cout
    x = _rand((2, C, 10, 11), 41)
    w = _rand((K, cin, 3, 3), 41, 1)
    y, _ = oracle.conv2d(x, w, None, 1, 1, 1, groups)
    parts = [oracle.conv2d(x[:, g * cin:(g + 1) * cin], w[g * cout:(g + 1) * cout], None, 1, 1, 1, 1)[0]
             for g in range(groups)]
    assert np.array_equal(y, np.concatenate(parts, axis=1))


def _random_geometries(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        groups = int(rng.choice([1, 2, 3, 4]))
        cin, cout = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        R, S = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        stride, pad, dil = int(rng.integers(1, 4)), int(rng.integers(0, 3)), int(rng.integers(1, 3))
        H, W = int(rng.integers(1, 14)), int(rng.integers(1, 14))
        if H + 2 * pad - dil * (R - 1) - 1 < 0 or W + 2 * pad - dil * (S - 1) - 1 < 0:
            continue
        out.append((2, groups * cin, H, W, groups * cout, R, S, stride, pad, dil, groups))
    return out


@pytest.mark.parametrize("geom", _random_geometries(24, 5))
def test_matches_torch_conv2d_float64(geom):
    N, C, H, W, K, R, S, stride, pad, dil, groups = geom
    x = _rand((N, C, H, W), 51)
    w = _rand((K, C // groups, R, S), 51, 1)
    b = _rand((K,), 51, 2)
    y, A = oracle.conv2d(x, w, b, stride, pad, dil, groups)
    np.testing.assert_allclose(y, _torch_conv(x, w, b, stride, pad, dil, groups), rtol=1e-12, atol=1e-13)
    # the bound is the same correlation of the absolute values (plus |bias|)
    np.testing.assert_allclose(A, _torch_conv(np.abs(x), np.abs(w), np.abs(b), stride, pad, dil, groups),
                               rtol=1e-12, atol=1e-13)
    assert np.all(A + 1e-12 >= np.abs(y))


def _scatter_conv(x, w, stride, pad, dil, groups):
    """Loop over input pixels and taps, adding each product into the output it feeds."""
    N, C, H, W = x.shape
    K, cin, R, S = w.shape
    cout = K // groups
    Ho = oracle.out_dim(H, R, stride, pad, dil)
    Wo = oracle.out_dim(W, S, stride, pad, dil)
    y = np.zeros((N, K, Ho, Wo))
    for n in range(N):
        for ic in range(C):
            g = ic // cin
            for ih in range(H):
                for iw in range(W):
                    for r in range(R):
                        num_h = ih + pad - r * dil
                        if num_h % stride or not (0 <= num_h // stride < Ho):
                            continue
                        for s in range(S):
                            num_w = iw + pad - s * dil
                            if num_w % stride or not (0 <= num_w // stride < Wo):
                                continue
                            for kl in range(cout):
                                k = g * cout + kl
                                y[n, k, num_h // stride, num_w // stride] += x[n, ic, ih, iw] * w[k, ic - g * cin, r, s]
    return y


@pytest.mark.parametrize("geom", [(1, 2, 5, 6, 2, 3, 3, 1, 1, 1, 1), (2, 4, 7, 7, 4, 3, 5, 2, 2, 1, 2),
                                  (1, 4, 9, 7, 8, 3, 2, 1, 1, 2, 4), (2, 3, 7, 5, 3, 2, 4, 3, 0, 1, 3),
                                  (1, 2, 4, 4, 2, 1, 1, 2, 1, 1, 2)])
def test_scatter_bruteforce_exact_on_integers(geom):
    N, C, H, W, K, R, S, stride, pad, dil, groups = geom
    x = synth.integers((N, C, H, W), -2, 2, 61, 0)
    w = synth.integers((K, C // groups, R, S), -2, 2, 61, 1)
    y, _ = oracle.conv2d(x, w, None, stride, pad, dil, groups)
    assert np.array_equal(y, _scatter_conv(x, w, stride, pad, dil, groups))


def test_points_equal_full_output():
    x = _rand((2, 6, 20, 23), 71)
    w = _rand((4, 3, 5, 9), 71, 1)
    y, A = oracle.conv2d(x, w, None, 1, 2, 1, 2)
    idx = np.random.default_rng(1).integers(0, y.size, 200)
    yp, Ap = oracle.conv2d_points(x, w, idx, None, 1, 2, 1, 2)
    assert np.array_equal(yp, y.ravel()[idx]) and np.array_equal(Ap, A.ravel()[idx])


def test_rejects_bad_geometry():
    x = np.zeros((1, 4, 5, 5), np.float32)
    with pytest.raises(ValueError):
        oracle.conv2d(x, np.zeros((4, 4, 7, 7), np.float32))          # window larger than input
    with pytest.raises(ValueError):
        oracle.conv2d(x, np.zeros((3, 2, 3, 3), np.float32), groups=2)  # K not divisible by groups
    assert oracle.out_dim(5, 7, 1, 0, 1) == 0


# ---------------------------------------------------------------- fused GroupNorm chain


def _fused_case(N=2, C=3, H=12, W=13, K=8, seed=81, pad=0, stride=1):
    x = _rand((N, C, H, W), seed, 0, 0.0, 1.0)
    w = _rand((K, C, 3, 3), seed, 1, -1 / math.sqrt(9 * C), 1 / math.sqrt(9 * C))
    b = synth.normal((K,), 0.1, seed, 2)
    s = synth.normal((K,), 0.1, seed, 3)
    return x, w, b, s


@pytest.mark.parametrize("G,pad,stride", [(4, 0, 1), (2, 1, 1), (8, 1, 2), (1, 0, 1)])
def test_fused_gn_matches_torch_group_norm(G, pad, stride):
    x, w, b, s = _fused_case(pad=pad, stride=stride)
    K = w.shape[0]
    gamma = _rand((K,), 82, 0, 0.5, 1.5)
    beta = _rand((K,), 82, 1, -0.5, 0.5)
    out, v = oracle.fused_gn(x, w, b, s, gamma, beta, G, 1e-5, stride, pad, 1, 1, want_v=True)
    y = torch.from_numpy(_torch_conv(x, w, None, stride, pad, 1, 1))
    t = (y + torch.from_numpy(b.astype(np.float64))[None, :, None, None]) * \
        torch.from_numpy(s.astype(np.float64))[None, :, None, None]
    v_ref = torch.sigmoid(t)
    ref = F.group_norm(v_ref, G, torch.from_numpy(gamma.astype(np.float64)),
                       torch.from_numpy(beta.astype(np.float64)), 1e-5)
    np.testing.assert_allclose(v, v_ref.numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-9, atol=1e-10)


def test_fused_gn_sigmoid_is_logistic_of_biased_scaled_conv():
    x, w, b, s = _fused_case()
    _, v = oracle.fused_gn(x, w, b, s, None, None, 4, want_v=True)
    y, _ = oracle.conv2d(x, w)
    t = (y + b.astype(np.float64)[None, :, None, None]) * s.astype(np.float64)[None, :, None, None]
    np.testing.assert_allclose(v, scipy.special.expit(t), rtol=1e-14, atol=0)
    # sigma(-t) = 1 - sigma(t): flipping the sign of scale flips t
    _, v_neg = oracle.fused_gn(x, w, b, -s, None, None, 4, want_v=True)
    np.testing.assert_allclose(v + v_neg, 1.0, rtol=0, atol=1e-15)


def test_fused_gn_closed_form_moments():
    x, w, b, s = _fused_case(N=3, K=12)
    G, eps = 3, 1e-5
    out, v = oracle.fused_gn(x, w, b, s, None, None, G, eps, want_v=True)
    N, K = out.shape[:2]
    for n in range(N):
        for g in range(G):
            og = out[n, g * K // G:(g + 1) * K // G]
            var = np.var(v[n, g * K // G:(g + 1) * K // G])
            assert abs(og.mean()) < 1e-12
            np.testing.assert_allclose((og ** 2).mean(), var / (var + eps), rtol=1e-10)


def test_fused_gn_degenerate_cases():
    x, w, b, s = _fused_case()
    K = w.shape[0]
    beta = _rand((K,), 91, 0)
    gamma = _rand((K,), 91, 1)
    # scale = 0: v = sigmoid(0) = 1/2 everywhere, zero variance, out = beta
    out, v = oracle.fused_gn(x, w, b, np.zeros(K, np.float32), gamma, beta, 4, want_v=True)
    assert np.all(v == 0.5)
    assert np.array_equal(out, np.broadcast_to(beta.astype(np.float64)[None, :, None, None], out.shape))
    # affine parameters act per channel after normalization
    out1 = oracle.fused_gn(x, w, b, s, None, None, 4)
    outg = oracle.fused_gn(x, w, b, s, gamma, beta, 4)
    np.testing.assert_allclose(outg, out1 * gamma.astype(np.float64)[None, :, None, None]
                               + beta.astype(np.float64)[None, :, None, None], rtol=1e-12, atol=1e-13)


def test_fused_gn_rejects_bad_groups():
    x, w, b, s = _fused_case()
    with pytest.raises(ValueError):
        oracle.fused_gn(x, w, b, s, None, None, 3)   # 8 channels do not split into 3 groups
    with pytest.raises(ValueError):
        oracle.fused_gn(x, w, b, s, None, None, 4, eps=0.0)


def test_workload_recipes_are_deterministic():
    wl = synth.WORKLOADS["c1_grouped_cpg4"]
    a, b = synth.make_inputs(wl), synth.make_inputs(wl)
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["w"], b["w"])
    assert a["x"].dtype == np.float32 and a["x"].min() >= -1 and a["x"].max() <= 1
    assert np.abs(a["w"]).max() <= 1 / 6


# ---- per-axis stride, padding and dilation (the (h, w) form of the oracle)

def _random_axis_geometries(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        groups = int(rng.integers(1, 4))
        cin, cout = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        R, S = int(rng.integers(1, 7)), int(rng.integers(1, 7))
        sh, sw = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        ph, pw = int(rng.integers(0, 3)), int(rng.integers(0, 3))
        dh, dw = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        H, W = int(rng.integers(1, 14)), int(rng.integers(1, 14))
        if H + 2 * ph - dh * (R - 1) - 1 < 0 or W + 2 * pw - dw * (S - 1) - 1 < 0:
            continue
        if (sh, ph, dh) == (sw, pw, dw):
            continue  # keep only geometries that differ between the axes
        out.append((2, groups * cin, H, W, groups * cout, R, S, (sh, sw), (ph, pw), (dh, dw), groups))
    return out


@pytest.mark.parametrize("geom", _random_axis_geometries(24, 7))
def test_per_axis_matches_torch_conv2d_float64(geom):
    N, C, H, W, K, R, S, stride, pad, dil, groups = geom
    x = _rand((N, C, H, W), 81)
    w = _rand((K, C // groups, R, S), 81, 1)
    b = _rand((K,), 81, 2)
    y, A = oracle.conv2d(x, w, b, stride, pad, dil, groups)
    np.testing.assert_allclose(y, _torch_conv(x, w, b, stride, pad, dil, groups), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(A, _torch_conv(np.abs(x), np.abs(w), np.abs(b), stride, pad, dil, groups),
                               rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("geom", _random_axis_geometries(12, 8))
def test_per_axis_transposition(geom):
    """Swapping the image axes swaps the roles of (h, w) parameters and
    transposes the output: conv(x, w; s, p, d)^T == conv(x^T, w^T; s', p', d')."""
    N, C, H, W, K, R, S, stride, pad, dil, groups = geom
    x = _rand((N, C, H, W), 82)
    w = _rand((K, C // groups, R, S), 82, 1)
    y, _ = oracle.conv2d(x, w, None, stride, pad, dil, groups)
    yt, _ = oracle.conv2d(np.swapaxes(x, 2, 3), np.swapaxes(w, 2, 3), None, stride[::-1], pad[::-1], dil[::-1],
                          groups)
    # the transposed problem sums the same products in another order
    np.testing.assert_allclose(np.swapaxes(yt, 2, 3), y, rtol=1e-12, atol=1e-13)


def _scatter_conv_axes(x, w, stride, pad, dil, groups):
    """Scatter form with per-axis parameters: each input pixel adds its
    products into the outputs whose windows cover it."""
    (sh, sw), (ph, pw), (dh, dw) = stride, pad, dil
    N, C, H, W = x.shape
    K, cin, R, S = w.shape
    cout = K // groups
    Ho = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
    Wo = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
    y = np.zeros((N, K, Ho, Wo))
    for n in range(N):
        for ic in range(C):
            g = ic // cin
            for ih in range(H):
                for iw in range(W):
                    for r in range(R):
                        num_h = ih + ph - r * dh
                        if num_h % sh or not (0 <= num_h // sh < Ho):
                            continue
                        for s in range(S):
                            num_w = iw + pw - s * dw
                            if num_w % sw or not (0 <= num_w // sw < Wo):
                                continue
                            for kl in range(cout):
                                k = g * cout + kl
                                y[n, k, num_h // sh, num_w // sw] += x[n, ic, ih, iw] * w[k, ic - g * cin, r, s]
    return y


@pytest.mark.parametrize("geom", [(1, 2, 7, 6, 2, 3, 3, (2, 1), (1, 0), (1, 2), 1),
                                  (2, 4, 6, 9, 4, 2, 3, (1, 3), (0, 2), (2, 1), 2),
                                  (1, 3, 8, 5, 3, 3, 2, (3, 2), (2, 1), (1, 1), 3)])
def test_per_axis_scatter_bruteforce_exact_on_integers(geom):
    N, C, H, W, K, R, S, stride, pad, dil, groups = geom
    x = synth.integers((N, C, H, W), -2, 2, 63, 0)
    w = synth.integers((K, C // groups, R, S), -2, 2, 63, 1)
    y, _ = oracle.conv2d(x, w, None, stride, pad, dil, groups)
    assert np.array_equal(y, _scatter_conv_axes(x, w, stride, pad, dil, groups))


def test_per_axis_symmetric_equals_scalar_form():
    x = _rand((2, 4, 11, 13), 84)
    w = _rand((6, 2, 3, 5), 84, 1)
    a, _ = oracle.conv2d(x, w, None, 2, 1, 2, 2)
    b, _ = oracle.conv2d(x, w, None, (2, 2), (1, 1), (2, 2), 2)
    assert np.array_equal(a, b)
    f1 = oracle.fused_gn(x, w, _rand((6,), 84, 2), _rand((6,), 84, 3), None, None, 3, 1e-5, 1, 1, 1, 2)
    f2 = oracle.fused_gn(x, w, _rand((6,), 84, 2), _rand((6,), 84, 3), None, None, 3, 1e-5, (1, 1), (1, 1),
                         (1, 1), 2)
    assert np.array_equal(f1, f2)
