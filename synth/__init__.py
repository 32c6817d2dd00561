"""Seeded synthetic inputs shared by the tests, the smoke entry and the benchmark.

This module only draws random numbers: it holds no convolution or
normalisation arithmetic, so the oracle and the HIP path can both consume
its buffers without sharing any of the method.

Every tensor comes from its own numpy PCG64 stream, seeded with
``seed * 16 + slot`` (slot 0 = x, 1 = w, 2 = bias, 3 = scale), so a tensor
does not change when another tensor of the same workload changes shape.
Uniform draws are ``lo + (hi - lo) * u`` with ``u`` in [0, 1) in float64,
normal draws are ``std * z``; both are rounded once to float32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

SLOT_X, SLOT_W, SLOT_BIAS, SLOT_SCALE = 0, 1, 2, 3


def _rng(seed: int, slot: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed * 16 + slot))


def uniform(shape, lo: float, hi: float, seed: int, slot: int) -> np.ndarray:
    u = _rng(seed, slot).random(int(np.prod(shape)), dtype=np.float64)
    return (lo + (hi - lo) * u).astype(np.float32).reshape(shape)


def normal(shape, std: float, seed: int, slot: int) -> np.ndarray:
    z = _rng(seed, slot).standard_normal(int(np.prod(shape)), dtype=np.float64)
    return (std * z).astype(np.float32).reshape(shape)


def integers(shape, lo: int, hi: int, seed: int, slot: int) -> np.ndarray:
    """Small integers in [lo, hi] as float32 (exact sums for parity-by-bits)."""
    v = _rng(seed, slot).integers(lo, hi + 1, size=int(np.prod(shape)))
    return v.astype(np.float32).reshape(shape)


@dataclass(frozen=True)
class Workload:
    """One convolution problem with its input recipe.

    x_dist / w_dist / bias_dist / scale_dist are ("uniform", lo, hi) or
    ("normal", std).  gn_groups > 0 marks the fused GroupNorm chain.
    """
    name: str
    N: int
    C: int
    H: int
    W: int
    K: int
    R: int
    S: int
    stride: int
    pad: object  # an int, or an (h, w) pair
    dil: int
    groups: int
    seed: int
    x_dist: Tuple
    w_dist: Tuple
    bias_dist: Optional[Tuple] = None
    scale_dist: Optional[Tuple] = None
    gn_groups: int = 0
    eps: float = 1e-5
    note: str = field(default="", compare=False)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def fused(self) -> bool:
        return self.gn_groups > 0


def _draw(dist, shape, seed, slot):
    if dist is None:
        return None
    if dist[0] == "uniform":
        return uniform(shape, dist[1], dist[2], seed, slot)
    if dist[0] == "normal":
        return normal(shape, dist[1], seed, slot)
    if dist[0] == "int":
        return integers(shape, dist[1], dist[2], seed, slot)
    raise ValueError(dist)


def make_inputs(wl: Workload) -> dict:
    """x, w (and bias, scale, gamma, beta for the fused chain) as float32."""
    out = {
        "x": _draw(wl.x_dist, (wl.N, wl.C, wl.H, wl.W), wl.seed, SLOT_X),
        "w": _draw(wl.w_dist, (wl.K, wl.C // wl.groups, wl.R, wl.S), wl.seed, SLOT_W),
        "bias": _draw(wl.bias_dist, (wl.K,), wl.seed, SLOT_BIAS),
        "scale": _draw(wl.scale_dist, (wl.K,), wl.seed, SLOT_SCALE),
    }
    if wl.fused:
        out["gamma"] = np.ones((wl.K,), dtype=np.float32)
        out["beta"] = np.zeros((wl.K,), dtype=np.float32)
    return out


def _u(b):
    return ("uniform", -b, b)


# The five workloads (seven shape rows).  Weight bounds are +-1/sqrt(fan_in)
# with fan_in = (C/groups)*R*S.
WORKLOADS = {
    "c1_grouped_cpg4": Workload("c1_grouped_cpg4", 1, 8, 16, 16, 8, 3, 3, 1, 1, 1, 2, 1001,
                                ("uniform", -1.0, 1.0), _u(1 / math.sqrt(36))),
    "c2_depthwise_144": Workload("c2_depthwise_144", 4, 144, 56, 56, 144, 3, 3, 1, 1, 1, 144, 1002,
                                 ("normal", 1.0), _u(1 / 3)),
    "c3a_grouped_g64": Workload("c3a_grouped_g64", 32, 256, 64, 64, 256, 3, 3, 1, 1, 1, 64, 1003,
                                ("uniform", -1.0, 1.0), _u(1 / math.sqrt(36))),
    "c3b_grouped_g128": Workload("c3b_grouped_g128", 32, 256, 64, 64, 256, 3, 3, 1, 1, 1, 128, 1004,
                                 ("uniform", -1.0, 1.0), _u(1 / math.sqrt(18))),
    "c3c_depthwise_g256": Workload("c3c_depthwise_g256", 32, 256, 64, 64, 256, 3, 3, 1, 1, 1, 256, 1005,
                                   ("uniform", -1.0, 1.0), _u(1 / 3)),
    "c4_dense_5x9": Workload("c4_dense_5x9", 8, 32, 256, 256, 64, 5, 9, 1, 0, 1, 1, 1006,
                             ("uniform", 0.0, 1.0), _u(1 / math.sqrt(1440))),
    "c5_fused_gn": Workload("c5_fused_gn", 64, 8, 256, 256, 32, 3, 3, 1, 0, 1, 1, 1007,
                            ("uniform", 0.0, 1.0), _u(1 / math.sqrt(72)),
                            bias_dist=("normal", 0.1), scale_dist=("normal", 0.1),
                            gn_groups=8, eps=1e-5),
}

ROW_ORDER = list(WORKLOADS)

# Depthwise layers ("same" padding dil * (R // 2), batch 16) of MobileNet-,
# EfficientNet-, ConvNeXt- and atrous (dilated) networks, and a grouped
# stride-2 layer: the general-geometry shapes measured beside the five
# workloads (not part of the benchmark step).
EXTRA_WORKLOADS = {
    "dw3s2_mobilenet_144x112": Workload("dw3s2_mobilenet_144x112", 16, 144, 112, 112, 144, 3, 3, 2, 1, 1, 144,
                                        211, ("uniform", -1.0, 1.0), _u(1 / 3)),
    "dw5_efficientnet_240x28": Workload("dw5_efficientnet_240x28", 16, 240, 28, 28, 240, 5, 5, 1, 2, 1, 240,
                                        212, ("uniform", -1.0, 1.0), _u(1 / 5)),
    "dw7_convnext_96x56": Workload("dw7_convnext_96x56", 16, 96, 56, 56, 96, 7, 7, 1, 3, 1, 96,
                                   213, ("uniform", -1.0, 1.0), _u(1 / 7)),
    "dw5s2_efficientnet_144x56": Workload("dw5s2_efficientnet_144x56", 16, 144, 56, 56, 144, 5, 5, 2, 2, 1, 144,
                                          214, ("uniform", -1.0, 1.0), _u(1 / 5)),
    "dw3d2_atrous_576x32": Workload("dw3d2_atrous_576x32", 16, 576, 32, 32, 576, 3, 3, 1, 2, 2, 576,
                                    215, ("uniform", -1.0, 1.0), _u(1 / 3)),
    # grouped 3x3 at stride 2 with 4 channels per group (a downsampling
    # grouped layer)
    "g3s2_cpg4_256x56": Workload("g3s2_cpg4_256x56", 16, 256, 56, 56, 256, 3, 3, 2, 1, 1, 64,
                                 216, ("uniform", -1.0, 1.0), _u(1 / 6)),
    # the same at 8 channels per group (32 groups: a ResNeXt-style
    # downsampling layer)
    "g3s2_cpg8_256x56": Workload("g3s2_cpg8_256x56", 16, 256, 56, 56, 256, 3, 3, 2, 1, 1, 32,
                                 217, ("uniform", -1.0, 1.0), _u(1 / math.sqrt(72))),
    # depthwise 5x5 with a channel multiplier of 2 (one input and two output
    # channels per group)
    "dwm5_mult2_96x56": Workload("dwm5_mult2_96x56", 16, 96, 56, 56, 192, 5, 5, 1, 2, 1, 96,
                                 218, ("uniform", -1.0, 1.0), _u(1 / 5)),
    # late-stage depthwise layers whose output width is not a multiple of 4
    # (14 and 7 columns)
    "dw5_efficientnet_672x14": Workload("dw5_efficientnet_672x14", 16, 672, 14, 14, 672, 5, 5, 1, 2, 1, 672,
                                        219, ("uniform", -1.0, 1.0), _u(1 / 5)),
    "dw7_convnext_768x7": Workload("dw7_convnext_768x7", 16, 768, 7, 7, 768, 7, 7, 1, 3, 1, 768,
                                   220, ("uniform", -1.0, 1.0), _u(1 / 7)),
    "dw3s2_mobilenet_576x14": Workload("dw3s2_mobilenet_576x14", 16, 576, 14, 14, 576, 3, 3, 2, 1, 1, 576,
                                       221, ("uniform", -1.0, 1.0), _u(1 / 3)),
    # late-stage depthwise 3x3 stride-1 layers (14x14 and 7x7 planes)
    "dw3_mobilenet_576x14": Workload("dw3_mobilenet_576x14", 16, 576, 14, 14, 576, 3, 3, 1, 1, 1, 576,
                                     222, ("uniform", -1.0, 1.0), _u(1 / 3)),
    "dw3_mobilenet_960x7": Workload("dw3_mobilenet_960x7", 16, 960, 7, 7, 960, 3, 3, 1, 1, 1, 960,
                                    223, ("uniform", -1.0, 1.0), _u(1 / 3)),
}

# Dense and 32-channel-group layers on the implicit GEMM (ResNet- and
# ResNeXt-style shapes at batch 16), 3x3 at stride 1 and 2, a 1x1
# reduction, 3x3 at dilation 2, 5x5 and 7x7 at stride 2, two 3-channel
# first layers and an Inception-style 1x7 / 7x1 pair; x ~ U[-1, 1],
# w ~ U[+-1/sqrt(cin * R * S)].
IGEMM_WORKLOADS = {
    "g3s2_cpg32_1024x28": Workload("g3s2_cpg32_1024x28", 16, 1024, 28, 28, 1024, 3, 3, 2, 1, 1, 32, 901,
                                   ("uniform", -1.0, 1.0), _u(1 / math.sqrt(32 * 9))),
    "g3_cpg32_512x28": Workload("g3_cpg32_512x28", 16, 512, 28, 28, 512, 3, 3, 1, 1, 1, 16, 903,
                                ("uniform", -1.0, 1.0), _u(1 / math.sqrt(32 * 9))),
    "dense3_64x56": Workload("dense3_64x56", 16, 64, 56, 56, 64, 3, 3, 1, 1, 1, 1, 904,
                             ("uniform", -1.0, 1.0), _u(1 / math.sqrt(64 * 9))),
    "dense3_128x112": Workload("dense3_128x112", 16, 128, 112, 112, 128, 3, 3, 1, 1, 1, 1, 915,
                               ("uniform", -1.0, 1.0), _u(1 / math.sqrt(128 * 9))),
    "dense3_128x28": Workload("dense3_128x28", 16, 128, 28, 28, 128, 3, 3, 1, 1, 1, 1, 916,
                              ("uniform", -1.0, 1.0), _u(1 / math.sqrt(128 * 9))),
    "dense3_256x14": Workload("dense3_256x14", 16, 256, 14, 14, 256, 3, 3, 1, 1, 1, 1, 917,
                              ("uniform", -1.0, 1.0), _u(1 / math.sqrt(256 * 9))),
    "dense3s2_128x56": Workload("dense3s2_128x56", 16, 128, 56, 56, 128, 3, 3, 2, 1, 1, 1, 905,
                                ("uniform", -1.0, 1.0), _u(1 / math.sqrt(128 * 9))),
    "dense1_256x56": Workload("dense1_256x56", 16, 256, 56, 56, 64, 1, 1, 1, 0, 1, 1, 906,
                              ("uniform", -1.0, 1.0), _u(1 / 16.0)),
    # geometries on the flattened-pixel kernel only: a dilated 3x3 (a
    # DeepLab-style dilated stage), dense 5x5 and 7x7 at stride 2
    "dense3d2_256x28": Workload("dense3d2_256x28", 16, 256, 28, 28, 256, 3, 3, 1, 2, 2, 1, 907,
                                ("uniform", -1.0, 1.0), _u(1 / math.sqrt(256 * 9))),
    "dense3d4_256x28": Workload("dense3d4_256x28", 16, 256, 28, 28, 256, 3, 3, 1, 4, 4, 1, 914,
                                ("uniform", -1.0, 1.0), _u(1 / math.sqrt(256 * 9))),
    "dense5s2_64x56": Workload("dense5s2_64x56", 16, 64, 56, 56, 64, 5, 5, 2, 2, 1, 1, 908,
                               ("uniform", -1.0, 1.0), _u(1 / math.sqrt(64 * 25))),
    "dense7s2_16x112": Workload("dense7s2_16x112", 16, 16, 112, 112, 64, 7, 7, 2, 3, 1, 1, 909,
                                ("uniform", -1.0, 1.0), _u(1 / math.sqrt(16 * 49))),
    # first layers with 3 input channels: a ResNet-style stem (7x7 stride 2)
    # and a 3x3 stride-2 stem
    "stem7s2_3x224": Workload("stem7s2_3x224", 16, 3, 224, 224, 64, 7, 7, 2, 3, 1, 1, 910,
                              ("uniform", -1.0, 1.0), _u(1 / math.sqrt(3 * 49))),
    "stem3s2_3x224": Workload("stem3s2_3x224", 16, 3, 224, 224, 32, 3, 3, 2, 1, 1, 1, 911,
                              ("uniform", -1.0, 1.0), _u(1 / math.sqrt(3 * 9))),
    # the factorized 7x7 of an Inception-style 17x17 block: 1x7 then 7x1
    "incep1x7_160x17": Workload("incep1x7_160x17", 16, 160, 17, 17, 160, 1, 7, 1, (0, 3), 1, 1, 912,
                                ("uniform", -1.0, 1.0), _u(1 / math.sqrt(160 * 7))),
    "incep7x1_160x17": Workload("incep7x1_160x17", 16, 160, 17, 17, 160, 7, 1, 1, (3, 0), 1, 1, 913,
                                ("uniform", -1.0, 1.0), _u(1 / math.sqrt(160 * 7))),
}

# Grouped 3x3 shape grid (stride 1, padding 1, dilation 1, no bias, the
# fixed experiment of the GroupConv Atlas): 80 shapes standing in for the
# Atlas's own 80-shape list, which is not published.  Batch {1, 8} x
# channels {64, 256} x square images {14, 28, 56, 112} x channels per group
# {1, 2, 4, 8, 16}; C = K, x ~ U[-1, 1], w ~ U[+-1/sqrt(9 * cpg)], seed
# 3000 + position in the grid.
ATLAS_BATCH = (1, 8)
ATLAS_CHANNELS = (64, 256)
ATLAS_SIZES = (14, 28, 56, 112)
ATLAS_CPG = (1, 2, 4, 8, 16)


def _atlas_grid():
    grid = {}
    for n in ATLAS_BATCH:
        for c in ATLAS_CHANNELS:
            for hw in ATLAS_SIZES:
                for cpg in ATLAS_CPG:
                    name = "g3_n%d_c%d_%dx%d_cpg%d" % (n, c, hw, hw, cpg)
                    grid[name] = Workload(name, n, c, hw, hw, c, 3, 3, 1, 1, 1, c // cpg, 3000 + len(grid),
                                          ("uniform", -1.0, 1.0), _u(1 / math.sqrt(9 * cpg)))
    return grid


ATLAS_GRID = _atlas_grid()
