"""Seeded synthetic convolution workloads.

This module only draws random tensors and describes layer shapes. It holds none of the
quantization or convolution arithmetic: both the GPU library's tests/benchmark and the CPU
oracle take their inputs from here, and nothing else is shared between them.

Shapes follow the layer types the MicroQonv pages experiment with (onedev.kr paper digest,
sections "How it is used" and "Premises and limits": ResNet-18 style 3x3 bodies, YOLO-nano style
stacks with a large share of 1x1 convolutions, NVFP4 / NVFP6 element formats). The public
datasets the pages train on are not available, so every tensor is synthetic:

* activations X: ReLU or SiLU of N(0,1), or a heavy-tailed Student-t(3) scaled by 0.5
* weights W: Kaiming-normal, std = sqrt(2 / (Cin*Kh*Kw))
* output gradients G_Y: N(0, 1e-3)

Generation is numpy ``Generator(PCG64(seed))`` in float64, drawn in the order X, W, G_Y, then
cast to float32. Tensors come out in the framework layouts NCHW (X, G_Y) and OIHW (W).
"""
from __future__ import annotations

import dataclasses
from typing import List, Tuple

import numpy as np

FP4 = 4  # NVFP4: E2M1 elements, E4M3 scale per 4x4 square, fp32 tensor scale
FP6 = 6  # NVFP6: E2M3 elements, same scaling


@dataclasses.dataclass(frozen=True)
class ConvLayer:
    """One convolution layer's shape and the recipe for its synthetic tensors."""

    name: str
    N: int
    Cin: int
    H: int
    W: int
    Cout: int
    Kh: int
    Kw: int
    stride: int = 1             # stride along the height (and the width unless stride_w is set)
    pad: int = 0                # zero padding along the height (and the width unless pad_w is set)
    fmt: int = FP4
    x_dist: str = "normal"      # normal | relu | silu | t3
    w_dist: str = "kaiming"     # normal | kaiming
    g_dist: str = "normal1e-3"  # normal | normal1e-3
    seed: int = 0
    sr_seed: int = 1
    stride_w: int = -1          # stride along the width; -1: the same as `stride`
    pad_w: int = -1             # padding along the width; -1: the same as `pad`

    @property
    def sw(self) -> int:
        return self.stride if self.stride_w < 0 else self.stride_w

    @property
    def pw(self) -> int:
        return self.pad if self.pad_w < 0 else self.pad_w

    @property
    def Ho(self) -> int:
        return (self.H + 2 * self.pad - self.Kh) // self.stride + 1

    @property
    def Wo(self) -> int:
        return (self.W + 2 * self.pw - self.Kw) // self.sw + 1

    def gemm_flops(self) -> int:
        """2*Cout*Cin*Kh*Kw*N*Ho*Wo: the algorithmic flop count of one of the three GEMMs."""
        return 2 * self.Cout * self.Cin * self.Kh * self.Kw * self.N * self.Ho * self.Wo

    def conv_tuple(self) -> Tuple[int, ...]:
        """(N, Cin, H, W, Cout, Kh, Kw, stride_h, stride_w, pad_h, pad_w)."""
        return (self.N, self.Cin, self.H, self.W, self.Cout, self.Kh, self.Kw,
                self.stride, self.sw, self.pad, self.pw)


def _draw(rng: np.random.Generator, shape, dist: str, fan_in: int) -> np.ndarray:
    if dist == "normal":
        a = rng.standard_normal(shape)
    elif dist == "relu":
        a = np.maximum(rng.standard_normal(shape), 0.0)
    elif dist == "silu":
        z = rng.standard_normal(shape)
        a = z / (1.0 + np.exp(-z))
    elif dist == "t3":
        a = 0.5 * rng.standard_t(3.0, size=shape)
    elif dist == "kaiming":
        a = rng.standard_normal(shape) * np.sqrt(2.0 / fan_in)
    elif dist == "normal1e-3":
        a = rng.standard_normal(shape) * 1e-3
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return a.astype(np.float32)


def make_tensors(layer: ConvLayer):
    """Return (X [N,Cin,H,W], W [Cout,Cin,Kh,Kw], G_Y [N,Cout,Ho,Wo]) as float32 numpy arrays."""
    rng = np.random.Generator(np.random.PCG64(layer.seed))
    fan_in = layer.Cin * layer.Kh * layer.Kw
    x = _draw(rng, (layer.N, layer.Cin, layer.H, layer.W), layer.x_dist, fan_in)
    w = _draw(rng, (layer.Cout, layer.Cin, layer.Kh, layer.Kw), layer.w_dist, fan_in)
    g = _draw(rng, (layer.N, layer.Cout, layer.Ho, layer.Wo), layer.g_dist, fan_in)
    return x, w, g


def random_array(shape, seed: int, dist: str = "normal", fan_in: int = 1) -> np.ndarray:
    """A single seeded float32 array (used by unit tests for shapes outside the layer list)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _draw(rng, shape, dist, fan_in)


# --- the five workloads -------------------------------------------------------------------

def config1() -> List[ConvLayer]:
    """Single 3x3 conv, stride 1, no padding, N=2, 16->16 channels at 8x8, NVFP4."""
    return [ConvLayer("c1", N=2, Cin=16, H=8, W=8, Cout=16, Kh=3, Kw=3, stride=1, pad=0,
                      fmt=FP4, x_dist="normal", w_dist="normal", g_dist="normal",
                      seed=0, sr_seed=1)]


def config2() -> List[ConvLayer]:
    """ResNet-style 3x3 conv, stride 1, pad 1, N=32, 64->64 channels at 56x56, NVFP4."""
    return [ConvLayer("c2", N=32, Cin=64, H=56, W=56, Cout=64, Kh=3, Kw=3, stride=1, pad=1,
                      fmt=FP4, x_dist="relu", seed=2, sr_seed=1)]


def config3() -> List[ConvLayer]:
    """Strided 3x3 conv, stride 2, pad 1, N=64, 128->256 channels, 28x28 -> 14x14, NVFP4."""
    return [ConvLayer("c3", N=64, Cin=128, H=28, W=28, Cout=256, Kh=3, Kw=3, stride=2, pad=1,
                      fmt=FP4, x_dist="t3", seed=3, sr_seed=1)]


def config4() -> List[ConvLayer]:
    """YOLO-nano-like stack of 8 convs at N=16 (3 of 8 are 1x1), 160x160 -> 20x20, NVFP6."""
    spec = [  # (Cin, Cout, H, K, stride)
        (16, 16, 160, 3, 1),
        (16, 32, 160, 3, 2),
        (32, 32, 80, 1, 1),
        (32, 64, 80, 3, 2),
        (64, 64, 40, 1, 1),
        (64, 128, 40, 3, 2),
        (128, 256, 20, 1, 1),
        (256, 256, 20, 3, 1),
    ]
    out = []
    for i, (ci, co, h, k, s) in enumerate(spec):
        out.append(ConvLayer(f"c4.l{i + 1}", N=16, Cin=ci, H=h, W=h, Cout=co, Kh=k, Kw=k,
                             stride=s, pad=k // 2, fmt=FP6, x_dist="silu",
                             seed=40 + i, sr_seed=1))
    return out


def config5() -> List[ConvLayer]:
    """ResNet-18 conv body at N=128 (224x224 input; stem conv and FC stay fp32), NVFP4."""
    spec = []  # (Cin, Cout, H_in, K, stride)
    spec += [(64, 64, 56, 3, 1)] * 4
    for cin, cout, h in ((64, 128, 56), (128, 256, 28), (256, 512, 14)):
        spec.append((cin, cout, h, 3, 2))        # first conv of the stage
        spec.append((cin, cout, h, 1, 2))        # 1x1 stride-2 downsample
        spec += [(cout, cout, h // 2, 3, 1)] * 3
    out = []
    for i, (ci, co, h, k, s) in enumerate(spec):
        out.append(ConvLayer(f"c5.l{i + 1}", N=128, Cin=ci, H=h, W=h, Cout=co, Kh=k, Kw=k,
                             stride=s, pad=k // 2, fmt=FP4, x_dist="relu",
                             seed=50 + i, sr_seed=1 + i))
    return out


def random_layers(count: int = 40, seed: int = 2024) -> List[ConvLayer]:
    """Seeded random layer shapes for a parity sweep: batches of 1-40 (so both the 16- and the
    32-element batch tiles, ragged), 1-96 channels (partial row blocks and channel squares),
    kernels 1x1 to 3x3 with unequal sides and now and then 4 or 5 (the generic kernel), strides
    1-3 (now and then apart per axis), paddings below the kernel size and now and then equal to
    it, NVFP4 or NVFP6, and every value
    distribution. Each layer's GEMM stays below about 2*10^7 multiply-adds, so the CPU oracle
    checks every output element in a fraction of a second."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out: List[ConvLayer] = []
    dists = ["normal", "relu", "silu", "t3"]
    while len(out) < count:
        k = len(out)
        N = int(rng.integers(1, 17) if rng.random() < 0.5 else rng.integers(17, 41))
        Cin, Cout = (int(v) for v in rng.integers(1, 97, size=2))
        if rng.random() < 0.15:
            Kh = Kw = int(rng.integers(4, 6))
        else:
            Kh, Kw = (int(v) for v in rng.integers(1, 4, size=2))
        sh, sw = (int(v) for v in rng.integers(1, 4, size=2)) if rng.random() < 0.15 else (
            (int(rng.integers(1, 3)),) * 2)
        ph = int(rng.integers(0, Kh + (1 if rng.random() < 0.1 else 0)))
        pw = int(rng.integers(0, Kw + (1 if rng.random() < 0.1 else 0)))
        H, W = (int(v) for v in rng.integers(1, 25, size=2))
        Ho = (H + 2 * ph - Kh) // sh + 1
        Wo = (W + 2 * pw - Kw) // sw + 1
        if Ho < 1 or Wo < 1 or Cout * Cin * Kh * Kw * N * Ho * Wo > 20_000_000:
            continue
        out.append(ConvLayer(f"r{k:02d}", N=N, Cin=Cin, H=H, W=W, Cout=Cout, Kh=Kh, Kw=Kw,
                             stride=sh, pad=ph, stride_w=sw, pad_w=pw,
                             fmt=FP6 if rng.random() < 0.35 else FP4,
                             x_dist=dists[int(rng.integers(0, 4))], seed=300 + k,
                             sr_seed=int(rng.integers(1, 1 << 30))))
    return out


CONFIGS = {
    "c1": config1,
    "c2": config2,
    "c3": config3,
    "c4": config4,
    "c5": config5,
}


def persistent_layers() -> List[ConvLayer]:
    """Layers with enough 64-row, 2 x 8 pixel, 32-batch work items for the persistent forward and
    input-gradient launches (at least 640), whose items are not all whole: a ragged last batch
    block (36 elements) and an output row block partly past the channels (80 output channels).
    The outputs of whole items partly leave through LDS under the next item's MFMAs; these
    layers put whole and partial items in one launch. The third is NVFP6, with whole items only
    in its forward launch.
    """
    return [
        ConvLayer("q.b36.80x64", N=36, Cin=64, H=80, W=64, Cout=64, Kh=3, Kw=3, stride=1, pad=1,
                  x_dist="relu", seed=131, sr_seed=35),
        ConvLayer("q.m80.80x64", N=32, Cin=16, H=80, W=64, Cout=80, Kh=3, Kw=3, stride=1, pad=1,
                  x_dist="normal", seed=132, sr_seed=36),
        ConvLayer("q.fp6.80x64", N=64, Cin=32, H=80, W=64, Cout=64, Kh=3, Kw=3, stride=1, pad=1,
                  fmt=FP6, x_dist="silu", seed=133, sr_seed=37),
    ]


def parity_layers() -> List[ConvLayer]:
    """Mid-sized layers that span several kernel tiles with ragged tails everywhere.

    Sized so that the CPU oracle finishes each in well under a second.
    """
    return [
        ConvLayer("p.3x3s1p1", N=6, Cin=20, H=11, W=13, Cout=24, Kh=3, Kw=3, stride=1, pad=1,
                  x_dist="relu", seed=101, sr_seed=7),
        ConvLayer("p.3x3s2p1", N=5, Cin=13, H=9, W=10, Cout=17, Kh=3, Kw=3, stride=2, pad=1,
                  x_dist="t3", seed=102, sr_seed=8),
        ConvLayer("p.1x1s1", N=8, Cin=36, H=7, W=6, Cout=40, Kh=1, Kw=1, stride=1, pad=0,
                  x_dist="silu", seed=103, sr_seed=9),
        ConvLayer("p.1x1s2", N=3, Cin=12, H=10, W=9, Cout=20, Kh=1, Kw=1, stride=2, pad=0,
                  x_dist="relu", seed=104, sr_seed=10),
        ConvLayer("p.3x3s1p0.fp6", N=7, Cin=9, H=12, W=12, Cout=70, Kh=3, Kw=3, stride=1,
                  pad=0, fmt=FP6, x_dist="silu", seed=105, sr_seed=11),
        ConvLayer("p.3x3s2p1.fp6", N=4, Cin=40, H=15, W=16, Cout=36, Kh=3, Kw=3, stride=2,
                  pad=1, fmt=FP6, x_dist="normal", seed=106, sr_seed=12),
        ConvLayer("p.wide", N=36, Cin=72, H=9, W=9, Cout=136, Kh=3, Kw=3, stride=1, pad=1,
                  x_dist="relu", seed=107, sr_seed=13),
        ConvLayer("p.5x5s1p2", N=4, Cin=8, H=10, W=10, Cout=12, Kh=5, Kw=5, stride=1, pad=2,
                  x_dist="normal", seed=108, sr_seed=14),
        # more pixel tiles than the GPU has CUs: workgroups loop over several work items
        ConvLayer("p.many.s1", N=8, Cin=8, H=66, W=70, Cout=12, Kh=3, Kw=3, stride=1, pad=1,
                  x_dist="relu", seed=109, sr_seed=15),
        ConvLayer("p.many.s2", N=4, Cin=8, H=100, W=100, Cout=8, Kh=3, Kw=3, stride=2, pad=1,
                  x_dist="normal", seed=110, sr_seed=16),
        # batches of whole 16-element groups, stride 1: the weight gradient's stages then hold
        # exactly one staging item per producer lane (15-pixel stages for 16 batch elements,
        # 7-pixel stages for 32 and more), with ragged pixel blocks and channel tiles
        ConvLayer("p.b16.s1", N=16, Cin=20, H=17, W=19, Cout=24, Kh=3, Kw=3, stride=1, pad=1,
                  x_dist="relu", seed=111, sr_seed=17),
        ConvLayer("p.b32.s1", N=32, Cin=12, H=9, W=23, Cout=40, Kh=3, Kw=3, stride=1, pad=1,
                  x_dist="normal", seed=112, sr_seed=18),
        ConvLayer("p.b48.1x1.fp6", N=48, Cin=36, H=6, W=11, Cout=20, Kh=1, Kw=1, stride=1,
                  pad=0, fmt=FP6, x_dist="silu", seed=113, sr_seed=19),
        ConvLayer("p.b16.k2", N=16, Cin=8, H=7, W=9, Cout=8, Kh=2, Kw=2, stride=1, pad=0,
                  x_dist="t3", seed=114, sr_seed=20),
        # the same at stride 2 (10-pixel stages for 16 batch elements, 5 for 32 and more)
        ConvLayer("p.b16.s2", N=16, Cin=20, H=15, W=17, Cout=24, Kh=3, Kw=3, stride=2, pad=1,
                  x_dist="relu", seed=115, sr_seed=21),
        ConvLayer("p.b32.s2.fp6", N=32, Cin=12, H=11, W=13, Cout=20, Kh=3, Kw=3, stride=2,
                  pad=1, fmt=FP6, x_dist="normal", seed=116, sr_seed=22),
        ConvLayer("p.b32.1x1s2", N=32, Cin=24, H=9, W=10, Cout=36, Kh=1, Kw=1, stride=2, pad=0,
                  x_dist="silu", seed=117, sr_seed=23),
        # kernels, strides and paddings that differ between height and width, stride 3, and a
        # padding as large as the kernel
        ConvLayer("p.1x3.p01", N=6, Cin=12, H=9, W=11, Cout=20, Kh=1, Kw=3, stride=1, pad=0,
                  pad_w=1, x_dist="relu", seed=118, sr_seed=24),
        ConvLayer("p.3x1.p10.fp6", N=8, Cin=16, H=10, W=7, Cout=12, Kh=3, Kw=1, stride=1, pad=1,
                  pad_w=0, fmt=FP6, x_dist="silu", seed=119, sr_seed=25),
        ConvLayer("p.3x3.s12", N=5, Cin=10, H=9, W=12, Cout=14, Kh=3, Kw=3, stride=1, pad=1,
                  stride_w=2, x_dist="normal", seed=120, sr_seed=26),
        ConvLayer("p.3x3.p01", N=16, Cin=20, H=8, W=9, Cout=24, Kh=3, Kw=3, stride=1, pad=0,
                  pad_w=1, x_dist="t3", seed=121, sr_seed=27),
        ConvLayer("p.3x3.s3", N=4, Cin=8, H=13, W=14, Cout=12, Kh=3, Kw=3, stride=3, pad=1,
                  x_dist="relu", seed=122, sr_seed=28),
        ConvLayer("p.1x1.p1", N=8, Cin=12, H=6, W=7, Cout=16, Kh=1, Kw=1, stride=1, pad=1,
                  x_dist="normal", seed=123, sr_seed=29),
        # batches of at most 16 (two pixels per MFMA): a ragged batch at stride 2 with a row
        # block that is partly past the output channels, and an odd width with 72 output rows
        ConvLayer("p.b12.s2", N=12, Cin=40, H=21, W=30, Cout=28, Kh=3, Kw=3, stride=2, pad=1,
                  x_dist="silu", seed=124, sr_seed=30),
        ConvLayer("p.b16.w23.fp6", N=16, Cin=36, H=13, W=23, Cout=72, Kh=3, Kw=3, stride=1,
                  pad=1, fmt=FP6, x_dist="relu", seed=125, sr_seed=31),
        # at most 16 channels on both sides and whole 16-element batch groups: the weight
        # gradient's 16-row slots with two pixels per MFMA, for 32-element stages at stride 1
        # and 2 and 16-element stages at stride 2, each over several ragged pixel blocks
        ConvLayer("p.b32.c16", N=32, Cin=12, H=19, W=71, Cout=16, Kh=3, Kw=3, stride=1, pad=1,
                  x_dist="relu", seed=126, sr_seed=32),
        ConvLayer("p.b48.c16.s2.fp6", N=48, Cin=8, H=17, W=91, Cout=16, Kh=3, Kw=3, stride=2,
                  pad=1, fmt=FP6, x_dist="normal", seed=127, sr_seed=33),
        ConvLayer("p.b16.c16.s2.fp6", N=16, Cin=16, H=21, W=101, Cout=12, Kh=3, Kw=3, stride=2,
                  pad=1, fmt=FP6, x_dist="silu", seed=128, sr_seed=34),
    ]
