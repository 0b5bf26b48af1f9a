"""PyTorch modules over the library: a quantize-once convolution for training and inference.

``MQConv2d`` is a drop-in ``nn.Conv2d`` (groups 1, dilation 1, no bias) whose three GEMMs run
through the library, following the onedev.kr MicroQonv digest (sections "How it works" and "How it
differs"):

  forward   X (NCHW) -> quantized channel-batch-first squares  } one batched call
            W (OIHW) -> quantized tap-major squares             } (quantize once, RNE)
            Y = conv_fwd(Xq, Wq), back to NCHW
  backward  G_Y (NCHW) -> quantized channel-batch-first squares, one call (quantize once, SR)
            G_W = conv_wgrad(G_Yq, Xq) (the forward's Xq is kept, not re-quantized)
            G_X = conv_dgrad(Wq, G_Yq)   (the forward's Wq is kept)

so each of X, W and G_Y is quantized exactly once per step and reused by both GEMMs that read it.
Every layout change, quantization and GEMM is a library call on torch's current stream; the
module only allocates buffers and marshals arguments. Batch norm, activations, residual adds,
pooling and the first and last layers stay in PyTorch fp32, the precision policy the digest's
experiments use for the layers it does not quantize.

Stochastic rounding draws its bits from a seed per call: ``seed_base + layer_index +
layers * step`` with ``step`` counted by the module (one per training forward), so a run is
reproducible and no two layers or steps share a stream of random bits.

In eval mode with ``cache_weight=True`` the weight is quantized once and reused until the
parameter changes (its version counter moves): the inference path then quantizes only
activations.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import torch
from torch import nn

from . import (MQ_NVFP4, MQ_QUANTIZE_WS_BYTES, MQ_ROLE_ACT, MQ_ROLE_GRAD, MQ_ROLE_WEIGHT,
               MQ_RNE, MQ_SR, MQ_SRC_NCHW, MQ_SRC_OIHW, QTensor, mq_conv_backward,
               mq_conv_dgrad, mq_conv_fwd, mq_conv_wgrad, mq_quantize_batch, mq_quantize_nchw, mq_quantize_weight,
               mq_relayout_cbf, mq_relayout_weight, mq_wgrad_workspace_bytes, out_hw,
               quant_job)


def _check_input(t: torch.Tensor, what: str, ndim: int = 4):
    if not t.is_cuda or t.dtype != torch.float32 or t.dim() != ndim:
        raise ValueError(f"{what}: expected a {ndim}-D float32 CUDA tensor, got "
                         f"{tuple(t.shape)} {t.dtype} on {t.device}")


def quantize_weight(weight: torch.Tensor, fmt: int, ws: torch.Tensor) -> QTensor:
    """OIHW fp32 weight -> quantized tap-major weight (RNE), one library call."""
    Cout, Cin, Kh, Kw = weight.shape
    qw = QTensor(Kh, Kw, Cout, Cin, fmt, MQ_ROLE_WEIGHT, weight.device)
    mq_quantize_weight(weight, qw, MQ_RNE, 0, ws)
    return qw


def quantize_activation(x: torch.Tensor, fmt: int, rnd: int, seed: int, role: int,
                        ws: torch.Tensor) -> QTensor:
    """NCHW fp32 tensor -> quantized channel-batch-first tensor with the given rounding (one
    library call: amax pass, then a pass that reads NCHW and writes squares)."""
    N, C, H, W = x.shape
    q = QTensor(H, W, C, N, fmt, role, x.device)
    mq_quantize_nchw(x, q, rnd, seed, ws)
    return q


class MQConv2dFunction(torch.autograd.Function):
    """Autograd function: forward and backward of one convolution through the library."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, weight: torch.Tensor, stride: int, padding: int, fmt: int,
                sr_seed: int, qw_cached: Optional[QTensor]):
        _check_input(x, "input")
        _check_input(weight, "weight")
        x = x.contiguous()
        weight = weight.contiguous()
        N, Cin, H, W = x.shape
        Cout, Cin_w, Kh, Kw = weight.shape
        if Cin_w != Cin:
            raise ValueError(f"input has {Cin} channels, weight expects {Cin_w}")
        conv = (N, Cin, H, W, Cout, Kh, Kw, stride, stride, padding, padding)
        Ho, Wo = out_hw(conv)
        dev = x.device
        ws = torch.empty(2 * MQ_QUANTIZE_WS_BYTES, dtype=torch.uint8, device=dev)
        if qw_cached is not None:
            qx = quantize_activation(x, fmt, MQ_RNE, 0, MQ_ROLE_ACT, ws[:MQ_QUANTIZE_WS_BYTES])
            qw = qw_cached
        else:  # X and W together: one amax launch and one quantizing launch
            qx = QTensor(H, W, Cin, N, fmt, MQ_ROLE_ACT, dev)
            qw = QTensor(Kh, Kw, Cout, Cin, fmt, MQ_ROLE_WEIGHT, dev)
            mq_quantize_batch([
                quant_job(x, MQ_SRC_NCHW, qx, MQ_RNE, 0, ws[:MQ_QUANTIZE_WS_BYTES]),
                quant_job(weight, MQ_SRC_OIHW, qw, MQ_RNE, 0, ws[MQ_QUANTIZE_WS_BYTES:])])
        yc = torch.empty(Ho * Wo * Cout * N, dtype=torch.float32, device=dev)
        mq_conv_fwd(conv, qx, qw, yc)
        y = torch.empty((N, Cout, Ho, Wo), dtype=torch.float32, device=dev)
        mq_relayout_cbf(yc, y, N, Cout, Ho, Wo, 1)
        ctx.conv, ctx.fmt, ctx.sr_seed = conv, fmt, sr_seed
        ctx.qx, ctx.qw = qx, qw
        return y

    @staticmethod
    def backward(ctx, gy: torch.Tensor):
        conv, fmt = ctx.conv, ctx.fmt
        N, Cin, H, W, Cout, Kh, Kw = conv[:7]
        Ho, Wo = out_hw(conv)
        gy = gy.contiguous().float()
        dev = gy.device
        ws = torch.empty(MQ_QUANTIZE_WS_BYTES, dtype=torch.uint8, device=dev)
        qg = quantize_activation(gy, fmt, MQ_SR, ctx.sr_seed, MQ_ROLE_GRAD, ws)
        gx = gw = None
        need_x, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if need_w:
            gwk = torch.empty(Kh * Kw * Cout * Cin, dtype=torch.float32, device=dev)
            wsb = torch.empty(max(1, mq_wgrad_workspace_bytes(conv)), dtype=torch.uint8,
                              device=dev)
        if need_x:
            gxc = torch.empty(H * W * Cin * N, dtype=torch.float32, device=dev)
        if need_w and need_x:  # both gradients in one call (their launches overlap)
            mq_conv_backward(conv, ctx.qw, qg, ctx.qx, gwk, gxc, wsb)
        elif need_w:
            mq_conv_wgrad(conv, qg, ctx.qx, gwk, wsb)
        elif need_x:
            mq_conv_dgrad(conv, ctx.qw, qg, gxc)
        if need_w:
            gw = torch.empty((Cout, Cin, Kh, Kw), dtype=torch.float32, device=dev)
            mq_relayout_weight(gwk, gw, Cout, Cin, Kh, Kw, 1)
        if need_x:
            gx = torch.empty((N, Cin, H, W), dtype=torch.float32, device=dev)
            mq_relayout_cbf(gxc, gx, N, Cin, H, W, 1)
        ctx.qx = ctx.qw = None
        return gx, gw, None, None, None, None, None


class MQConv2d(nn.Module):
    """Square-kernel convolution (stride s, zero padding p, no bias) whose forward and backward
    GEMMs run on quantized operands (NVFP4 or NVFP6); fp32 master weight."""

    def __init__(self, in_channels: int, out_channels: int, kernel_size: int, stride: int = 1,
                 padding: int = 0, fmt: int = MQ_NVFP4, layer_index: int = 0, layers: int = 1,
                 seed_base: int = 1, cache_weight: bool = False):
        super().__init__()
        self.in_channels, self.out_channels = in_channels, out_channels
        self.kernel_size, self.stride, self.padding = kernel_size, stride, padding
        self.fmt = fmt
        self.layer_index, self.layers, self.seed_base = layer_index, layers, seed_base
        self.cache_weight = cache_weight
        self.weight = nn.Parameter(torch.empty(out_channels, in_channels, kernel_size,
                                               kernel_size))
        nn.init.kaiming_normal_(self.weight, mode="fan_in", nonlinearity="relu")
        self.step = 0
        self._qw: Optional[QTensor] = None
        self._qw_key: Optional[Tuple[int, int]] = None

    def sr_seed(self) -> int:
        return self.seed_base + self.layer_index + self.layers * self.step

    def _cached_weight(self) -> Optional[QTensor]:
        if self.training or not self.cache_weight:
            return None
        key = (self.weight.data_ptr(), self.weight._version)
        if self._qw is None or self._qw_key != key:
            ws = torch.empty(MQ_QUANTIZE_WS_BYTES, dtype=torch.uint8, device=self.weight.device)
            with torch.no_grad():
                self._qw = quantize_weight(self.weight.detach().contiguous(), self.fmt, ws)
            self._qw_key = key
        return self._qw

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        seed = self.sr_seed()
        if self.training:
            self.step += 1
        return MQConv2dFunction.apply(x, self.weight, self.stride, self.padding, self.fmt, seed,
                                      self._cached_weight())

    def extra_repr(self) -> str:
        return (f"{self.in_channels}, {self.out_channels}, kernel_size={self.kernel_size}, "
                f"stride={self.stride}, padding={self.padding}, fmt=NVFP{self.fmt}")


# ---- ResNet-18 with the 19 body convolutions quantized ---------------------------------------

class BasicBlock(nn.Module):
    def __init__(self, cin: int, cout: int, stride: int, convs: List[MQConv2d]):
        super().__init__()
        self.conv1 = convs[0]
        self.bn1 = nn.BatchNorm2d(cout)
        self.conv2 = convs[1]
        self.bn2 = nn.BatchNorm2d(cout)
        self.down = None
        if len(convs) == 3:
            self.down = convs[2]
            self.bn_down = nn.BatchNorm2d(cout)

    def forward(self, x):
        out = torch.relu(self.bn1(self.conv1(x)))
        out = self.bn2(self.conv2(out))
        sc = x if self.down is None else self.bn_down(self.down(x))
        return torch.relu(out + sc)


class ResNet18MQ(nn.Module):
    """ResNet-18 whose 19 body convolutions (layer1..layer4, downsample 1x1 included) are
    MQConv2d; the 7x7 stem, batch norms, pooling and the classifier stay fp32 PyTorch."""

    BODY = ([(64, 64, 1)] * 2 + [(64, 128, 2), (128, 128, 1)] + [(128, 256, 2), (256, 256, 1)] +
            [(256, 512, 2), (512, 512, 1)])

    def __init__(self, num_classes: int = 1000, fmt: int = MQ_NVFP4, seed_base: int = 1):
        super().__init__()
        self.stem = nn.Conv2d(3, 64, 7, 2, 3, bias=False)
        self.bn = nn.BatchNorm2d(64)
        self.pool = nn.MaxPool2d(3, 2, 1)
        specs = []  # (cin, cout, k, stride, pad) of every quantized conv, network order
        for cin, cout, s in self.BODY:
            specs.append((cin, cout, 3, s, 1))
            specs.append((cout, cout, 3, 1, 1))
            if s != 1 or cin != cout:
                specs.append((cin, cout, 1, s, 0))
        n = len(specs)
        convs = [MQConv2d(ci, co, k, s, p, fmt, i, n, seed_base) for i, (ci, co, k, s, p)
                 in enumerate(specs)]
        self.mq_convs = nn.ModuleList(convs)
        blocks, i = [], 0
        for cin, cout, s in self.BODY:
            k = 3 if (s != 1 or cin != cout) else 2
            blocks.append(BasicBlock(cin, cout, s, convs[i:i + k]))
            i += k
        self.blocks = nn.Sequential(*blocks)
        self.fc = nn.Linear(512, num_classes)

    def forward(self, x):
        x = self.pool(torch.relu(self.bn(self.stem(x))))
        x = self.blocks(x)
        return self.fc(torch.flatten(nn.functional.adaptive_avg_pool2d(x, 1), 1))
