"""One convolution layer's pass through the quantize-once path, as a list of library calls.

Device buffers for one layer (fp32 inputs, their channel-batch-first copies, the three quantized
tensors, the outputs and the weight-gradient workspace) and the calls of one pass, in order:

  quantize_x   X NCHW -> quantized channel-batch-first squares (round to nearest)
  quantize_w   W OIHW -> quantized tap-major squares (round to nearest), one call
  quantize_g   G_Y (stochastic, seed per pass)   conv_fwd / conv_wgrad / conv_dgrad

X goes from NCHW to its quantized channel-batch-first layout in one call (mq_quantize_nchw: an
amax pass, then a pass that reads NCHW and writes squares; no fp32 channel-batch-first copy).
W goes from OIHW to its quantized tap-major layout in one call (mq_quantize_weight). G_Y's
quantization runs its own amax pass.

G_Y is taken as already channel-batch-first (it is the next layer's input-gradient output).
Every call goes through the C ABI on the current stream; nothing here computes.
"""
from __future__ import annotations

from collections import OrderedDict
from typing import Callable, Dict

import torch

from . import (MQ_QUANTIZE_WS_BYTES, MQ_ROLE_ACT, MQ_ROLE_GRAD,
               MQ_ROLE_WEIGHT, MQ_RNE, MQ_SR, QTensor, conv_struct,
               mq_conv_dgrad, mq_conv_fwd, mq_conv_wgrad, mq_quantize, mq_quantize_nchw,
               mq_quantize_weight, mq_wgrad_workspace_bytes, out_hw)


class LayerStep:
    """conv = (N, Cin, H, W, Cout, Kh, Kw, sh, sw, ph, pw); x: NCHW, w: OIHW, g_cbf: G_Y in
    [Ho][Wo][Cout][N] order (all fp32 device tensors, any shape with the right element count)."""

    def __init__(self, conv, fmt: int, x: torch.Tensor, w: torch.Tensor, g_cbf: torch.Tensor,
                 sr_seed_base: int = 1):
        self.p = conv_struct(conv)
        c = self.p
        dev = x.device
        Ho, Wo = out_hw(c)
        self.fmt, self.sr_seed_base = int(fmt), int(sr_seed_base)
        self.x, self.w, self.gc = x, w, g_cbf
        f32 = dict(dtype=torch.float32, device=dev)
        nws = MQ_QUANTIZE_WS_BYTES
        self.amax = torch.empty(3 * nws, dtype=torch.uint8, device=dev)
        self.qx = QTensor(c.H, c.W, c.Cin, c.N, fmt, MQ_ROLE_ACT, dev)
        self.qw = QTensor(c.Kh, c.Kw, c.Cout, c.Cin, fmt, MQ_ROLE_WEIGHT, dev)
        self.qg = QTensor(Ho, Wo, c.Cout, c.N, fmt, MQ_ROLE_GRAD, dev)
        self.y = torch.empty(Ho * Wo * c.Cout * c.N, **f32)
        self.gw = torch.empty(c.Kh * c.Kw * c.Cout * c.Cin, **f32)
        self.gx = torch.empty(c.H * c.W * c.Cin * c.N, **f32)
        self.ws = torch.empty(max(1, mq_wgrad_workspace_bytes(self.p)), dtype=torch.uint8,
                              device=dev)
        a0, a1, a2 = (self.amax[i * nws:(i + 1) * nws] for i in range(3))
        p = self.p
        self.ops: Dict[str, Callable[[int], None]] = OrderedDict([
            ("quantize_x", lambda s: mq_quantize_nchw(self.x, self.qx, MQ_RNE, 0, a0)),
            ("quantize_w", lambda s: mq_quantize_weight(self.w, self.qw, MQ_RNE, 0, a1)),
            ("quantize_g", lambda s: mq_quantize(self.gc, self.qg, MQ_SR,
                                                 self.sr_seed_base + s, a2)),
            ("conv_fwd", lambda s: mq_conv_fwd(p, self.qx, self.qw, self.y)),
            ("conv_wgrad", lambda s: mq_conv_wgrad(p, self.qg, self.qx, self.gw, self.ws)),
            ("conv_dgrad", lambda s: mq_conv_dgrad(p, self.qw, self.qg, self.gx)),
        ])

    def run(self, s: int = 0):
        for f in self.ops.values():
            f(s)

    def direct_calls(self, stream) -> Dict[str, Callable[[int], None]]:
        """The same calls with their C arguments marshalled once, for a fixed stream: each call
        is then one foreign-function call (the per-call cost that matters when launches are
        timed back to back). Each returns nothing and raises MQError on a failed status."""
        import ctypes
        from . import MQ_OK, MQError, _lib, _stream
        c = self.p
        hs = _stream(stream)
        P = lambda t: ctypes.c_void_p(t.data_ptr())
        conv = ctypes.byref(c)
        qx, qw, qg = self.qx.struct(), self.qw.struct(), self.qg.struct()
        self._keep = (qx, qw, qg, conv)
        bx, bw, bg = ctypes.byref(qx), ctypes.byref(qw), ctypes.byref(qg)
        a = [ctypes.c_void_p(self.amax.data_ptr() + MQ_QUANTIZE_WS_BYTES * i) for i in range(3)]
        wsb = MQ_QUANTIZE_WS_BYTES
        nws = self.ws.numel()
        L = _lib

        def chk(st, name):
            if st != MQ_OK:
                raise MQError(st, name)

        fixed = {
            "quantize_x": (L.mq_quantize_nchw, (P(self.x), bx, MQ_RNE, 0, a[0], wsb, 0, hs)),
            "quantize_w": (L.mq_quantize_weight, (P(self.w), bw, MQ_RNE, 0, a[1], wsb, hs)),
            "conv_fwd": (L.mq_conv_fwd, (conv, bx, bw, P(self.y), hs)),
            "conv_wgrad": (L.mq_conv_wgrad, (conv, bg, bx, P(self.gw), P(self.ws), nws, hs)),
            "conv_dgrad": (L.mq_conv_dgrad, (conv, bw, bg, P(self.gx), hs)),
        }
        out: Dict[str, Callable[[int], None]] = OrderedDict()
        for name in self.ops:
            if name == "quantize_g":
                gsrc = P(self.gc)
                out[name] = lambda s, f=L.mq_quantize, g=gsrc: chk(
                    f(g, bg, MQ_SR, (self.sr_seed_base + s) & (2 ** 64 - 1), a[2], wsb, 0, hs),
                    "mq_quantize")
            else:
                f, args = fixed[name]
                out[name] = lambda s, f=f, args=args, n=name: chk(f(*args), n)
        return out

    def outputs(self):
        """The tensors one pass writes (quantized codes, scales, T and the three GEMM results)."""
        out = []
        for q in (self.qx, self.qw, self.qg):
            out += [q.codes, q.scales, q.tscale]
        return out + [self.y, self.gw, self.gx]
