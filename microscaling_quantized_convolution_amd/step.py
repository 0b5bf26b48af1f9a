"""One convolution layer's pass through the quantize-once path, as a list of library calls.

Device buffers for one layer (fp32 inputs, their channel-batch-first copies, the three quantized
tensors, the outputs and the weight-gradient workspace) and the calls of one pass, in order:

  quantize_xw  X NCHW -> quantized channel-batch-first squares and W OIHW -> quantized
               tap-major squares (both round to nearest), one batched call
  quantize_g   G_Y (stochastic, seed per pass)
  conv_fwd     Y = W.X'
  conv_backward  G_W = G_Y.X'^T and G_X = W^T.G_Y in one call (mq_conv_backward: the weight
               gradient's split sum rides in the input-gradient launch)

conv_wgrad and conv_dgrad, the two gradients as calls of their own, stay available in
`parts` (same results, bit for bit), next to the variants that hand the next quantization its
tensor amax: conv_fwd_amax and conv_backward_amax write the partial maxima of Y and G_X from
their epilogues, and quantize_g_ready quantizes G_Y from partial maxima already in its workspace
(as a producer's epilogue would leave them; the pass's own quantize_g writes them there).

X and W are quantized together, as a layer's forward pass does (mq_quantize_batch: one amax
launch over both, then one launch that reads X in NCHW and W in OIHW order and writes their
squares; no fp32 channel-batch-first or tap-major copy). G_Y, which only exists in the backward
pass, is quantized on its own, with its own amax pass.

G_Y is taken as already channel-batch-first (it is the next layer's input-gradient output).
Every call goes through the C ABI on the current stream; nothing here computes.
"""
from __future__ import annotations

from collections import OrderedDict
from typing import Callable, Dict

import torch

from . import (MQ_QUANTIZE_AMAX_READY, MQ_QUANTIZE_WS_BYTES, MQ_ROLE_ACT, MQ_ROLE_GRAD,
               MQ_ROLE_WEIGHT, MQ_RNE, MQ_SR, MQ_SRC_NCHW, MQ_SRC_OIHW, QTensor, conv_struct,
               mq_conv_backward, mq_conv_backward_amax, mq_conv_dgrad, mq_conv_fwd,
               mq_conv_fwd_amax, mq_conv_wgrad, mq_quant_job, mq_quantize, mq_quantize_batch,
               mq_wgrad_workspace_bytes, out_hw, quant_job)


class LayerStep:
    """conv = (N, Cin, H, W, Cout, Kh, Kw, sh, sw, ph, pw); x: NCHW, w: OIHW, g_cbf: G_Y in
    [Ho][Wo][Cout][N] order (all fp32 device tensors, any shape with the right element count)."""

    def __init__(self, conv, fmt: int, x: torch.Tensor, w: torch.Tensor, g_cbf: torch.Tensor,
                 sr_seed_base: int = 1, seed_stride: int = 1):
        self.p = conv_struct(conv)
        c = self.p
        dev = x.device
        Ho, Wo = out_hw(c)
        # G_Y's stochastic-rounding seed in pass s: sr_seed_base + seed_stride * s (a network of
        # L layers with bases 1..L and stride L gives every (layer, pass) its own seed)
        self.fmt, self.sr_seed_base, self.seed_stride = int(fmt), int(sr_seed_base), int(seed_stride)
        self.x, self.w, self.gc = x, w, g_cbf
        f32 = dict(dtype=torch.float32, device=dev)
        nws = MQ_QUANTIZE_WS_BYTES
        # amax workspaces: X, W, G_Y, and the epilogue partials of Y and G_X
        self.amax = torch.empty(5 * nws, dtype=torch.uint8, device=dev)
        self.qx = QTensor(c.H, c.W, c.Cin, c.N, fmt, MQ_ROLE_ACT, dev)
        self.qw = QTensor(c.Kh, c.Kw, c.Cout, c.Cin, fmt, MQ_ROLE_WEIGHT, dev)
        self.qg = QTensor(Ho, Wo, c.Cout, c.N, fmt, MQ_ROLE_GRAD, dev)
        self.y = torch.empty(Ho * Wo * c.Cout * c.N, **f32)
        self.gw = torch.empty(c.Kh * c.Kw * c.Cout * c.Cin, **f32)
        self.gx = torch.empty(c.H * c.W * c.Cin * c.N, **f32)
        self.ws = torch.empty(max(1, mq_wgrad_workspace_bytes(self.p)), dtype=torch.uint8,
                              device=dev)
        a0, a1, a2, a3, a4 = (self.amax[i * nws:(i + 1) * nws] for i in range(5))
        self._a0 = a0
        p = self.p
        self.xw_jobs = [quant_job(self.x, MQ_SRC_NCHW, self.qx, MQ_RNE, 0, a0),
                        quant_job(self.w, MQ_SRC_OIHW, self.qw, MQ_RNE, 0, a1)]
        self.ops: Dict[str, Callable[[int], None]] = OrderedDict([
            ("quantize_xw", lambda s: mq_quantize_batch(self.xw_jobs)),
            ("quantize_g", lambda s: mq_quantize(self.gc, self.qg, MQ_SR, self.seed(s), a2)),
            ("conv_fwd", lambda s: mq_conv_fwd(p, self.qx, self.qw, self.y)),
            ("conv_backward", lambda s: mq_conv_backward(p, self.qw, self.qg, self.qx, self.gw,
                                                         self.gx, self.ws)),
        ])
        self.parts: Dict[str, Callable[[int], None]] = OrderedDict([
            ("conv_wgrad", lambda s: mq_conv_wgrad(p, self.qg, self.qx, self.gw, self.ws)),
            ("conv_dgrad", lambda s: mq_conv_dgrad(p, self.qw, self.qg, self.gx)),
            ("conv_fwd_amax", lambda s: mq_conv_fwd_amax(p, self.qx, self.qw, self.y, a3)),
            ("conv_backward_amax", lambda s: mq_conv_backward_amax(
                p, self.qw, self.qg, self.qx, self.gw, self.gx, self.ws, a4)),
            ("quantize_g_ready", lambda s: mq_quantize(self.gc, self.qg, MQ_SR, self.seed(s), a2,
                                                       MQ_QUANTIZE_AMAX_READY)),
        ])

    def seed(self, s: int) -> int:
        """G_Y's stochastic-rounding seed in pass s."""
        return (self.sr_seed_base + self.seed_stride * s) & (2 ** 64 - 1)

    def run(self, s: int = 0):
        for f in self.ops.values():
            f(s)

    def direct_calls(self, stream) -> Dict[str, Callable[[int], None]]:
        """The same calls with their C arguments marshalled once, for a fixed stream: each call
        is then one foreign-function call (the per-call cost that matters when launches are
        timed back to back): the ops of a pass, then the two gradients as calls of their own.
        Each returns nothing and raises MQError on a failed status."""
        import ctypes
        from . import MQ_OK, MQError, _lib, _stream
        c = self.p
        hs = _stream(stream)
        P = lambda t: ctypes.c_void_p(t.data_ptr())
        conv = ctypes.byref(c)
        qx, qw, qg = self.qx.struct(), self.qw.struct(), self.qg.struct()
        self._keep = (qx, qw, qg, conv)
        bx, bw, bg = ctypes.byref(qx), ctypes.byref(qw), ctypes.byref(qg)
        a = [ctypes.c_void_p(self.amax.data_ptr() + MQ_QUANTIZE_WS_BYTES * i) for i in range(5)]
        wsb = MQ_QUANTIZE_WS_BYTES
        nws = self.ws.numel()
        L = _lib

        def chk(st, name):
            if st != MQ_OK:
                raise MQError(st, name)

        jobs = (mq_quant_job * 2)(*self.xw_jobs)
        self._keep = self._keep + (jobs,)
        fixed = {
            "quantize_xw": (L.mq_quantize_batch, (jobs, 2, hs)),
            "conv_fwd": (L.mq_conv_fwd, (conv, bx, bw, P(self.y), hs)),
            "conv_backward": (L.mq_conv_backward, (conv, bw, bg, bx, P(self.gw), P(self.gx),
                                                   P(self.ws), nws, hs)),
            "conv_wgrad": (L.mq_conv_wgrad, (conv, bg, bx, P(self.gw), P(self.ws), nws, hs)),
            "conv_dgrad": (L.mq_conv_dgrad, (conv, bw, bg, P(self.gx), hs)),
            "conv_fwd_amax": (L.mq_conv_fwd_amax, (conv, bx, bw, P(self.y), a[3], wsb, hs)),
            "conv_backward_amax": (L.mq_conv_backward_amax, (conv, bw, bg, bx, P(self.gw),
                                                             P(self.gx), P(self.ws), nws, a[4],
                                                             wsb, hs)),
        }
        out: Dict[str, Callable[[int], None]] = OrderedDict()
        for name in list(self.ops) + list(self.parts):
            if name in ("quantize_g", "quantize_g_ready"):
                gsrc = P(self.gc)
                fl = MQ_QUANTIZE_AMAX_READY if name == "quantize_g_ready" else 0
                out[name] = lambda s, f=L.mq_quantize, g=gsrc, fl=fl: chk(
                    f(g, bg, MQ_SR, self.seed(s), a[2], wsb, fl, hs),
                    "mq_quantize")
            else:
                f, args = fixed[name]
                out[name] = lambda s, f=f, args=args, n=name: chk(f(*args), n)
        return out

    def inference_calls(self, stream) -> Dict[str, Callable[[int], None]]:
        """The forward pass with the weight already quantized: X alone (mq_quantize_nchw), then
        the forward GEMM, as direct foreign-function calls on a fixed stream."""
        import ctypes
        from . import MQ_OK, MQError, _lib, _stream
        hs = _stream(stream)
        qx, qw = self.qx.struct(), self.qw.struct()
        conv = ctypes.byref(self.p)
        self._keep_inf = (qx, qw, conv)
        a0 = ctypes.c_void_p(self._a0.data_ptr())
        calls = {
            "quantize_x": (_lib.mq_quantize_nchw, (ctypes.c_void_p(self.x.data_ptr()),
                                                   ctypes.byref(qx), MQ_RNE, 0, a0,
                                                   MQ_QUANTIZE_WS_BYTES, 0, hs)),
            "conv_fwd": (_lib.mq_conv_fwd, (conv, ctypes.byref(qx), ctypes.byref(qw),
                                            ctypes.c_void_p(self.y.data_ptr()), hs)),
        }
        out: Dict[str, Callable[[int], None]] = OrderedDict()
        for name, (f, args) in calls.items():
            def call(s, f=f, args=args, n=name):
                st = f(*args)
                if st != MQ_OK:
                    raise MQError(st, n)
            out[name] = call
        return out

    def outputs(self):
        """The tensors one pass writes (quantized codes, scales, T and the three GEMM results)."""
        out = []
        for q in (self.qx, self.qw, self.qg):
            out += [q.codes, q.scales, q.tscale]
        return out + [self.y, self.gw, self.gx]
