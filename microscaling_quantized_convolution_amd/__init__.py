"""Python binding of the microscaling-quantized convolution library (libmq.so, gfx950).

Argument marshalling only: every step of the hot path runs in the library's HIP kernels. torch
supplies device memory and the current stream. The functions keep the C ABI's names
(``include/mq.h``) and raise :class:`MQError` on a non-OK status. If the library is not built
this module raises on import: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmq.so")

MQ_OK, MQ_ERR_ARG, MQ_ERR_SHAPE, MQ_ERR_UNSUPPORTED, MQ_ERR_WORKSPACE, MQ_ERR_LAUNCH = range(6)
MQ_NVFP4, MQ_NVFP6 = 4, 6
MQ_ROLE_ACT, MQ_ROLE_WEIGHT, MQ_ROLE_GRAD = 0, 1, 2
MQ_RNE, MQ_SR = 0, 1
MQ_QUANTIZE_WS_BYTES = 8192  # tensor-amax workspace (mq_quantize, relayouts)
MQ_QUANTIZE_AMAX_READY = 1   # mq_quantize flag: the workspace already holds this tensor's amax
MQ_SRC_DENSE, MQ_SRC_NCHW, MQ_SRC_OIHW = 0, 1, 2  # mq_quant_job.layout
MQ_QUANTIZE_BATCH_MAX = 4
MQ_NOALLOC_SCRATCH_BYTES = 32 << 20  # library-owned split-K scratch of mq_conv_backward_noalloc

EXPORTS = (
    "mq_status_str", "mq_codes_bytes", "mq_scales_bytes", "mq_relayout_cbf",
    "mq_relayout_weight", "mq_quantize", "mq_quantize_nchw", "mq_quantize_batch",
    "mq_quantize_weight", "mq_conv_fwd",
    "mq_wgrad_workspace_bytes",
    "mq_conv_wgrad", "mq_conv_dgrad", "mq_conv_backward", "mq_conv_backward_noalloc",
    "mq_conv_fwd_amax", "mq_conv_backward_amax",
)


class MQError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {_lib.mq_status_str(status).decode()}")
        self.status = status


class mq_qtensor(ctypes.Structure):
    _fields_ = [("o0", ctypes.c_int32), ("o1", ctypes.c_int32), ("r", ctypes.c_int32),
                ("s", ctypes.c_int32), ("fmt", ctypes.c_int32), ("role", ctypes.c_int32),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tscale", ctypes.c_void_p)]


class mq_quant_job(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("layout", ctypes.c_int32), ("rnd", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("flags", ctypes.c_uint32), ("dst", mq_qtensor),
                ("amax_ws", ctypes.c_void_p), ("amax_ws_bytes", ctypes.c_size_t)]


class mq_conv(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("N", "Cin", "H", "W", "Cout", "Kh", "Kw",
                                              "stride_h", "stride_w", "pad_h", "pad_w")]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          f"python microscaling_quantized_convolution_amd/_build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
    L.mq_status_str.restype = ctypes.c_char_p
    L.mq_status_str.argtypes = [ctypes.c_int]
    L.mq_codes_bytes.restype = sz
    L.mq_codes_bytes.argtypes = [i32] * 5
    L.mq_scales_bytes.restype = sz
    L.mq_scales_bytes.argtypes = [i32] * 4
    L.mq_relayout_cbf.argtypes = [P, P, i32, i32, i32, i32, i32, P, sz, P]
    L.mq_relayout_weight.argtypes = [P, P, i32, i32, i32, i32, i32, P, sz, P]
    L.mq_quantize.argtypes = [P, ctypes.POINTER(mq_qtensor), i32, u64, P, sz, ctypes.c_uint32, P]
    L.mq_quantize_nchw.argtypes = [P, ctypes.POINTER(mq_qtensor), i32, u64, P, sz,
                                   ctypes.c_uint32, P]
    L.mq_quantize_weight.argtypes = [P, ctypes.POINTER(mq_qtensor), i32, u64, P, sz, P]
    L.mq_quantize_batch.argtypes = [ctypes.POINTER(mq_quant_job), i32, P]
    L.mq_conv_fwd.argtypes = [ctypes.POINTER(mq_conv), ctypes.POINTER(mq_qtensor),
                              ctypes.POINTER(mq_qtensor), P, P]
    L.mq_wgrad_workspace_bytes.restype = sz
    L.mq_wgrad_workspace_bytes.argtypes = [ctypes.POINTER(mq_conv)]
    L.mq_conv_wgrad.argtypes = [ctypes.POINTER(mq_conv), ctypes.POINTER(mq_qtensor),
                                ctypes.POINTER(mq_qtensor), P, P, sz, P]
    L.mq_conv_dgrad.argtypes = [ctypes.POINTER(mq_conv), ctypes.POINTER(mq_qtensor),
                                ctypes.POINTER(mq_qtensor), P, P]
    L.mq_conv_backward.argtypes = [ctypes.POINTER(mq_conv), ctypes.POINTER(mq_qtensor),
                                   ctypes.POINTER(mq_qtensor), ctypes.POINTER(mq_qtensor), P, P,
                                   P, sz, P]
    L.mq_conv_backward_noalloc.argtypes = [ctypes.POINTER(mq_conv), ctypes.POINTER(mq_qtensor),
                                           ctypes.POINTER(mq_qtensor), ctypes.POINTER(mq_qtensor),
                                           P, P, P]
    L.mq_conv_fwd_amax.argtypes = [ctypes.POINTER(mq_conv), ctypes.POINTER(mq_qtensor),
                                   ctypes.POINTER(mq_qtensor), P, P, sz, P]
    L.mq_conv_backward_amax.argtypes = [ctypes.POINTER(mq_conv), ctypes.POINTER(mq_qtensor),
                                        ctypes.POINTER(mq_qtensor), ctypes.POINTER(mq_qtensor),
                                        P, P, P, sz, P, sz, P]
    for name in EXPORTS:
        getattr(L, name).restype = getattr(L, name).restype or ctypes.c_int
    return L


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(st: int, where: str):
    if st != MQ_OK:
        raise MQError(st, where)


ConvLike = Union[mq_conv, Sequence[int]]


def conv_struct(p: ConvLike) -> mq_conv:
    """(N, Cin, H, W, Cout, Kh, Kw, stride_h, stride_w, pad_h, pad_w) -> mq_conv."""
    return p if isinstance(p, mq_conv) else mq_conv(*[int(v) for v in p])


class QTensor:
    """Device buffers of one quantized tensor (codes, scales, tensor scale) and its shape."""

    def __init__(self, o0: int, o1: int, r: int, s: int, fmt: int, role: int,
                 device: Union[str, torch.device] = "cuda"):
        self.shape = (int(o0), int(o1), int(r), int(s))
        self.fmt, self.role = int(fmt), int(role)
        nc = _lib.mq_codes_bytes(*self.shape, self.fmt)
        ns = _lib.mq_scales_bytes(*self.shape)
        if nc == 0 or ns == 0:
            raise MQError(MQ_ERR_ARG, "QTensor")
        self.codes = torch.empty(nc, dtype=torch.uint8, device=device)
        self.scales = torch.empty(ns, dtype=torch.uint8, device=device)
        self.tscale = torch.empty(1, dtype=torch.float32, device=device)

    def struct(self) -> mq_qtensor:
        return mq_qtensor(*self.shape, self.fmt, self.role, self.codes.data_ptr(),
                          self.scales.data_ptr(), self.tscale.data_ptr())


def mq_codes_bytes(o0, o1, r, s, fmt) -> int:
    return int(_lib.mq_codes_bytes(o0, o1, r, s, fmt))


def mq_scales_bytes(o0, o1, r, s) -> int:
    return int(_lib.mq_scales_bytes(o0, o1, r, s))


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def mq_relayout_cbf(src: torch.Tensor, dst: torch.Tensor, N: int, C: int, H: int, W: int,
                    inverse: int = 0, amax_ws: Optional[torch.Tensor] = None, stream=None):
    _check(_lib.mq_relayout_cbf(_ptr(src), _ptr(dst), N, C, H, W, inverse, _ptr(amax_ws),
                                _nbytes(amax_ws), _stream(stream)), "mq_relayout_cbf")


def mq_relayout_weight(src: torch.Tensor, dst: torch.Tensor, Cout: int, Cin: int, Kh: int,
                       Kw: int, inverse: int = 0, amax_ws: Optional[torch.Tensor] = None,
                       stream=None):
    _check(_lib.mq_relayout_weight(_ptr(src), _ptr(dst), Cout, Cin, Kh, Kw, inverse,
                                   _ptr(amax_ws), _nbytes(amax_ws), _stream(stream)),
           "mq_relayout_weight")


def quantize_workspace(device: Union[str, torch.device] = "cuda") -> torch.Tensor:
    """Device scratch for mq_quantize's amax pass."""
    return torch.empty(MQ_QUANTIZE_WS_BYTES, dtype=torch.uint8, device=device)


def mq_quantize(src: torch.Tensor, dst: QTensor, rnd: int, seed: int, amax_ws: torch.Tensor,
                flags: int = 0, stream=None):
    q = dst.struct()
    _check(_lib.mq_quantize(_ptr(src), ctypes.byref(q), rnd, seed & (2 ** 64 - 1),
                            _ptr(amax_ws), _nbytes(amax_ws), flags, _stream(stream)),
           "mq_quantize")


def mq_quantize_nchw(src_nchw: torch.Tensor, dst: QTensor, rnd: int, seed: int,
                     amax_ws: torch.Tensor, flags: int = 0, stream=None):
    """NCHW fp32 activation / gradient -> quantized channel-batch-first tensor (same result as
    mq_relayout_cbf then mq_quantize, without the fp32 copy)."""
    q = dst.struct()
    _check(_lib.mq_quantize_nchw(_ptr(src_nchw), ctypes.byref(q), rnd, seed & (2 ** 64 - 1),
                                 _ptr(amax_ws), _nbytes(amax_ws), flags, _stream(stream)),
           "mq_quantize_nchw")


def quant_job(src: torch.Tensor, layout: int, dst: QTensor, rnd: int, seed: int,
              amax_ws: torch.Tensor, flags: int = 0) -> mq_quant_job:
    """One mq_quant_job (the caller keeps src, dst and amax_ws alive until the call is done)."""
    return mq_quant_job(ctypes.c_void_p(src.data_ptr()), layout, rnd, seed & (2 ** 64 - 1), flags,
                        dst.struct(), ctypes.c_void_p(amax_ws.data_ptr()), _nbytes(amax_ws))


def mq_quantize_batch(jobs: Sequence[mq_quant_job], stream=None):
    """Several tensors in one amax launch and one quantizing launch (see quant_job)."""
    arr = (mq_quant_job * len(jobs))(*jobs)
    _check(_lib.mq_quantize_batch(arr, len(jobs), _stream(stream)), "mq_quantize_batch")


def mq_quantize_weight(w_oihw: torch.Tensor, dst: QTensor, rnd: int, seed: int,
                       amax_ws: torch.Tensor, stream=None):
    """OIHW fp32 weight -> quantized tap-major weight (same result as mq_relayout_weight then
    mq_quantize, without the fp32 copy)."""
    q = dst.struct()
    _check(_lib.mq_quantize_weight(_ptr(w_oihw), ctypes.byref(q), rnd, seed & (2 ** 64 - 1),
                                   _ptr(amax_ws), _nbytes(amax_ws), _stream(stream)),
           "mq_quantize_weight")


def mq_conv_fwd(p: ConvLike, x: QTensor, w: QTensor, y: torch.Tensor, stream=None):
    c, qx, qw = conv_struct(p), x.struct(), w.struct()
    _check(_lib.mq_conv_fwd(ctypes.byref(c), ctypes.byref(qx), ctypes.byref(qw), _ptr(y),
                            _stream(stream)), "mq_conv_fwd")


def mq_wgrad_workspace_bytes(p: ConvLike) -> int:
    c = conv_struct(p)
    return int(_lib.mq_wgrad_workspace_bytes(ctypes.byref(c)))


def mq_conv_wgrad(p: ConvLike, gy: QTensor, x: QTensor, gw: torch.Tensor,
                  ws: Optional[torch.Tensor], stream=None):
    c, qg, qx = conv_struct(p), gy.struct(), x.struct()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.mq_conv_wgrad(ctypes.byref(c), ctypes.byref(qg), ctypes.byref(qx), _ptr(gw),
                              _ptr(ws), nbytes, _stream(stream)), "mq_conv_wgrad")


def mq_conv_dgrad(p: ConvLike, w: QTensor, gy: QTensor, gx: torch.Tensor, stream=None):
    c, qw, qg = conv_struct(p), w.struct(), gy.struct()
    _check(_lib.mq_conv_dgrad(ctypes.byref(c), ctypes.byref(qw), ctypes.byref(qg), _ptr(gx),
                              _stream(stream)), "mq_conv_dgrad")


def mq_conv_backward(p: ConvLike, w: QTensor, gy: QTensor, x: QTensor, gw: torch.Tensor,
                     gx: torch.Tensor, ws: torch.Tensor, stream=None):
    """Both gradients (G_W as mq_conv_wgrad, G_X as mq_conv_dgrad) in one call."""
    c, qw, qg, qx = conv_struct(p), w.struct(), gy.struct(), x.struct()
    _check(_lib.mq_conv_backward(ctypes.byref(c), ctypes.byref(qw), ctypes.byref(qg),
                                 ctypes.byref(qx), _ptr(gw), _ptr(gx), _ptr(ws), _nbytes(ws),
                                 _stream(stream)), "mq_conv_backward")


def mq_conv_backward_noalloc(p: ConvLike, w: QTensor, gy: QTensor, x: QTensor,
                             gw: torch.Tensor, gx: torch.Tensor, stream=None):
    """mq_conv_backward without a workspace argument: the split-K partials live in the
    library's own device array (for callers that cannot allocate)."""
    c, qw, qg, qx = conv_struct(p), w.struct(), gy.struct(), x.struct()
    _check(_lib.mq_conv_backward_noalloc(ctypes.byref(c), ctypes.byref(qw), ctypes.byref(qg),
                                         ctypes.byref(qx), _ptr(gw), _ptr(gx), _stream(stream)),
           "mq_conv_backward_noalloc")


def mq_conv_fwd_amax(p: ConvLike, x: QTensor, w: QTensor, y: torch.Tensor,
                     amax_ws: torch.Tensor, stream=None):
    """mq_conv_fwd, plus the partial maxima of |Y| in amax_ws (for MQ_QUANTIZE_AMAX_READY)."""
    c, qx, qw = conv_struct(p), x.struct(), w.struct()
    _check(_lib.mq_conv_fwd_amax(ctypes.byref(c), ctypes.byref(qx), ctypes.byref(qw), _ptr(y),
                                 _ptr(amax_ws), _nbytes(amax_ws), _stream(stream)),
           "mq_conv_fwd_amax")


def mq_conv_backward_amax(p: ConvLike, w: QTensor, gy: QTensor, x: QTensor, gw: torch.Tensor,
                          gx: torch.Tensor, ws: torch.Tensor, gx_amax_ws: torch.Tensor,
                          stream=None):
    """mq_conv_backward, plus the partial maxima of |G_X| in gx_amax_ws."""
    c, qw, qg, qx = conv_struct(p), w.struct(), gy.struct(), x.struct()
    _check(_lib.mq_conv_backward_amax(ctypes.byref(c), ctypes.byref(qw), ctypes.byref(qg),
                                      ctypes.byref(qx), _ptr(gw), _ptr(gx), _ptr(ws), _nbytes(ws),
                                      _ptr(gx_amax_ws), _nbytes(gx_amax_ws), _stream(stream)),
           "mq_conv_backward_amax")


def out_hw(p: ConvLike) -> Tuple[int, int]:
    c = conv_struct(p)
    return ((c.H + 2 * c.pad_h - c.Kh) // c.stride_h + 1,
            (c.W + 2 * c.pad_w - c.Kw) // c.stride_w + 1)
