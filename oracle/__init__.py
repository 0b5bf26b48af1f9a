"""CPU oracle for microscaling-quantized convolution -- TEST INFRASTRUCTURE ONLY.

The plain, slow reference the GPU library is checked against (C in ``mq_oracle.c``, built with
gcc, loaded here with ctypes). Only the test-suite, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package. It shares no code with the GPU library;
both take their inputs from ``workloads``.

It follows the onedev.kr paper digest of MicroQonv ("합성곱 텐서 레이아웃 재배열로 ... MicroQonv"):
the channel-batch-first layout (section "How it works"), the 2-D reshapes, the three GEMMs and
the NVFP4 square-block recipe (section "How it differs"), NVFP6 (section "How it is used").

Parity pins: every function here is pinned by a ``-m "not gpu"`` test against something other
than itself (library casts, closed forms, invariants, brute force, torch float64 convolutions,
the published Philox4x32-10 known-answer vectors).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mq_oracle.c")
_LIB = os.path.join(_HERE, "libmq_oracle.so")
_CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-Wall"]

FP4, FP6 = 4, 6
RNE, SR = 0, 1

_lock = threading.Lock()
_lib = None


def build() -> str:
    """Compile the oracle with gcc (always recompiles). Returns the library path."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


class _Conv(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("N", "Cin", "H", "W", "Cout", "Kh", "Kw", "sh", "sw", "ph", "pw")]


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            L = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            i32, i64, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
            L.mqo_e2m1_value.restype = ctypes.c_double
            L.mqo_e2m3_value.restype = ctypes.c_double
            L.mqo_e4m3_value.restype = ctypes.c_double
            L.mqo_e4m3_cast.argtypes = [ctypes.c_float]
            L.mqo_quantize.argtypes = [P, i32, i32, i32, i32, i32, i32, u64, P, P, P]
            L.mqo_num_squares.restype = i64
            L.mqo_num_squares.argtypes = [i32, i32, i32, i32]
            L.mqo_packed_bytes.restype = i64
            L.mqo_packed_bytes.argtypes = [i64, i32]
            L.mqo_pack.argtypes = [P, i64, i32, P]
            L.mqo_unpack.argtypes = [P, i64, i32, P]
            L.mqo_dequant.argtypes = [P, P, ctypes.c_float, i32, i32, i32, i32, i32, P]
            for f in ("mqo_nchw_to_cbf", "mqo_cbf_to_nchw"):
                getattr(L, f).argtypes = [P, P, i32, i32, i32, i32]
            for f in ("mqo_oihw_to_tap_major", "mqo_tap_major_to_oihw"):
                getattr(L, f).argtypes = [P, P, i32, i32, i32, i32]
            for f in ("mqo_conv_fwd", "mqo_conv_wgrad", "mqo_conv_dgrad"):
                getattr(L, f).argtypes = [P, P, P, P, P]
            for f in ("mqo_conv_fwd_at", "mqo_conv_wgrad_at", "mqo_conv_dgrad_at"):
                getattr(L, f).argtypes = [P, P, P, P, i64, P, P]
            L.mqo_e4m3_cast_array.argtypes = [P, i64, P]
            L.mqo_elem_rne_array.argtypes = [i32, P, i64, P]
            L.mqo_elem_sr_array.argtypes = [i32, P, P, i64, P]
            L.mqo_sr_u16_array.argtypes = [u64, P, P, i64, P]
            L.mqo_sr_u16.restype = ctypes.c_uint32
            L.mqo_sr_u16.argtypes = [u64, i64, ctypes.c_int]
            L.mqo_philox4x32_10.argtypes = [P, P, P]
            _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ---- formats -------------------------------------------------------------------------------

def elem_value(fmt: int, code: int) -> float:
    return lib().mqo_e2m1_value(code) if fmt == FP4 else lib().mqo_e2m3_value(code)


def e4m3_value(code: int) -> float:
    return lib().mqo_e4m3_value(code)


def e4m3_cast(s: np.ndarray) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.empty(s.shape, np.uint8)
    lib().mqo_e4m3_cast_array(_p(s), s.size, _p(out))
    return out


def elem_rne(fmt: int, a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().mqo_elem_rne_array(fmt, _p(a), a.size, _p(out))
    return out


def elem_sr(fmt: int, a: np.ndarray, u16: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = np.ascontiguousarray(np.broadcast_to(u16, a.shape), dtype=np.uint32)
    out = np.empty(a.shape, np.uint8)
    lib().mqo_elem_sr_array(fmt, _p(a), _p(u), a.size, _p(out))
    return out


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, np.uint32)
    lib().mqo_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def sr_u16(seed: int, t: np.ndarray, e: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.int64)
    e = np.ascontiguousarray(np.broadcast_to(e, t.shape), dtype=np.int32)
    out = np.empty(t.shape, np.uint32)
    lib().mqo_sr_u16_array(seed, _p(t), _p(e), t.size, _p(out))
    return out


# ---- quantization --------------------------------------------------------------------------

def num_squares(shape) -> int:
    O0, O1, R, S = shape
    return O0 * O1 * ((R + 3) // 4) * ((S + 3) // 4)


def quantize(src: np.ndarray, fmt: int, rnd: int, seed: int = 0):
    """Quantize a float32 [O0][O1][R][S] tensor. Returns (codes [nsq,16] u8, scales [nsq] u8,
    T float32) with one code per byte, element e = (r%4)*4 + s%4 of square t."""
    src = np.ascontiguousarray(src, dtype=np.float32)
    assert src.ndim == 4
    nsq = num_squares(src.shape)
    codes = np.empty((nsq, 16), np.uint8)
    scales = np.empty(nsq, np.uint8)
    T = np.zeros(1, np.float32)
    rc = lib().mqo_quantize(_p(src), *src.shape, fmt, rnd, seed, _p(codes), _p(scales), _p(T))
    if rc:
        raise ValueError(f"mqo_quantize failed ({rc})")
    return codes, scales, T[0]


def pack(codes: np.ndarray, fmt: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    nsq = codes.shape[0]
    out = np.empty(lib().mqo_packed_bytes(nsq, fmt), np.uint8)
    lib().mqo_pack(_p(codes), nsq, fmt, _p(out))
    return out


def unpack(packed: np.ndarray, nsq: int, fmt: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    codes = np.empty((nsq, 16), np.uint8)
    lib().mqo_unpack(_p(packed), nsq, fmt, _p(codes))
    return codes


def dequant(codes, scales, T, shape, fmt: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty(shape, np.float64)
    lib().mqo_dequant(_p(codes), _p(scales), float(T), *shape, fmt, _p(out))
    return out


# ---- layouts -------------------------------------------------------------------------------

def nchw_to_cbf(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    N, C, H, W = x.shape
    out = np.empty((H, W, C, N), np.float32)
    lib().mqo_nchw_to_cbf(_p(x), _p(out), N, C, H, W)
    return out


def cbf_to_nchw(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    H, W, C, N = x.shape
    out = np.empty((N, C, H, W), np.float32)
    lib().mqo_cbf_to_nchw(_p(x), _p(out), N, C, H, W)
    return out


def oihw_to_tap_major(w: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.float32)
    Co, Ci, Kh, Kw = w.shape
    out = np.empty((Kh, Kw, Co, Ci), np.float32)
    lib().mqo_oihw_to_tap_major(_p(w), _p(out), Co, Ci, Kh, Kw)
    return out


def tap_major_to_oihw(w: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(w, dtype=np.float32)
    Kh, Kw, Co, Ci = w.shape
    out = np.empty((Co, Ci, Kh, Kw), np.float32)
    lib().mqo_tap_major_to_oihw(_p(w), _p(out), Co, Ci, Kh, Kw)
    return out


# ---- convolutions (double, explicit im2col) ------------------------------------------------

def _conv(p) -> _Conv:
    return _Conv(*[int(v) for v in p])


def out_hw(p):
    N, Cin, H, W, Cout, Kh, Kw, sh, sw, ph, pw = p
    return (H + 2 * ph - Kh) // sh + 1, (W + 2 * pw - Kw) // sw + 1


def conv_fwd(p, x: np.ndarray, w: np.ndarray):
    """p = (N,Cin,H,W,Cout,Kh,Kw,sh,sw,ph,pw); x [H][W][Cin][N], w [Kh][Kw][Cout][Cin] (double).
    Returns (y, yabs) as [Ho][Wo][Cout][N]."""
    N, Cin, H, W, Cout, Kh, Kw = p[:7]
    Ho, Wo = out_hw(p)
    x = np.ascontiguousarray(x, np.float64)
    w = np.ascontiguousarray(w, np.float64)
    assert x.shape == (H, W, Cin, N) and w.shape == (Kh, Kw, Cout, Cin)
    y = np.empty((Ho, Wo, Cout, N)); ya = np.empty_like(y)
    c = _conv(p)
    if lib().mqo_conv_fwd(ctypes.byref(c), _p(x), _p(w), _p(y), _p(ya)):
        raise RuntimeError("mqo_conv_fwd failed")
    return y, ya


def conv_wgrad(p, g: np.ndarray, x: np.ndarray):
    """g [Ho][Wo][Cout][N], x [H][W][Cin][N] -> (gw, gwabs) [Kh][Kw][Cout][Cin]."""
    N, Cin, H, W, Cout, Kh, Kw = p[:7]
    Ho, Wo = out_hw(p)
    g = np.ascontiguousarray(g, np.float64)
    x = np.ascontiguousarray(x, np.float64)
    assert g.shape == (Ho, Wo, Cout, N) and x.shape == (H, W, Cin, N)
    gw = np.empty((Kh, Kw, Cout, Cin)); ga = np.empty_like(gw)
    c = _conv(p)
    if lib().mqo_conv_wgrad(ctypes.byref(c), _p(g), _p(x), _p(gw), _p(ga)):
        raise RuntimeError("mqo_conv_wgrad failed")
    return gw, ga


def conv_dgrad(p, w: np.ndarray, g: np.ndarray):
    """w [Kh][Kw][Cout][Cin], g [Ho][Wo][Cout][N] -> (gx, gxabs) [H][W][Cin][N]."""
    N, Cin, H, W, Cout, Kh, Kw = p[:7]
    Ho, Wo = out_hw(p)
    w = np.ascontiguousarray(w, np.float64)
    g = np.ascontiguousarray(g, np.float64)
    assert w.shape == (Kh, Kw, Cout, Cin) and g.shape == (Ho, Wo, Cout, N)
    gx = np.empty((H, W, Cin, N)); ga = np.empty_like(gx)
    c = _conv(p)
    if lib().mqo_conv_dgrad(ctypes.byref(c), _p(w), _p(g), _p(gx), _p(ga)):
        raise RuntimeError("mqo_conv_dgrad failed")
    return gx, ga


def _at(fn, p, a, b, idx):
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(-1, 4)
    a = np.ascontiguousarray(a, np.float64)
    b = np.ascontiguousarray(b, np.float64)
    out = np.empty(idx.shape[0]); outa = np.empty(idx.shape[0])
    c = _conv(p)
    if fn(ctypes.byref(c), _p(a), _p(b), _p(idx), idx.shape[0], _p(out), _p(outa)):
        raise RuntimeError("oracle sampled conv failed")
    return out, outa


def conv_fwd_at(p, x, w, idx):
    """Sampled forward outputs at idx rows (ho, wo, co, n)."""
    return _at(lib().mqo_conv_fwd_at, p, x, w, idx)


def conv_wgrad_at(p, g, x, idx):
    """Sampled weight-gradient outputs at idx rows (kh, kw, co, ci)."""
    return _at(lib().mqo_conv_wgrad_at, p, g, x, idx)


def conv_dgrad_at(p, w, g, idx):
    """Sampled input-gradient outputs at idx rows (h, w, ci, n)."""
    return _at(lib().mqo_conv_dgrad_at, p, w, g, idx)


# ---- convenience: a whole tensor through quantize + dequantize ------------------------------

def quant_dequant(src: np.ndarray, fmt: int, rnd: int, seed: int = 0):
    """Returns (codes, scales, T, dequantized float64 tensor of src's shape)."""
    codes, scales, T = quantize(src, fmt, rnd, seed)
    return codes, scales, T, dequant(codes, scales, T, src.shape, fmt)
