"""The C-ABI library loads on the CPU, exports every symbol include/mq.h declares, and validates
arguments on the host (no compute call is made here: there is no GPU)."""
import ctypes
import os
import re

import pytest

import microscaling_quantized_convolution_amd as mq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "mq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mq_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 10
    assert set(names) == set(mq.EXPORTS)
    lib = ctypes.CDLL(mq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for st in range(6):
        s = mq.lib().mq_status_str(st).decode()
        assert s.startswith("MQ_")
    assert mq.lib().mq_status_str(99).decode() == "unknown mq_status"


def test_size_queries():
    # 2*3*ceil(5/4)*ceil(6/4) = 24 squares
    assert mq.mq_scales_bytes(2, 3, 5, 6) == 24
    assert mq.mq_codes_bytes(2, 3, 5, 6, mq.MQ_NVFP4) == 24 * 8
    assert mq.mq_codes_bytes(2, 3, 5, 6, mq.MQ_NVFP6) == 24 * 12
    assert mq.mq_codes_bytes(2, 3, 5, 6, 5) == 0
    assert mq.mq_codes_bytes(0, 3, 5, 6, mq.MQ_NVFP4) == 0
    assert mq.mq_scales_bytes(1, 1, -1, 1) == 0
    assert mq.mq_wgrad_workspace_bytes((32, 64, 56, 56, 64, 3, 3, 1, 1, 1, 1)) > 0
    assert mq.mq_wgrad_workspace_bytes((32, 64, 2, 2, 64, 3, 3, 1, 1, 0, 0)) == 0


def _fake_q(shape, fmt=mq.MQ_NVFP4, role=mq.MQ_ROLE_ACT, null=False):
    p = 0 if null else 0x1000
    return mq.mq_qtensor(*shape, fmt, role, p, p, p)


def test_validation_errors_without_gpu():
    L = mq.lib()
    conv = mq.conv_struct((2, 16, 8, 8, 16, 3, 3, 1, 1, 0, 0))
    x = _fake_q((8, 8, 16, 2))
    w = _fake_q((3, 3, 16, 16), role=mq.MQ_ROLE_WEIGHT)
    g = _fake_q((6, 6, 16, 2), role=mq.MQ_ROLE_GRAD)
    y = ctypes.c_void_p(0x2000)
    s0 = ctypes.c_void_p(0)
    # null pointers / bad enums -> MQ_ERR_ARG
    ws = mq.MQ_QUANTIZE_WS_BYTES
    assert L.mq_relayout_cbf(None, y, 1, 1, 1, 1, 0, None, 0, s0) == mq.MQ_ERR_ARG
    assert L.mq_relayout_cbf(y, y, 1, 0, 1, 1, 0, None, 0, s0) == mq.MQ_ERR_ARG
    assert L.mq_relayout_cbf(y, y, 1, 1, 1, 1, 2, None, 0, s0) == mq.MQ_ERR_ARG
    assert L.mq_relayout_cbf(y, y, 1, 1, 1, 1, 0, y, ws - 1, s0) == mq.MQ_ERR_WORKSPACE
    assert L.mq_relayout_cbf(y, y, 1, 1, 1, 1, 0, ctypes.c_void_p(0x2002), ws, s0) == mq.MQ_ERR_ARG
    assert L.mq_relayout_weight(y, None, 1, 1, 1, 1, 0, None, 0, s0) == mq.MQ_ERR_ARG
    assert L.mq_relayout_weight(y, y, 1, 1, 1, 1, 0, y, 16, s0) == mq.MQ_ERR_WORKSPACE
    assert L.mq_quantize(y, ctypes.byref(x), 2, 0, y, ws, 0, s0) == mq.MQ_ERR_ARG
    assert L.mq_quantize(y, ctypes.byref(x), 0, 0, y, ws, 2, s0) == mq.MQ_ERR_ARG  # unknown flag
    assert L.mq_quantize(y, ctypes.byref(x), 0, 0, None, ws, 0, s0) == mq.MQ_ERR_WORKSPACE
    assert L.mq_quantize(y, ctypes.byref(x), 0, 0, y, ws - 4, 0, s0) == mq.MQ_ERR_WORKSPACE
    bad = _fake_q((8, 8, 16, 2), fmt=5)
    assert L.mq_quantize(y, ctypes.byref(bad), 0, 0, y, ws, 0, s0) == mq.MQ_ERR_ARG
    nul = _fake_q((8, 8, 16, 2), null=True)
    assert L.mq_quantize(y, ctypes.byref(nul), 0, 0, y, ws, 0, s0) == mq.MQ_ERR_ARG
    # weights straight from OIHW
    assert L.mq_quantize_weight(None, ctypes.byref(w), 0, 0, y, ws, s0) == mq.MQ_ERR_ARG
    assert L.mq_quantize_weight(y, ctypes.byref(w), 3, 0, y, ws, s0) == mq.MQ_ERR_ARG
    assert L.mq_quantize_weight(y, ctypes.byref(x), 0, 0, y, ws, s0) == mq.MQ_ERR_SHAPE  # role
    assert L.mq_quantize_weight(y, ctypes.byref(w), 0, 0, None, ws, s0) == mq.MQ_ERR_WORKSPACE
    assert L.mq_quantize_weight(y, ctypes.byref(w), 0, 0, y, ws - 1, s0) == mq.MQ_ERR_WORKSPACE
    assert L.mq_quantize_weight(y, ctypes.byref(w), 0, 0, ctypes.c_void_p(0x2002), ws, s0) == mq.MQ_ERR_ARG
    # NCHW activations / gradients straight to the quantized layout
    assert L.mq_quantize_nchw(None, ctypes.byref(x), 0, 0, y, ws, 0, s0) == mq.MQ_ERR_ARG
    assert L.mq_quantize_nchw(y, ctypes.byref(x), 2, 0, y, ws, 0, s0) == mq.MQ_ERR_ARG
    assert L.mq_quantize_nchw(y, ctypes.byref(x), 0, 0, y, ws, 4, s0) == mq.MQ_ERR_ARG  # flag
    assert L.mq_quantize_nchw(y, ctypes.byref(w), 0, 0, y, ws, 0, s0) == mq.MQ_ERR_SHAPE  # role
    assert L.mq_quantize_nchw(y, ctypes.byref(g), 1, 0, None, ws, 0, s0) == mq.MQ_ERR_WORKSPACE
    assert L.mq_quantize_nchw(y, ctypes.byref(g), 1, 0, y, ws - 4, 0, s0) == mq.MQ_ERR_WORKSPACE
    assert L.mq_quantize_nchw(y, ctypes.byref(g), 1, 0, ctypes.c_void_p(0x2002), ws, 0, s0) == mq.MQ_ERR_ARG
    assert L.mq_quantize_nchw(y, ctypes.byref(bad), 0, 0, y, ws, 0, s0) == mq.MQ_ERR_ARG
    big = _fake_q((1024, 1024, 32, 16))  # 2^31 source bytes once padded
    assert L.mq_quantize_nchw(y, ctypes.byref(big), 0, 0, y, ws, 0, s0) == mq.MQ_ERR_UNSUPPORTED
    # batched quantization
    x6 = _fake_q((8, 8, 16, 2), fmt=mq.MQ_NVFP6)

    def job(src=y, layout=mq.MQ_SRC_NCHW, dst=x, rnd=0, flags=0, ws_ptr=0x3000, nbytes=ws):
        return mq.mq_quant_job(src, layout, rnd, 0, flags, dst, ws_ptr, nbytes)

    def batch(*js):
        arr = (mq.mq_quant_job * max(1, len(js)))(*js)
        return L.mq_quantize_batch(arr, len(js), s0)
    assert L.mq_quantize_batch(None, 1, s0) == mq.MQ_ERR_ARG
    assert batch() == mq.MQ_ERR_ARG  # no jobs
    assert batch(*[job(ws_ptr=0x3000 + 0x4000 * i) for i in range(5)]) == mq.MQ_ERR_UNSUPPORTED
    assert batch(job(src=None)) == mq.MQ_ERR_ARG
    assert batch(job(layout=3)) == mq.MQ_ERR_ARG
    assert batch(job(rnd=2)) == mq.MQ_ERR_ARG
    assert batch(job(flags=2)) == mq.MQ_ERR_ARG
    assert batch(job(nbytes=ws - 4)) == mq.MQ_ERR_WORKSPACE
    assert batch(job(ws_ptr=0)) == mq.MQ_ERR_WORKSPACE
    assert batch(job(ws_ptr=0x3002)) == mq.MQ_ERR_ARG
    assert batch(job(), job(dst=g, rnd=1)) == mq.MQ_ERR_ARG  # shared workspace
    assert batch(job(), job(dst=x6, ws_ptr=0x8000)) == mq.MQ_ERR_SHAPE  # formats differ
    assert batch(job(dst=w)) == mq.MQ_ERR_SHAPE  # NCHW source, weight role
    assert batch(job(layout=mq.MQ_SRC_OIHW, dst=x)) == mq.MQ_ERR_SHAPE  # OIHW, not a weight
    assert batch(job(dst=_fake_q((1024, 1024, 32, 16)))) == mq.MQ_ERR_UNSUPPORTED
    # misaligned codes (16 B) or scales (4 B) -> MQ_ERR_ARG
    mis = mq.mq_qtensor(8, 8, 16, 2, mq.MQ_NVFP4, mq.MQ_ROLE_ACT, 0x1008, 0x1000, 0x1000)
    assert L.mq_quantize(y, ctypes.byref(mis), 0, 0, y, ws, 0, s0) == mq.MQ_ERR_ARG
    mis = mq.mq_qtensor(8, 8, 16, 2, mq.MQ_NVFP4, mq.MQ_ROLE_ACT, 0x1000, 0x1002, 0x1000)
    assert L.mq_conv_fwd(ctypes.byref(conv), ctypes.byref(mis), ctypes.byref(w), y, s0) == mq.MQ_ERR_ARG
    assert L.mq_conv_fwd(ctypes.byref(conv), ctypes.byref(x), ctypes.byref(w), None, s0) == mq.MQ_ERR_ARG
    # shape / role / format mismatches -> MQ_ERR_SHAPE
    assert L.mq_conv_fwd(ctypes.byref(conv), ctypes.byref(w), ctypes.byref(x), y, s0) == mq.MQ_ERR_SHAPE
    x6 = _fake_q((8, 8, 16, 2), fmt=mq.MQ_NVFP6)
    assert L.mq_conv_fwd(ctypes.byref(conv), ctypes.byref(x6), ctypes.byref(w), y, s0) == mq.MQ_ERR_SHAPE
    xw = _fake_q((8, 8, 16, 3))
    assert L.mq_conv_fwd(ctypes.byref(conv), ctypes.byref(xw), ctypes.byref(w), y, s0) == mq.MQ_ERR_SHAPE
    assert L.mq_conv_dgrad(ctypes.byref(conv), ctypes.byref(w), ctypes.byref(x), y, s0) == mq.MQ_ERR_SHAPE
    g7 = _fake_q((7, 6, 16, 2), role=mq.MQ_ROLE_GRAD)
    assert L.mq_conv_dgrad(ctypes.byref(conv), ctypes.byref(w), ctypes.byref(g7), y, s0) == mq.MQ_ERR_SHAPE
    # workspace missing or small -> MQ_ERR_WORKSPACE
    assert L.mq_conv_wgrad(ctypes.byref(conv), ctypes.byref(g), ctypes.byref(x), y, None, 0, s0) == mq.MQ_ERR_WORKSPACE
    need = L.mq_wgrad_workspace_bytes(ctypes.byref(conv))
    assert L.mq_conv_wgrad(ctypes.byref(conv), ctypes.byref(g), ctypes.byref(x), y, y, need - 1, s0) == mq.MQ_ERR_WORKSPACE
    # both gradients in one call
    bw = lambda *a: L.mq_conv_backward(ctypes.byref(conv), *a, s0)
    assert bw(ctypes.byref(w), ctypes.byref(g), ctypes.byref(x), y, None, y, need, ) == mq.MQ_ERR_ARG
    assert bw(ctypes.byref(w), ctypes.byref(g), ctypes.byref(x), None, y, y, need) == mq.MQ_ERR_ARG
    assert bw(ctypes.byref(x), ctypes.byref(g), ctypes.byref(x), y, y, y, need) == mq.MQ_ERR_SHAPE
    assert bw(ctypes.byref(w), ctypes.byref(g7), ctypes.byref(x), y, y, y, need) == mq.MQ_ERR_SHAPE
    assert bw(ctypes.byref(w), ctypes.byref(g), ctypes.byref(x6), y, y, y, need) == mq.MQ_ERR_SHAPE
    assert bw(ctypes.byref(w), ctypes.byref(g), ctypes.byref(x), y, y, None, 0) == mq.MQ_ERR_WORKSPACE
    assert bw(ctypes.byref(w), ctypes.byref(g), ctypes.byref(x), y, y, y, need - 1) == mq.MQ_ERR_WORKSPACE
    # an impossible convolution -> MQ_ERR_ARG
    badc = mq.conv_struct((2, 16, 2, 2, 16, 3, 3, 1, 1, 0, 0))
    assert L.mq_conv_fwd(ctypes.byref(badc), ctypes.byref(x), ctypes.byref(w), y, s0) == mq.MQ_ERR_ARG
    badc = mq.conv_struct((2, 16, 8, 8, 16, 3, 3, 0, 1, 0, 0))
    assert L.mq_conv_fwd(ctypes.byref(badc), ctypes.byref(x), ctypes.byref(w), y, s0) == mq.MQ_ERR_ARG


def test_header_constants_match_binding():
    import re
    hdr = open(os.path.join(ROOT, "include", "mq.h")).read()
    m = re.search(r"#define MQ_QUANTIZE_WS_BYTES (\d+)", hdr)
    assert m and int(m.group(1)) == mq.MQ_QUANTIZE_WS_BYTES
    m = re.search(r"#define MQ_QUANTIZE_AMAX_READY (\d+)u", hdr)
    assert m and int(m.group(1)) == mq.MQ_QUANTIZE_AMAX_READY


def test_backward_noalloc_validation_without_gpu():
    """mq_conv_backward_noalloc checks its arguments on the host before it touches the device:
    the statuses of mq_conv_backward, and MQ_ERR_UNSUPPORTED for a convolution whose split-K
    partials exceed the library's own array."""
    L = mq.lib()
    conv = mq.conv_struct((2, 16, 8, 8, 16, 3, 3, 1, 1, 0, 0))
    x = _fake_q((8, 8, 16, 2))
    w = _fake_q((3, 3, 16, 16), role=mq.MQ_ROLE_WEIGHT)
    g = _fake_q((6, 6, 16, 2), role=mq.MQ_ROLE_GRAD)
    g7 = _fake_q((7, 6, 16, 2), role=mq.MQ_ROLE_GRAD)
    y = ctypes.c_void_p(0x2000)
    s0 = ctypes.c_void_p(0)
    na = lambda c, *a: L.mq_conv_backward_noalloc(ctypes.byref(c), *a, s0)
    assert L.mq_conv_backward_noalloc(None, ctypes.byref(w), ctypes.byref(g), ctypes.byref(x),
                                      y, y, s0) == mq.MQ_ERR_ARG
    assert na(conv, ctypes.byref(w), ctypes.byref(g), ctypes.byref(x), None, y) == mq.MQ_ERR_ARG
    assert na(conv, ctypes.byref(w), ctypes.byref(g), ctypes.byref(x), y, None) == mq.MQ_ERR_ARG
    assert na(conv, ctypes.byref(x), ctypes.byref(g), ctypes.byref(x), y, y) == mq.MQ_ERR_SHAPE
    assert na(conv, ctypes.byref(w), ctypes.byref(g7), ctypes.byref(x), y, y) == mq.MQ_ERR_SHAPE
    # a 5x5 512->512 convolution at N=128 on 14x14 needs more partial sums than the array holds
    big = (128, 512, 14, 14, 512, 5, 5, 1, 1, 2, 2)
    assert mq.mq_wgrad_workspace_bytes(big) > mq.MQ_NOALLOC_SCRATCH_BYTES
    bc = mq.conv_struct(big)
    bx = _fake_q((14, 14, 512, 128))
    bw_ = _fake_q((5, 5, 512, 512), role=mq.MQ_ROLE_WEIGHT)
    bg = _fake_q((14, 14, 512, 128), role=mq.MQ_ROLE_GRAD)
    assert na(bc, ctypes.byref(bw_), ctypes.byref(bg), ctypes.byref(bx), y, y) == \
        mq.MQ_ERR_UNSUPPORTED
    # every workload layer fits
    import workloads
    for l in (workloads.config2() + workloads.config3() + workloads.config4() +
              workloads.config5()):
        assert 0 < mq.mq_wgrad_workspace_bytes(l.conv_tuple()) <= mq.MQ_NOALLOC_SCRATCH_BYTES


def test_noalloc_scratch_size_matches_binding():
    hdr = open(os.path.join(ROOT, "include", "mq.h")).read()
    m = re.search(r"#define MQ_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == mq.MQ_NOALLOC_SCRATCH_BYTES


def test_fused_amax_validation_without_gpu():
    """mq_conv_fwd_amax and mq_conv_backward_amax reject a missing, short or misaligned amax
    workspace, and the shape errors of the plain calls, on the host before any launch."""
    L = mq.lib()
    conv = mq.conv_struct((2, 16, 8, 8, 16, 3, 3, 1, 1, 0, 0))
    x = _fake_q((8, 8, 16, 2))
    w = _fake_q((3, 3, 16, 16), role=mq.MQ_ROLE_WEIGHT)
    g = _fake_q((6, 6, 16, 2), role=mq.MQ_ROLE_GRAD)
    y = ctypes.c_void_p(0x2000)
    s0 = ctypes.c_void_p(0)
    ws = mq.MQ_QUANTIZE_WS_BYTES
    wgb = mq.mq_wgrad_workspace_bytes((2, 16, 8, 8, 16, 3, 3, 1, 1, 0, 0))
    fa = lambda *a: L.mq_conv_fwd_amax(ctypes.byref(conv), *a, s0)
    ba = lambda *a: L.mq_conv_backward_amax(ctypes.byref(conv), *a, s0)
    X, W, G = ctypes.byref(x), ctypes.byref(w), ctypes.byref(g)
    assert fa(X, W, y, None, ws) == mq.MQ_ERR_WORKSPACE
    assert fa(X, W, y, y, ws - 4) == mq.MQ_ERR_WORKSPACE
    assert fa(X, W, y, ctypes.c_void_p(0x3002), ws) == mq.MQ_ERR_ARG
    assert fa(X, W, None, y, ws) == mq.MQ_ERR_ARG
    assert fa(G, W, y, y, ws) == mq.MQ_ERR_SHAPE  # a gradient where X belongs
    assert L.mq_conv_fwd_amax(None, X, W, y, y, ws, s0) == mq.MQ_ERR_ARG
    assert ba(W, G, X, y, y, y, wgb, None, ws) == mq.MQ_ERR_WORKSPACE
    assert ba(W, G, X, y, y, y, wgb, y, ws - 1) == mq.MQ_ERR_WORKSPACE
    assert ba(W, G, X, y, y, y, wgb, ctypes.c_void_p(0x3002), ws) == mq.MQ_ERR_ARG
    assert ba(W, G, X, y, y, None, wgb, y, ws) == mq.MQ_ERR_WORKSPACE  # split-K workspace
    assert ba(X, G, X, y, y, y, wgb, y, ws) == mq.MQ_ERR_SHAPE
