"""Pins of the oracle's three convolution GEMMs and layouts (CPU only).

The oracle forms the explicit im2col matrix X' and evaluates Y = W.X', G_W = G_Y.X'^T and
G_X' = W^T.G_Y (followed by col2im) on the 2-D reshapes W_{fCout,Cin} and G_{YfCout,N}
(onedev.kr MicroQonv digest, section "How it differs"), on channel-batch-first tensors (section
"How it works"). Pins: torch's float64 conv2d / conv2d_weight / conv2d_input (a library special
case: the same convolution without quantization-specific code), an exact rational direct
convolution on tiny inputs, and numpy transposes for the layouts.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.grad as tgrad

import oracle
import workloads


def _deq(layer):
    """Quantize-dequantize the layer's synthetic tensors through the oracle (CBF layouts)."""
    x, w, g = workloads.make_tensors(layer)
    xc = oracle.nchw_to_cbf(x)
    wc = oracle.oihw_to_tap_major(w)
    gc = oracle.nchw_to_cbf(g)
    xh = oracle.quant_dequant(xc, layer.fmt, oracle.RNE)[3]
    wh = oracle.quant_dequant(wc, layer.fmt, oracle.RNE)[3]
    gh = oracle.quant_dequant(gc, layer.fmt, oracle.SR, layer.sr_seed)[3]
    return xh, wh, gh


def _nchw(t):  # CBF [H][W][C][N] -> NCHW
    return torch.from_numpy(np.ascontiguousarray(t.transpose(3, 2, 0, 1)))


def _oihw(t):  # [Kh][Kw][Cout][Cin] -> OIHW
    return torch.from_numpy(np.ascontiguousarray(t.transpose(2, 3, 0, 1)))


LAYERS = workloads.config1() + workloads.parity_layers()


@pytest.mark.parametrize("layer", LAYERS, ids=lambda l: l.name)
def test_gemms_match_torch_float64(layer):
    p = layer.conv_tuple()
    s, pad = (layer.stride, layer.sw), (layer.pad, layer.pw)
    xh, wh, gh = _deq(layer)
    y, ya = oracle.conv_fwd(p, xh, wh)
    gw, gwa = oracle.conv_wgrad(p, gh, xh)
    gx, gxa = oracle.conv_dgrad(p, wh, gh)
    X, Wt, G = _nchw(xh), _oihw(wh), _nchw(gh)
    ref_y = torch.nn.functional.conv2d(X, Wt, stride=s, padding=pad).numpy()
    ref_ya = torch.nn.functional.conv2d(X.abs(), Wt.abs(), stride=s, padding=pad).numpy()
    ref_gw = tgrad.conv2d_weight(X, Wt.shape, G, stride=s, padding=pad).numpy()
    ref_gwa = tgrad.conv2d_weight(X.abs(), Wt.shape, G.abs(), stride=s, padding=pad).numpy()
    ref_gx = tgrad.conv2d_input(X.shape, Wt, G, stride=s, padding=pad).numpy()
    ref_gxa = tgrad.conv2d_input(X.shape, Wt.abs(), G.abs(), stride=s, padding=pad).numpy()
    for got, gota, ref, refa, tr in (
            (y, ya, ref_y, ref_ya, (3, 2, 0, 1)),
            (gw, gwa, ref_gw, ref_gwa, (2, 3, 0, 1)),
            (gx, gxa, ref_gx, ref_gxa, (3, 2, 0, 1))):
        got_t, gota_t = got.transpose(tr), gota.transpose(tr)
        assert got_t.shape == ref.shape
        assert np.all(np.abs(got_t - ref) <= 1e-12 * refa + 1e-300)
        assert np.allclose(gota_t, refa, rtol=1e-12, atol=0)
        assert np.abs(ref).max() > 0


def _exact_direct(layer, xh, wh, gh):
    """Textbook direct convolution and its two gradients in exact rationals (NCHW/OIHW)."""
    N, Ci, H, W, Co, Kh, Kw = (layer.N, layer.Cin, layer.H, layer.W, layer.Cout, layer.Kh,
                               layer.Kw)
    sh, sw, ph, pw, Ho, Wo = layer.stride, layer.sw, layer.pad, layer.pw, layer.Ho, layer.Wo
    X = [[[[Fraction(float(xh[h, w, c, n])) for w in range(W)] for h in range(H)]
          for c in range(Ci)] for n in range(N)]
    Wf = [[[[Fraction(float(wh[kh, kw, o, c])) for kw in range(Kw)] for kh in range(Kh)]
           for c in range(Ci)] for o in range(Co)]
    G = [[[[Fraction(float(gh[ho, wo, o, n])) for wo in range(Wo)] for ho in range(Ho)]
          for o in range(Co)] for n in range(N)]

    def xin(n, c, h, w):
        return X[n][c][h][w] if 0 <= h < H and 0 <= w < W else Fraction(0)

    y = {}
    for n in range(N):
        for o in range(Co):
            for ho in range(Ho):
                for wo in range(Wo):
                    y[n, o, ho, wo] = sum(Wf[o][c][kh][kw] * xin(n, c, ho * sh - ph + kh, wo * sw - pw + kw)
                                          for c in range(Ci) for kh in range(Kh) for kw in range(Kw))
    gw = {}
    for o in range(Co):
        for c in range(Ci):
            for kh in range(Kh):
                for kw in range(Kw):
                    gw[o, c, kh, kw] = sum(G[n][o][ho][wo] * xin(n, c, ho * sh - ph + kh, wo * sw - pw + kw)
                                           for n in range(N) for ho in range(Ho) for wo in range(Wo))
    gx = {(n, c, h, w): Fraction(0) for n in range(N) for c in range(Ci) for h in range(H)
          for w in range(W)}
    for n in range(N):
        for o in range(Co):
            for ho in range(Ho):
                for wo in range(Wo):
                    for c in range(Ci):
                        for kh in range(Kh):
                            for kw in range(Kw):
                                h, w = ho * sh - ph + kh, wo * sw - pw + kw
                                if 0 <= h < H and 0 <= w < W:
                                    gx[n, c, h, w] += Wf[o][c][kh][kw] * G[n][o][ho][wo]
    return y, gw, gx


@pytest.mark.parametrize("sh,sw,ph,pw,kh,kw", [(2, 2, 1, 1, 3, 3), (1, 1, 0, 0, 3, 3),
                                               (1, 1, 1, 1, 1, 1), (2, 2, 0, 0, 1, 1),
                                               (1, 2, 0, 1, 1, 3), (3, 3, 1, 1, 3, 3),
                                               (2, 1, 1, 0, 3, 2)])
def test_gemms_match_exact_direct_convolution(sh, sw, ph, pw, kh, kw):
    layer = workloads.ConvLayer("tiny", N=2, Cin=3, H=5, W=6, Cout=2, Kh=kh, Kw=kw, stride=sh,
                                pad=ph, stride_w=sw, pad_w=pw, x_dist="normal", w_dist="normal",
                                g_dist="normal", seed=7, sr_seed=3)
    p = layer.conv_tuple()
    xh, wh, gh = _deq(layer)
    y, ya = oracle.conv_fwd(p, xh, wh)
    gw, gwa = oracle.conv_wgrad(p, gh, xh)
    gx, gxa = oracle.conv_dgrad(p, wh, gh)
    ey, egw, egx = _exact_direct(layer, xh, wh, gh)
    K = layer.Cin * kh * kw
    rel = 2.0 ** -52 * max(K, layer.N * layer.Ho * layer.Wo)
    for (n, o, ho, wo), v in ey.items():
        assert abs(Fraction(y[ho, wo, o, n]) - v) <= rel * Fraction(ya[ho, wo, o, n])
    for (o, c, kh, kw), v in egw.items():
        assert abs(Fraction(gw[kh, kw, o, c]) - v) <= rel * Fraction(gwa[kh, kw, o, c])
    for (n, c, h, w), v in egx.items():
        assert abs(Fraction(gx[h, w, c, n]) - v) <= rel * Fraction(gxa[h, w, c, n])


@pytest.mark.parametrize("layer", workloads.parity_layers()[:4] + workloads.config1(),
                         ids=lambda l: l.name)
def test_sampled_outputs_equal_full(layer):
    p = layer.conv_tuple()
    xh, wh, gh = _deq(layer)
    y, ya = oracle.conv_fwd(p, xh, wh)
    gw, gwa = oracle.conv_wgrad(p, gh, xh)
    gx, gxa = oracle.conv_dgrad(p, wh, gh)
    rng = np.random.default_rng(1)
    for full, fulla, fn, a, b in ((y, ya, oracle.conv_fwd_at, xh, wh),
                                  (gw, gwa, oracle.conv_wgrad_at, gh, xh),
                                  (gx, gxa, oracle.conv_dgrad_at, wh, gh)):
        idx = np.stack([rng.integers(0, d, 200) for d in full.shape], 1).astype(np.int32)
        v, va = fn(p, a, b, idx)
        assert (v == full[tuple(idx.T)]).all()
        assert (va == fulla[tuple(idx.T)]).all()


def test_relayouts_match_numpy():
    x = workloads.random_array((3, 5, 7, 2), seed=1)
    c = oracle.nchw_to_cbf(x)
    assert (c == x.transpose(2, 3, 1, 0)).all()
    assert (oracle.cbf_to_nchw(c) == x).all()
    w = workloads.random_array((6, 4, 3, 5), seed=2)
    t = oracle.oihw_to_tap_major(w)
    assert (t == w.transpose(2, 3, 0, 1)).all()
    assert (oracle.tap_major_to_oihw(t) == w).all()


def test_invalid_conv_rejected():
    z = np.zeros((1, 1, 1, 1))
    with pytest.raises(RuntimeError):
        oracle.conv_fwd((1, 1, 2, 2, 1, 3, 3, 1, 1, 0, 0), np.zeros((2, 2, 1, 1)), np.zeros((3, 3, 1, 1)))
    del z
