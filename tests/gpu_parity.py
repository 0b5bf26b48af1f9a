"""Helpers for the GPU-vs-oracle parity tests (test infrastructure).

The GPU side goes through the library's C ABI only (relayout, quantize, the three GEMMs); the
oracle side recomputes everything from the same seeded inputs on the CPU. Nothing computed on the
GPU is fed to the oracle.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import microscaling_quantized_convolution_amd as mq
import oracle
import workloads

TOL = 2.0 ** -10  # per element: |gpu - oracle| <= 2^-10 * sum |w * x|


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@dataclasses.dataclass
class GpuLayer:
    layer: workloads.ConvLayer
    qx: mq.QTensor
    qw: mq.QTensor
    qg: mq.QTensor
    y: torch.Tensor
    gw: torch.Tensor
    gx: torch.Tensor


def to_dev(a: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def gpu_quantize(src_cbf: torch.Tensor, shape, fmt, role, rnd, seed, dev="cuda"):
    q = mq.QTensor(*shape, fmt, role, dev)
    ws = mq.quantize_workspace(dev)
    mq.mq_quantize(src_cbf, q, rnd, seed, ws)
    return q


def run_gpu_layer(layer: workloads.ConvLayer, dev="cuda", tensors=None) -> GpuLayer:
    x, w, g = tensors if tensors is not None else workloads.make_tensors(layer)
    N, Ci, H, W, Co, Kh, Kw = (layer.N, layer.Cin, layer.H, layer.W, layer.Cout, layer.Kh,
                               layer.Kw)
    Ho, Wo = layer.Ho, layer.Wo
    p = layer.conv_tuple()
    xt, wt, gt = to_dev(x, dev), to_dev(w, dev), to_dev(g, dev)
    xc = torch.empty(H * W * Ci * N, dtype=torch.float32, device=dev)
    wc = torch.empty(Kh * Kw * Co * Ci, dtype=torch.float32, device=dev)
    gc = torch.empty(Ho * Wo * Co * N, dtype=torch.float32, device=dev)
    mq.mq_relayout_cbf(xt, xc, N, Ci, H, W, 0)
    mq.mq_relayout_weight(wt, wc, Co, Ci, Kh, Kw, 0)
    mq.mq_relayout_cbf(gt, gc, N, Co, Ho, Wo, 0)
    qx = gpu_quantize(xc, (H, W, Ci, N), layer.fmt, mq.MQ_ROLE_ACT, mq.MQ_RNE, 0, dev)
    qw = gpu_quantize(wc, (Kh, Kw, Co, Ci), layer.fmt, mq.MQ_ROLE_WEIGHT, mq.MQ_RNE, 0, dev)
    qg = gpu_quantize(gc, (Ho, Wo, Co, N), layer.fmt, mq.MQ_ROLE_GRAD, mq.MQ_SR,
                      layer.sr_seed, dev)
    y = torch.full((Ho * Wo * Co * N,), float("nan"), dtype=torch.float32, device=dev)
    gw = torch.full((Kh * Kw * Co * Ci,), float("nan"), dtype=torch.float32, device=dev)
    gx = torch.full((H * W * Ci * N,), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(mq.mq_wgrad_workspace_bytes(p), dtype=torch.uint8, device=dev)
    mq.mq_conv_fwd(p, qx, qw, y)
    mq.mq_conv_wgrad(p, qg, qx, gw, ws)
    mq.mq_conv_dgrad(p, qw, qg, gx)
    torch.cuda.synchronize()
    return GpuLayer(layer, qx, qw, qg, y, gw, gx)


def run_layer_step(layer: workloads.ConvLayer, dev="cuda", step=0) -> GpuLayer:
    """One pass of the path the benchmark times (LayerStep): X from NCHW and W from OIHW in one
    batched quantization, G_Y (already channel-batch-first, as the next layer's input gradient
    leaves it) with stochastic rounding and seed sr_seed + step, the forward GEMM and both
    gradients in one call. The outputs are filled with NaN first."""
    from microscaling_quantized_convolution_amd.step import LayerStep
    x, w, g = workloads.make_tensors(layer)
    gc = torch.empty(g.size, dtype=torch.float32, device=dev)
    mq.mq_relayout_cbf(to_dev(g, dev), gc, layer.N, layer.Cout, layer.Ho, layer.Wo, 0)
    st = LayerStep(layer.conv_tuple(), layer.fmt, to_dev(x, dev), to_dev(w, dev), gc,
                   sr_seed_base=layer.sr_seed)
    for t in (st.y, st.gw, st.gx):
        t.fill_(float("nan"))
    st.run(step)
    torch.cuda.synchronize()
    return GpuLayer(layer, st.qx, st.qw, st.qg, st.y, st.gw, st.gx)


@dataclasses.dataclass
class OracleLayer:
    q: dict          # name -> (codes, scales, T)
    deq: dict        # name -> dequantized float64 CBF tensor


def oracle_layer(layer: workloads.ConvLayer, tensors=None) -> OracleLayer:
    x, w, g = tensors if tensors is not None else workloads.make_tensors(layer)
    xc, wc, gc = oracle.nchw_to_cbf(x), oracle.oihw_to_tap_major(w), oracle.nchw_to_cbf(g)
    q, deq = {}, {}
    for name, t, rnd, seed in (("x", xc, oracle.RNE, 0), ("w", wc, oracle.RNE, 0),
                               ("g", gc, oracle.SR, layer.sr_seed)):
        codes, scales, T = oracle.quantize(t, layer.fmt, rnd, seed)
        q[name] = (codes, scales, T)
        deq[name] = oracle.dequant(codes, scales, T, t.shape, layer.fmt)
    return OracleLayer(q, deq)


def assert_quant_equal(qt: mq.QTensor, ref, fmt, what=""):
    codes, scales, T = ref
    got_codes = qt.codes.cpu().numpy()
    got_scales = qt.scales.cpu().numpy()
    got_T = qt.tscale.cpu().numpy().view(np.uint32)[0]
    exp_codes = oracle.pack(codes, fmt)
    assert got_T == np.float32(T).view(np.uint32), f"{what}: T {got_T:#x} vs {np.float32(T).view(np.uint32):#x}"
    bad_s = np.nonzero(got_scales != scales)[0]
    assert bad_s.size == 0, f"{what}: {bad_s.size} scales differ, first at square {bad_s[:5]}: " \
                            f"{got_scales[bad_s[:5]]} vs {scales[bad_s[:5]]}"
    bad_c = np.nonzero(got_codes != exp_codes)[0]
    assert bad_c.size == 0, f"{what}: {bad_c.size} code bytes differ, first at byte {bad_c[:5]}"


def check_layer(gl: GpuLayer, ol: OracleLayer, layer: workloads.ConvLayer):
    """Quantized tensors bit-exact, and every element of Y, G_W and G_X within the bound."""
    assert_quant_equal(gl.qx, ol.q["x"], layer.fmt, f"{layer.name} x")
    assert_quant_equal(gl.qw, ol.q["w"], layer.fmt, f"{layer.name} w")
    assert_quant_equal(gl.qg, ol.q["g"], layer.fmt, f"{layer.name} g")
    p = layer.conv_tuple()
    y, ya = oracle.conv_fwd(p, ol.deq["x"], ol.deq["w"])
    assert_conv_close(gl.y.cpu().numpy(), y, ya, f"{layer.name} fwd")
    del y, ya
    gw, gwa = oracle.conv_wgrad(p, ol.deq["g"], ol.deq["x"])
    assert_conv_close(gl.gw.cpu().numpy(), gw, gwa, f"{layer.name} wgrad")
    del gw, gwa
    gx, gxa = oracle.conv_dgrad(p, ol.deq["w"], ol.deq["g"])
    assert_conv_close(gl.gx.cpu().numpy(), gx, gxa, f"{layer.name} dgrad")


def assert_conv_close(got: np.ndarray, ref: np.ndarray, refabs: np.ndarray, what=""):
    got = got.astype(np.float64).reshape(ref.shape)
    err = np.abs(got - ref)
    lim = TOL * refabs
    bad = ~(err <= lim)
    if bad.any():
        i = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside 2^-10*sum|wx|; "
                             f"first {i.tolist()} got {got[bad][:5]} ref {ref[bad][:5]} "
                             f"sumabs {refabs[bad][:5]}")
    zero = refabs == 0
    assert (got[zero] == 0).all(), f"{what}: non-zero output where every term is zero"
