"""The tensor amax of a convolution's output produced in the forward / input-gradient epilogue
(mq_conv_fwd_amax, mq_conv_backward_amax) instead of an amax pass over the output.

The recipe's tensor scale is T = max|X| / (448 * Emax) (onedev.kr MicroQonv digest, section "How
it differs"); these calls hand max|Y| or max|G_X| to the quantization of that tensor through the
MQ_QUANTIZE_AMAX_READY workspace. Checked on the GPU, per layer:
- Y, G_W and G_X equal the plain calls' bit for bit;
- the partial maxima reduce to exactly max|output| (as fp32 bit patterns);
- quantizing the output with the epilogue's partials gives the codes, scales and T of the
  two-pass quantization of the same tensor (which the quantize parity tests pin to the oracle),
  with nearest and with stochastic rounding, also when the output holds NaN.
"""
import numpy as np
import pytest
import torch

import microscaling_quantized_convolution_amd as mq
import workloads
from gpu_parity import log, run_gpu_layer, to_dev

pytestmark = pytest.mark.gpu

LAYERS = (workloads.config1() + workloads.parity_layers() +
          [workloads.config2()[0], workloads.config3()[0], workloads.config4()[1],
           workloads.config5()[0], workloads.config5()[16]])


def _absmax_bits(t: torch.Tensor) -> int:
    return int((t.view(torch.int32) & 0x7FFFFFFF).max().item())


def _partials_max(ws: torch.Tensor) -> int:
    w = ws.view(torch.int32).cpu().numpy().view(np.uint32)
    P = int(w[0])
    assert 1 <= P <= 1024, P
    return int(w[1:1 + P].max())


def _quantize_both(t: torch.Tensor, shape, fmt, role, rnd, seed, amax_ws):
    """The same tensor quantized with the given partial maxima and with its own amax pass."""
    fused = mq.QTensor(*shape, fmt, role)
    mq.mq_quantize(t, fused, rnd, seed, amax_ws, mq.MQ_QUANTIZE_AMAX_READY)
    plain = mq.QTensor(*shape, fmt, role)
    mq.mq_quantize(t, plain, rnd, seed, mq.quantize_workspace())
    torch.cuda.synchronize()
    return fused, plain


def _assert_same_quant(a: mq.QTensor, b: mq.QTensor, what):
    assert torch.equal(a.tscale.view(torch.int32), b.tscale.view(torch.int32)), f"{what}: T"
    assert torch.equal(a.scales, b.scales), f"{what}: scales"
    assert torch.equal(a.codes, b.codes), f"{what}: codes"


@pytest.mark.parametrize("layer", LAYERS, ids=lambda l: l.name)
def test_fused_amax_matches_amax_pass(layer):
    log("fused amax", layer.name, layer.conv_tuple())
    gl = run_gpu_layer(layer)
    p = layer.conv_tuple()
    fmt = layer.fmt
    # forward: Y and its amax partials
    y = torch.full_like(gl.y, float("nan"))
    ya = torch.empty(mq.MQ_QUANTIZE_WS_BYTES, dtype=torch.uint8, device="cuda")
    mq.mq_conv_fwd_amax(p, gl.qx, gl.qw, y, ya)
    torch.cuda.synchronize()
    assert torch.equal(y, gl.y), f"{layer.name}: Y differs from mq_conv_fwd"
    assert _partials_max(ya) == _absmax_bits(y), f"{layer.name}: amax of Y"
    yshape = (layer.Ho, layer.Wo, layer.Cout, layer.N)
    f, q = _quantize_both(y, yshape, fmt, mq.MQ_ROLE_ACT, mq.MQ_RNE, 0, ya)
    _assert_same_quant(f, q, f"{layer.name} Y")
    # backward: G_W, G_X and the amax partials of G_X
    gw = torch.full_like(gl.gw, float("nan"))
    gx = torch.full_like(gl.gx, float("nan"))
    ws = torch.empty(mq.mq_wgrad_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    ga = torch.empty(mq.MQ_QUANTIZE_WS_BYTES, dtype=torch.uint8, device="cuda")
    mq.mq_conv_backward_amax(p, gl.qw, gl.qg, gl.qx, gw, gx, ws, ga)
    torch.cuda.synchronize()
    assert torch.equal(gw, gl.gw), f"{layer.name}: G_W differs from mq_conv_wgrad"
    assert torch.equal(gx, gl.gx), f"{layer.name}: G_X differs from mq_conv_dgrad"
    assert _partials_max(ga) == _absmax_bits(gx), f"{layer.name}: amax of G_X"
    xshape = (layer.H, layer.W, layer.Cin, layer.N)
    f, q = _quantize_both(gx, xshape, fmt, mq.MQ_ROLE_GRAD, mq.MQ_SR, layer.sr_seed + 5, ga)
    _assert_same_quant(f, q, f"{layer.name} G_X")


def test_fused_amax_propagates_nan():
    """A NaN input makes every output NaN: the partials carry it, and the quantization of the
    output gets T = NaN, scales 0x7F and codes 0, as with its own amax pass."""
    layer = workloads.parity_layers()[0]
    x, w, g = workloads.make_tensors(layer)
    x = x.copy()
    x[0, 0, 0, 0] = np.nan
    gl = run_gpu_layer(layer, tensors=(x, w, g))
    p = layer.conv_tuple()
    y = torch.empty_like(gl.y)
    ya = torch.empty(mq.MQ_QUANTIZE_WS_BYTES, dtype=torch.uint8, device="cuda")
    mq.mq_conv_fwd_amax(p, gl.qx, gl.qw, y, ya)
    torch.cuda.synchronize()
    assert _partials_max(ya) > 0x7F800000  # a NaN pattern
    f, q = _quantize_both(y, (layer.Ho, layer.Wo, layer.Cout, layer.N), layer.fmt,
                          mq.MQ_ROLE_ACT, mq.MQ_RNE, 0, ya)
    _assert_same_quant(f, q, "NaN Y")
    assert torch.isnan(f.tscale).all() and (f.scales == 0x7F).all()


def test_fused_amax_workspace_reused_for_a_smaller_output():
    """The workspace keeps a larger launch's partials; the count word limits what is read."""
    big, small = workloads.config2()[0], workloads.parity_layers()[0]
    ya = torch.empty(mq.MQ_QUANTIZE_WS_BYTES, dtype=torch.uint8, device="cuda")
    for layer in (big, small):
        gl = run_gpu_layer(layer)
        y = torch.empty_like(gl.y)
        mq.mq_conv_fwd_amax(layer.conv_tuple(), gl.qx, gl.qw, y, ya)
        torch.cuda.synchronize()
        assert _partials_max(ya) == _absmax_bits(y), layer.name
