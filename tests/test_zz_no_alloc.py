"""mq_conv_backward_noalloc (the split-K partials in the library's own device array) against
mq_conv_backward with a caller workspace: G_W and G_X equal bit for bit, on two calls in a row,
the second with a smaller convolution (the array keeps the first call's partials)."""
import pytest
import torch

import microscaling_quantized_convolution_amd as mq
import workloads
from gpu_parity import log, run_gpu_layer

pytestmark = pytest.mark.gpu


def _both(layer):
    gl = run_gpu_layer(layer)
    p = layer.conv_tuple()
    ws = torch.empty(mq.mq_wgrad_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    gw = torch.full_like(gl.gw, float("nan"))
    gx = torch.full_like(gl.gx, float("nan"))
    mq.mq_conv_backward(p, gl.qw, gl.qg, gl.qx, gw, gx, ws)
    gw_na = torch.full_like(gl.gw, float("nan"))
    gx_na = torch.full_like(gl.gx, float("nan"))
    mq.mq_conv_backward_noalloc(p, gl.qw, gl.qg, gl.qx, gw_na, gx_na)
    torch.cuda.synchronize()
    return (gw, gx), (gw_na, gx_na)


def test_noalloc_backward_equals_workspace_backward():
    first = workloads.config2()[0]       # ResNet 3x3 layer, N=32, 64->64 at 56x56
    second = workloads.parity_layers()[0]  # 3x3, N=6, 20->24 at 11x13: fewer partials
    assert mq.mq_wgrad_workspace_bytes(second.conv_tuple()) < \
        mq.mq_wgrad_workspace_bytes(first.conv_tuple())
    for layer in (first, second):
        log("noalloc backward", layer.name, layer.conv_tuple())
        (gw, gx), (gw_na, gx_na) = _both(layer)
        assert torch.equal(gw_na, gw), f"{layer.name}: G_W differs"
        assert torch.equal(gx_na, gx), f"{layer.name}: G_X differs"
        assert torch.isfinite(gw).all() and torch.isfinite(gx).all()


def test_noalloc_backward_in_a_graph():
    """The use it exists for: captured into a HIP graph (no allocation during capture), every
    replay equals the eager call bit for bit, also after eager calls of another convolution have
    overwritten the library's array in between."""
    layer, other = workloads.parity_layers()[6], workloads.parity_layers()[0]
    gl, go = run_gpu_layer(layer), run_gpu_layer(other)
    p, po = layer.conv_tuple(), other.conv_tuple()
    gw = torch.full_like(gl.gw, float("nan"))
    gx = torch.full_like(gl.gx, float("nan"))
    mq.mq_conv_backward_noalloc(p, gl.qw, gl.qg, gl.qx, gw, gx)
    torch.cuda.synchronize()
    want_w, want_x = gw.clone(), gx.clone()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        mq.mq_conv_backward_noalloc(p, gl.qw, gl.qg, gl.qx, gw, gx, stream=stream)
    ow = torch.empty_like(go.gw)
    ox = torch.empty_like(go.gx)
    for rep in range(3):
        mq.mq_conv_backward_noalloc(po, go.qw, go.qg, go.qx, ow, ox)  # overwrites the array
        gw.fill_(float("nan"))
        gx.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(gw, want_w), f"replay {rep}: G_W differs"
        assert torch.equal(gx, want_x), f"replay {rep}: G_X differs"
