"""GPU parity over a seeded sweep of random layer shapes (workloads.random_layers).

The hand-picked parity layers cover the cases the kernels were written for; this sweep draws 40
shapes at random (batches of 1-40, 1-96 channels, 1x1 to 5x5 kernels with unequal sides,
strides 1-3, paddings up to the kernel size, NVFP4 and NVFP6) so that combinations nobody chose
reach the tile selection, the batch-16 and batch-32 tiles, the XCD-aware workgroup numbering,
the small-channel weight gradient and the generic fallback. Every output element is compared
with the CPU oracle (codes, scales and T bit-exact; the GEMMs within 2^-10 * sum|w*x|, the
recipe of the onedev.kr MicroQonv digest, section "How it differs", in the readings the oracle
documents).
"""
import numpy as np
import pytest
import torch

import microscaling_quantized_convolution_amd as mq
import workloads
from gpu_parity import check_layer, log, oracle_layer, run_gpu_layer, run_layer_step

pytestmark = pytest.mark.gpu

LAYERS = workloads.random_layers()


@pytest.mark.parametrize("layer", LAYERS, ids=lambda l: l.name)
def test_random_layer_parity(layer):
    log("random layer", layer.name, layer.conv_tuple(), "fmt", layer.fmt)
    check_layer(run_gpu_layer(layer), oracle_layer(layer), layer)


@pytest.mark.parametrize("layer", LAYERS[::2], ids=lambda l: l.name)
def test_random_layer_step_parity(layer):
    """The calls the benchmark times: X (NCHW) and W (OIHW) in one batched quantization, G_Y
    with stochastic rounding, the forward GEMM and both gradients in one call."""
    log("random layer step", layer.name, layer.conv_tuple(), "fmt", layer.fmt)
    check_layer(run_layer_step(layer), oracle_layer(layer), layer)


def _partials_max(ws: torch.Tensor) -> int:
    w = ws.view(torch.int32).cpu().numpy().view(np.uint32)
    P = int(w[0])
    assert 1 <= P <= 1024, P
    return int(w[1:1 + P].max())


def _absmax_bits(t: torch.Tensor) -> int:
    return int((t.view(torch.int32) & 0x7FFFFFFF).max().item())


@pytest.mark.parametrize("layer", LAYERS[1::4], ids=lambda l: l.name)
def test_random_layer_fused_amax(layer):
    """The epilogue's amax partials reduce to max |Y| and max |G_X| exactly, and the outputs are
    those of the plain calls bit for bit."""
    log("random layer fused amax", layer.name, layer.conv_tuple())
    gl = run_gpu_layer(layer)
    p = layer.conv_tuple()
    y = torch.full_like(gl.y, float("nan"))
    ya = torch.empty(mq.MQ_QUANTIZE_WS_BYTES, dtype=torch.uint8, device="cuda")
    mq.mq_conv_fwd_amax(p, gl.qx, gl.qw, y, ya)
    gw = torch.full_like(gl.gw, float("nan"))
    gx = torch.full_like(gl.gx, float("nan"))
    ws = torch.empty(mq.mq_wgrad_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    ga = torch.empty(mq.MQ_QUANTIZE_WS_BYTES, dtype=torch.uint8, device="cuda")
    mq.mq_conv_backward_amax(p, gl.qw, gl.qg, gl.qx, gw, gx, ws, ga)
    torch.cuda.synchronize()
    assert torch.equal(y, gl.y) and torch.equal(gw, gl.gw) and torch.equal(gx, gl.gx)
    assert _partials_max(ya) == _absmax_bits(y), f"{layer.name}: amax of Y"
    assert _partials_max(ga) == _absmax_bits(gx), f"{layer.name}: amax of G_X"
