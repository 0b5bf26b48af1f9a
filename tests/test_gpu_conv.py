"""GPU parity of the three convolution GEMMs against the CPU oracle.

Forward Y = W.X', weight gradient G_W = G_Y.X'^T and input gradient G_X' = W^T.G_Y (col2im
fused), on channel-batch-first square-quantized tensors (onedev.kr MicroQonv digest, sections
"How it works" and "How it differs"). Per element |gpu - oracle| <= 2^-10 * sum|w*x| (the
GPU sums exact bf16 products in fp32), and exactly 0 where every term is 0.

Every layer is compared element by element: the small and ragged parity layers through the
single-tensor calls, and every full-size workload layer through the calls the benchmark times.
"""
import numpy as np
import pytest
import torch

import microscaling_quantized_convolution_amd as mq
import oracle
import workloads
from gpu_parity import (check_layer, log, oracle_layer, run_gpu_layer, run_layer_step)

pytestmark = pytest.mark.gpu

SMALL = workloads.config1() + workloads.parity_layers() + workloads.persistent_layers()


@pytest.mark.parametrize("layer", SMALL, ids=lambda l: l.name)
def test_conv_parity_full_tensor(layer):
    log("conv parity", layer.name)
    check_layer(run_gpu_layer(layer), oracle_layer(layer), layer)


def _distinct(layers):
    seen, out = set(), []
    for l in layers:
        key = l.conv_tuple() + (l.fmt,)
        if key not in seen:
            seen.add(key)
            out.append(l)
    return out


# Every full-size workload layer (each distinct shape of the ResNet-18 body once), through the
# calls the benchmark times: the batched NCHW/OIHW quantization, the stochastic G_Y quantization,
# the forward GEMM and the one-call backward. Every output element is compared.
FULL_SIZE = (workloads.config2() + workloads.config3() + workloads.config4() +
             _distinct(workloads.config5()))


@pytest.mark.parametrize("layer", FULL_SIZE, ids=lambda l: l.name)
def test_layer_step_parity_full_size(layer):
    log("layer step parity (full tensors)", layer.name, layer.conv_tuple())
    gl = run_layer_step(layer)
    check_layer(gl, oracle_layer(layer), layer)
    for t, what in ((gl.y, "fwd"), (gl.gw, "wgrad"), (gl.gx, "dgrad")):
        assert torch.isfinite(t).all(), f"{layer.name} {what}: non-finite output"


def test_conv_deterministic():
    layer = workloads.parity_layers()[6]
    a = run_gpu_layer(layer)
    b = run_gpu_layer(layer)
    for t1, t2 in ((a.y, b.y), (a.gw, b.gw), (a.gx, b.gx)):
        assert torch.equal(t1, t2)


def test_conv_nan_propagates():
    layer = workloads.parity_layers()[0]
    x, w, g = workloads.make_tensors(layer)
    x = x.copy()
    x[0, 0, 0, 0] = np.nan
    gl = run_gpu_layer(layer, tensors=(x, w, g))
    assert torch.isnan(gl.y).all()
    assert torch.isnan(gl.gw).all()
    assert not torch.isnan(gl.gx).any()  # dgrad does not read X


def test_conv_zero_weight_gives_exact_zero():
    layer = workloads.parity_layers()[1]
    x, w, g = workloads.make_tensors(layer)
    gl = run_gpu_layer(layer, tensors=(x, np.zeros_like(w), g))
    assert (gl.y == 0).all() and (gl.gx == 0).all()


def test_conv_one_hot_weight_reads_im2col_column():
    """A weight with one non-zero entry makes Y a copy of one im2col row: the on-chip im2col
    gathers exactly the dequantized input (zero in the padding)."""
    layer = workloads.ConvLayer("onehot", N=5, Cin=6, H=7, W=9, Cout=5, Kh=3, Kw=3, stride=2,
                                pad=1, x_dist="normal", seed=21)
    x, w, g = workloads.make_tensors(layer)
    ol = oracle_layer(layer, tensors=(x, w, g))
    for (co, ci, kh, kw) in ((0, 0, 0, 0), (3, 5, 2, 1), (4, 2, 1, 2)):
        w1 = np.zeros_like(w)
        w1[co, ci, kh, kw] = 1.0
        gl = run_gpu_layer(layer, tensors=(x, w1, g))
        y = gl.y.cpu().numpy().reshape(layer.Ho, layer.Wo, layer.Cout, layer.N)
        xh = ol.deq["x"]
        T_w = float(gl.qw.tscale.cpu().numpy()[0])
        for ho in range(layer.Ho):
            for wo in range(layer.Wo):
                h, ww = ho * 2 - 1 + kh, wo * 2 - 1 + kw
                exp = xh[h, ww, ci, :] if (0 <= h < layer.H and 0 <= ww < layer.W) else 0.0
                # quantized one-hot weight = 6 * 448 * T_w with T_w = 1/2688 -> exactly 1
                np.testing.assert_allclose(y[ho, wo, co, :], exp * (6 * 448 * T_w), rtol=2 ** -20,
                                           atol=0)
        others = [c for c in range(layer.Cout) if c != co]
        assert (y[:, :, others, :] == 0).all()


# full-size layers: the split sum on the CUs the input gradient leaves idle (c2), as its own
# kernel ahead of the input gradient (c3: too many passes), after a persistent input gradient
# that fills the chip (c5 layer 1), and NVFP6 at stride 2 with four parity classes (c4 layer 2)
BACKWARD_FULL = [workloads.config2()[0], workloads.config3()[0], workloads.config5()[0],
                 workloads.config4()[1]]


@pytest.mark.parametrize("layer", SMALL + BACKWARD_FULL, ids=lambda l: l.name)
def test_conv_backward_equals_separate_calls(layer):
    """mq_conv_backward (the weight gradient's split sum riding in the input-gradient launch)
    gives G_W and G_X bit for bit equal to mq_conv_wgrad and mq_conv_dgrad."""
    log("conv backward", layer.name)
    gl = run_gpu_layer(layer)
    p = layer.conv_tuple()
    gw = torch.full_like(gl.gw, float("nan"))
    gx = torch.full_like(gl.gx, float("nan"))
    ws = torch.empty(mq.mq_wgrad_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    mq.mq_conv_backward(p, gl.qw, gl.qg, gl.qx, gw, gx, ws)
    torch.cuda.synchronize()
    assert torch.equal(gw, gl.gw), f"{layer.name}: G_W differs"
    assert torch.equal(gx, gl.gx), f"{layer.name}: G_X differs"
