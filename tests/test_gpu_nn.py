"""GPU tests of the PyTorch integration (MQConv2d, ResNet18MQ).

The autograd function is checked against the CPU oracle end to end: NCHW input and OIHW weight
in, the forward output and both gradients out (after the layout changes the module does), with
the same per-element bound as the library's own parity tests: |gpu - oracle| <= 2^-10 * sum|w*x|
(the operands are quantized exactly once each, so the codes must match the oracle's and only the
fp32 summation order differs).
"""
import numpy as np
import pytest
import torch

import microscaling_quantized_convolution_amd as mq
from microscaling_quantized_convolution_amd.nn import MQConv2d, MQConv2dFunction, ResNet18MQ
import oracle
import workloads
from gpu_parity import assert_conv_close, log, oracle_layer

pytestmark = pytest.mark.gpu

LAYERS = [workloads.config1()[0]] + [l for l in workloads.parity_layers()
                                     if l.name in ("p.3x3s1p1", "p.3x3s2p1", "p.1x1s2",
                                                   "p.3x3s2p1.fp6")]


@pytest.mark.parametrize("layer", LAYERS, ids=lambda l: l.name)
def test_autograd_conv_matches_oracle(layer):
    log("nn parity", layer.name)
    x, w, g = workloads.make_tensors(layer)
    xt = torch.from_numpy(x).cuda().requires_grad_(True)
    wt = torch.from_numpy(w).cuda().requires_grad_(True)
    y = MQConv2dFunction.apply(xt, wt, layer.stride, layer.pad, layer.fmt, layer.sr_seed, None)
    y.backward(torch.from_numpy(g).cuda())
    torch.cuda.synchronize()

    ol = oracle_layer(layer, (x, w, g))
    p = layer.conv_tuple()
    yr, ya = oracle.conv_fwd(p, ol.deq["x"], ol.deq["w"])        # [Ho][Wo][Cout][N]
    gwr, gwa = oracle.conv_wgrad(p, ol.deq["g"], ol.deq["x"])    # [Kh][Kw][Cout][Cin]
    gxr, gxa = oracle.conv_dgrad(p, ol.deq["w"], ol.deq["g"])    # [H][W][Cin][N]
    to_nchw = lambda a: np.ascontiguousarray(a.transpose(3, 2, 0, 1))
    to_oihw = lambda a: np.ascontiguousarray(a.transpose(2, 3, 0, 1))
    assert tuple(y.shape) == (layer.N, layer.Cout, layer.Ho, layer.Wo)
    assert_conv_close(y.detach().cpu().numpy(), to_nchw(yr), to_nchw(ya), f"{layer.name} y")
    assert_conv_close(wt.grad.cpu().numpy(), to_oihw(gwr), to_oihw(gwa), f"{layer.name} gw")
    assert_conv_close(xt.grad.cpu().numpy(), to_nchw(gxr), to_nchw(gxa), f"{layer.name} gx")


def test_module_seeds_and_weight_cache():
    torch.manual_seed(0)
    conv = MQConv2d(16, 24, 3, 1, 1, layer_index=2, layers=5, seed_base=11).cuda()
    x = torch.randn(4, 16, 10, 10, device="cuda")
    assert conv.sr_seed() == 11 + 2
    conv.train()
    y_train = conv(x)
    assert conv.step == 1 and conv.sr_seed() == 11 + 2 + 5
    conv.eval()
    conv.cache_weight = True
    with torch.no_grad():
        y1 = conv(x)
        y2 = conv(x)
    assert torch.equal(y1, y_train.detach()) and torch.equal(y1, y2)
    qw_first = conv._qw
    with torch.no_grad():
        conv.weight.mul_(2.0)  # the version counter moves: the cached weight is stale
        y3 = conv(x)
    assert conv._qw is not qw_first
    conv.cache_weight = False
    with torch.no_grad():
        y4 = conv(x)
    assert torch.equal(y3, y4) and not torch.equal(y3, y1)


def test_module_rejects_bad_input():
    conv = MQConv2d(8, 8, 3, 1, 1).cuda()
    with pytest.raises(ValueError):
        conv(torch.randn(2, 8, 6, 6, device="cuda", dtype=torch.float64))
    with pytest.raises(ValueError):
        conv(torch.randn(2, 4, 6, 6, device="cuda"))


def test_resnet18_training_step_small():
    torch.manual_seed(0)
    model = ResNet18MQ(num_classes=10).cuda()
    assert len(model.mq_convs) == 19
    opt = torch.optim.SGD(model.parameters(), lr=0.05, momentum=0.9)
    x = torch.rand(4, 3, 64, 64, device="cuda")
    labels = torch.randint(0, 10, (4,), device="cuda")
    before = [c.weight.detach().clone() for c in model.mq_convs]
    losses = []
    for _ in range(3):
        opt.zero_grad(set_to_none=True)
        loss = torch.nn.functional.cross_entropy(model(x), labels)
        loss.backward()
        for c in model.mq_convs:
            assert c.weight.grad is not None and torch.isfinite(c.weight.grad).all()
        opt.step()
        losses.append(float(loss.detach()))
    torch.cuda.synchronize()
    log("resnet18 small losses", losses)
    assert all(np.isfinite(losses))
    assert all(not torch.equal(b, c.weight) for b, c in zip(before, model.mq_convs))
    assert [c.step for c in model.mq_convs] == [3] * 19


def test_each_tensor_quantized_once_per_step(monkeypatch):
    """One training step of a layer quantizes X and W once (one batched call) and G_Y once (one
    call), and both gradient GEMMs read those same quantized tensors: nothing is re-quantized
    between the GEMMs that share an operand (the quantize-once premise of the method)."""
    from microscaling_quantized_convolution_amd import nn as mqnn
    calls = []

    def wrap(name):
        real = getattr(mqnn, name)

        def rec(*args):
            calls.append((name, args))
            return real(*args)
        monkeypatch.setattr(mqnn, name, rec)

    for name in ("quant_job", "mq_quantize_batch", "mq_quantize_nchw", "mq_quantize_weight",
                 "mq_conv_fwd", "mq_conv_backward", "mq_conv_wgrad", "mq_conv_dgrad"):
        wrap(name)
    layer = workloads.parity_layers()[0]
    x, w, g = workloads.make_tensors(layer)
    xt = torch.from_numpy(x).cuda().requires_grad_(True)
    wt = torch.from_numpy(w).cuda().requires_grad_(True)
    y = MQConv2dFunction.apply(xt, wt, layer.stride, layer.pad, layer.fmt, layer.sr_seed, None)
    y.backward(torch.from_numpy(g).cuda())
    torch.cuda.synchronize()
    names = [c[0] for c in calls]
    assert names == ["quant_job", "quant_job", "mq_quantize_batch", "mq_conv_fwd",
                     "mq_quantize_nchw", "mq_conv_backward"]
    assert len(calls[2][1][0]) == 2          # the batch holds the two jobs
    qx, qw = calls[0][1][2], calls[1][1][2]  # quant_job(src, order, dst, ...): X, then W
    _, fqx, fqw, _ = calls[3][1]             # conv_fwd(conv, qx, qw, y)
    _, qg, _, _, _ = calls[4][1]             # quantize_nchw(gy, qg, rounding, seed, ws)
    _, bqw, bqg, bqx, _, _, _ = calls[5][1]  # conv_backward(conv, qw, qg, qx, gw, gx, ws)
    assert fqx is qx and fqw is qw
    assert bqw is qw and bqx is qx and bqg is qg
