"""HIP graph capture of one pass of the path (what bench.py times): every replay must equal the
eager pass bit for bit, with eager work and synchronizations between replays."""
import numpy as np
import pytest
import torch

import workloads
from gpu_parity import log, to_dev

import microscaling_quantized_convolution_amd as mq
from microscaling_quantized_convolution_amd.step import LayerStep

pytestmark = pytest.mark.gpu

LAYERS = [workloads.config1()[0]] + [l for l in workloads.parity_layers()
                                     if l.name in ("p.3x3s2p1", "p.3x3s1p0.fp6")]


def _snapshot(st):
    return [t.detach().cpu().numpy().copy() for t in st.outputs()]


@pytest.mark.parametrize("layer", LAYERS, ids=lambda l: l.name)
def test_graph_replays_equal_eager(layer):
    log("graph replay", layer.name)
    x, w, g = workloads.make_tensors(layer)
    gc = torch.empty(g.size, dtype=torch.float32, device="cuda")
    mq.mq_relayout_cbf(to_dev(g), gc, layer.N, layer.Cout, layer.Ho, layer.Wo, 0)
    st = LayerStep(layer.conv_tuple(), layer.fmt, to_dev(x), to_dev(w), gc,
                   sr_seed_base=layer.sr_seed)
    seed = 3
    st.run(seed)
    torch.cuda.synchronize()
    want = _snapshot(st)

    stream = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=stream):
        st.run(seed)
    for rep in range(4):
        # eager work in between: a different seed overwrites every output
        st.run(seed + 1 + rep)
        torch.cuda.synchronize()
        for t in st.outputs():
            if t.dtype == torch.float32:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        got = _snapshot(st)
        for i, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (layer.name, rep, i)
