"""GPU parity of relayout and quantization: bit-exact against the CPU oracle.

The quantizer follows the NVFP4 / NVFP6 recipe of the onedev.kr MicroQonv digest (section "How
it differs"); the channel-batch-first relayout follows section "How it works". Codes, scales and
the tensor scale must match the oracle byte for byte.
"""
import numpy as np
import pytest
import torch

import microscaling_quantized_convolution_amd as mq
import oracle
import workloads
from gpu_parity import assert_quant_equal, gpu_quantize, log, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [
    (1, 1, 1, 1), (1, 1, 4, 4), (2, 3, 5, 7), (3, 2, 8, 12), (4, 4, 13, 2), (1, 7, 33, 9),
    (6, 5, 16, 32), (2, 2, 64, 64), (5, 3, 17, 31),
]


@pytest.mark.parametrize("fmt", [4, 6])
@pytest.mark.parametrize("rnd", [0, 1])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dist", ["normal", "relu", "t3"])
def test_quantize_bit_exact(shape, fmt, rnd, dist):
    log("quantize", shape, fmt, rnd, dist)
    seed = 1234567 + 17 * rnd
    x = workloads.random_array(shape, seed=sum(shape) + len(dist), dist=dist)
    q = gpu_quantize(to_dev(x), shape, fmt, mq.MQ_ROLE_ACT, rnd, seed)
    torch.cuda.synchronize()
    assert_quant_equal(q, oracle.quantize(x, fmt, rnd, seed), fmt, f"{shape} {fmt} {rnd}")


SPECIAL = {
    "zeros": lambda s: np.zeros(s, np.float32),
    "neg_zeros": lambda s: -np.zeros(s, np.float32),
    "nan": lambda s: _with(workloads.random_array(s, 3), (0, 0, 1, 1), np.nan),
    "inf": lambda s: _with(workloads.random_array(s, 3), (0, 1, 2, 0), np.inf),
    "ninf": lambda s: _with(workloads.random_array(s, 3), (0, 1, 2, 0), -np.inf),
    "tiny": lambda s: (workloads.random_array(s, 4) * np.float32(1e-38)).astype(np.float32),
    "denormal": lambda s: (workloads.random_array(s, 5) * np.float32(1e-42)).astype(np.float32),
    "huge": lambda s: (workloads.random_array(s, 6) * np.float32(1e37)).astype(np.float32),
    "onehot": lambda s: _with(np.zeros(s, np.float32), (0, 0, 0, 0), 1.0),
    "sparse_zero_squares": lambda s: _zero_some(workloads.random_array(s, 7)),
    "ties": lambda s: _ties(s),
    "neg_zero_elements": lambda s: _neg_zero_elements(s),
}


def _neg_zero_elements(s):
    # -0.0 elements inside squares with a non-zero scale: their codes keep the sign bit of x
    a = workloads.random_array(s, 8)
    a.reshape(-1)[1::3] = -0.0
    a.reshape(-1)[2::7] = 0.0
    return a


def _with(a, idx, v):
    a = a.copy()
    a[idx] = v
    return a


def _zero_some(a):
    a = a.copy()
    a[:, :, :4, :4] = 0.0
    a[:, :, 4:8, :] = -0.0
    return a


def _ties(s):
    # values whose quotients land exactly on grid midpoints (T = 1, B = 448 squares)
    rng = np.random.default_rng(0)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.0625, 0.1875, 7.25, 6.75],
                    np.float32)
    a = rng.choice(mids, size=s).astype(np.float32) * 448
    a.reshape(-1)[0] = 2688.0
    return a * np.where(rng.random(s) < 0.5, -1, 1).astype(np.float32)


@pytest.mark.parametrize("fmt", [4, 6])
@pytest.mark.parametrize("rnd", [0, 1])
@pytest.mark.parametrize("case", sorted(SPECIAL))
def test_quantize_special_values(case, fmt, rnd):
    shape = (2, 3, 9, 10)
    log("quantize special", case, fmt, rnd)
    x = SPECIAL[case](shape)
    q = gpu_quantize(to_dev(x), shape, fmt, mq.MQ_ROLE_ACT, rnd, 99)
    torch.cuda.synchronize()
    assert_quant_equal(q, oracle.quantize(x, fmt, rnd, 99), fmt, case)


def _layer_tensors(name):
    out = []
    for layer in workloads.CONFIGS[name]():
        x, w, g = workloads.make_tensors(layer)
        out.append((layer, x, w, g))
    return out


@pytest.mark.parametrize("cfg", ["c1", "c2", "c3", "c4", "c5"])
def test_quantize_full_size_layers(cfg):
    """Every tensor of the workload layers at full size, through GPU relayout + quantize."""
    layers = workloads.CONFIGS[cfg]()
    if cfg == "c5":
        layers = layers[:2] + layers[4:7]  # one of each shape class keeps the run short
    for layer in layers:
        log("full-size quantize", layer.name)
        x, w, g = workloads.make_tensors(layer)
        N, Ci, H, W, Co, Kh, Kw = (layer.N, layer.Cin, layer.H, layer.W, layer.Cout, layer.Kh,
                                   layer.Kw)
        for name, a, shape, role, rnd, seed in (
                ("x", x, (H, W, Ci, N), mq.MQ_ROLE_ACT, 0, 0),
                ("w", w, (Kh, Kw, Co, Ci), mq.MQ_ROLE_WEIGHT, 0, 0),
                ("g", g, (layer.Ho, layer.Wo, Co, N), mq.MQ_ROLE_GRAD, 1, layer.sr_seed)):
            t = to_dev(a)
            dst = torch.empty(a.size, dtype=torch.float32, device="cuda")
            if name == "w":
                mq.mq_relayout_weight(t, dst, Co, Ci, Kh, Kw, 0)
                ref_src = oracle.oihw_to_tap_major(a)
            else:
                n_, c_, h_, w_ = a.shape
                mq.mq_relayout_cbf(t, dst, n_, c_, h_, w_, 0)
                ref_src = oracle.nchw_to_cbf(a)
            torch.cuda.synchronize()
            assert np.array_equal(dst.cpu().numpy().reshape(ref_src.shape), ref_src), \
                f"{layer.name} {name}: relayout differs"
            q = gpu_quantize(dst, shape, layer.fmt, role, rnd, seed)
            torch.cuda.synchronize()
            assert_quant_equal(q, oracle.quantize(ref_src, layer.fmt, rnd, seed), layer.fmt,
                               f"{layer.name}.{name}")


@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (3, 5, 7, 2), (2, 70, 9, 130), (64, 3, 1, 1)])
def test_relayout_roundtrip(shape):
    N, C, H, W = shape
    x = workloads.random_array(shape, seed=8)
    t = to_dev(x)
    c = torch.empty(x.size, dtype=torch.float32, device="cuda")
    back = torch.empty_like(c)
    mq.mq_relayout_cbf(t, c, N, C, H, W, 0)
    mq.mq_relayout_cbf(c, back, N, C, H, W, 1)
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy().reshape(H, W, C, N), oracle.nchw_to_cbf(x))
    assert np.array_equal(back.cpu().numpy().reshape(shape), x)
    w = workloads.random_array((C, N, 3, 2), seed=9)
    tw = to_dev(w)
    tm = torch.empty(w.size, dtype=torch.float32, device="cuda")
    wb = torch.empty_like(tm)
    mq.mq_relayout_weight(tw, tm, C, N, 3, 2, 0)
    mq.mq_relayout_weight(tm, wb, C, N, 3, 2, 1)
    torch.cuda.synchronize()
    assert np.array_equal(tm.cpu().numpy().reshape(3, 2, C, N), oracle.oihw_to_tap_major(w))
    assert np.array_equal(wb.cpu().numpy().reshape(w.shape), w)


def test_quantize_is_deterministic_and_seeded():
    shape = (4, 4, 16, 16)
    x = workloads.random_array(shape, seed=10)
    t = to_dev(x)
    a = gpu_quantize(t, shape, 4, mq.MQ_ROLE_GRAD, 1, 5)
    b = gpu_quantize(t, shape, 4, mq.MQ_ROLE_GRAD, 1, 5)
    c = gpu_quantize(t, shape, 4, mq.MQ_ROLE_GRAD, 1, 6)
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
    assert not torch.equal(a.codes, c.codes)
    assert torch.equal(a.scales, c.scales)


FUSED_CASES = [
    ("normal", (3, 7, 5, 9)), ("relu", (32, 64, 14, 14)), ("t3", (4, 12, 9, 10)),
    ("nan", (2, 3, 9, 10)), ("zeros", (2, 3, 9, 10)), ("denormal", (2, 3, 9, 10)),
]


@pytest.mark.parametrize("fmt", [4, 6])
@pytest.mark.parametrize("case,shape", FUSED_CASES)
def test_relayout_amax_then_quantize(case, shape, fmt):
    """The relayouts can write the tensor-amax partials; quantizing with MQ_QUANTIZE_AMAX_READY
    then skips the amax pass and must give the same bytes as the oracle."""
    log("relayout+amax", case, shape, fmt)
    N, C, H, W = shape
    x = SPECIAL[case](shape) if case in SPECIAL else workloads.random_array(shape, 21, dist=case)
    ws = mq.quantize_workspace()
    t = to_dev(x)
    xc = torch.empty(x.size, dtype=torch.float32, device="cuda")
    mq.mq_relayout_cbf(t, xc, N, C, H, W, 0, amax_ws=ws)
    for rnd in (0, 1):
        q = mq.QTensor(H, W, C, N, fmt, mq.MQ_ROLE_ACT)
        mq.mq_quantize(xc, q, rnd, 77, ws, mq.MQ_QUANTIZE_AMAX_READY)
        torch.cuda.synchronize()
        assert_quant_equal(q, oracle.quantize(oracle.nchw_to_cbf(x), fmt, rnd, 77), fmt,
                           f"cbf {case} {rnd}")
    # weights: OIHW (Cout, Cin, Kh, Kw) = shape
    wt = torch.empty(x.size, dtype=torch.float32, device="cuda")
    mq.mq_relayout_weight(t, wt, N, C, H, W, 0, amax_ws=ws)
    q = mq.QTensor(H, W, N, C, fmt, mq.MQ_ROLE_WEIGHT)
    mq.mq_quantize(wt, q, 0, 0, ws, mq.MQ_QUANTIZE_AMAX_READY)
    torch.cuda.synchronize()
    assert_quant_equal(q, oracle.quantize(oracle.oihw_to_tap_major(x), fmt, 0, 0), fmt,
                       f"weight {case}")


# ---- activations and gradients straight from NCHW (mq_quantize_nchw) ----------------------

NCHW_SHAPES = [  # (N, C, H, W): batch and channel counts off and on multiples of 4 and 16,
    # pixel counts below, at and past whole 64-pixel waves
    (1, 1, 1, 1), (2, 3, 5, 7), (4, 4, 8, 8), (5, 9, 3, 11), (16, 8, 8, 8), (32, 64, 14, 14),
    (7, 20, 9, 13), (12, 6, 16, 9), (8, 16, 1, 64), (3, 130, 2, 33),
]


@pytest.mark.parametrize("fmt", [4, 6])
@pytest.mark.parametrize("rnd", [0, 1])
@pytest.mark.parametrize("shape", NCHW_SHAPES)
def test_quantize_nchw_matches_relayout_then_quantize(shape, fmt, rnd):
    """Codes, scales and T bit-exact against the oracle's quantization of the channel-batch-first
    tensor, with the amax pass inside the call and with partials from a relayout."""
    N, C, H, W = shape
    log("quantize_nchw", shape, fmt, rnd)
    x = workloads.random_array(shape, seed=N * 31 + C + H, dist="relu" if rnd == 0 else "normal")
    seed = 4242 + rnd
    ref = oracle.quantize(oracle.nchw_to_cbf(x), fmt, rnd, seed)
    t = to_dev(x)
    role = mq.MQ_ROLE_GRAD if rnd else mq.MQ_ROLE_ACT
    ws = mq.quantize_workspace()
    q = mq.QTensor(H, W, C, N, fmt, role)
    mq.mq_quantize_nchw(t, q, rnd, seed, ws)
    torch.cuda.synchronize()
    assert_quant_equal(q, ref, fmt, f"nchw {shape} {fmt} {rnd}")
    # amax partials written by a relayout of the same values
    xc = torch.empty(x.size, dtype=torch.float32, device="cuda")
    ws2 = mq.quantize_workspace()
    mq.mq_relayout_cbf(t, xc, N, C, H, W, 0, amax_ws=ws2)
    q2 = mq.QTensor(H, W, C, N, fmt, role)
    mq.mq_quantize_nchw(t, q2, rnd, seed, ws2, mq.MQ_QUANTIZE_AMAX_READY)
    torch.cuda.synchronize()
    assert_quant_equal(q2, ref, fmt, f"nchw amax-ready {shape} {fmt} {rnd}")


@pytest.mark.parametrize("fmt", [4, 6])
@pytest.mark.parametrize("case", ["zeros", "neg_zeros", "nan", "inf", "tiny", "denormal", "huge",
                                  "sparse_zero_squares", "ties", "neg_zero_elements"])
def test_quantize_nchw_special_values(case, fmt):
    shape = (2, 3, 9, 10)
    x = SPECIAL[case](shape)
    for rnd in (0, 1):
        q = mq.QTensor(9, 10, 3, 2, fmt, mq.MQ_ROLE_ACT)
        mq.mq_quantize_nchw(to_dev(x), q, rnd, 99, mq.quantize_workspace())
        torch.cuda.synchronize()
        assert_quant_equal(q, oracle.quantize(oracle.nchw_to_cbf(x), fmt, rnd, 99), fmt,
                           f"nchw {case} {rnd}")


@pytest.mark.parametrize("cfg", ["c2", "c3", "c5"])
def test_quantize_nchw_full_size_layers(cfg):
    """The layer inputs (RNE) and output gradients (SR) of the workloads at full size."""
    layers = workloads.CONFIGS[cfg]()
    if cfg == "c5":
        layers = [layers[0], layers[5]]  # the largest input and a stride-2 output gradient
    for layer in layers:
        log("full-size quantize_nchw", layer.name)
        x, _, g = workloads.make_tensors(layer)
        for name, a, role, rnd, seed in (("x", x, mq.MQ_ROLE_ACT, 0, 0),
                                         ("g", g, mq.MQ_ROLE_GRAD, 1, layer.sr_seed)):
            n_, c_, h_, w_ = a.shape
            q = mq.QTensor(h_, w_, c_, n_, layer.fmt, role)
            mq.mq_quantize_nchw(to_dev(a), q, rnd, seed, mq.quantize_workspace())
            torch.cuda.synchronize()
            assert_quant_equal(q, oracle.quantize(oracle.nchw_to_cbf(a), layer.fmt, rnd, seed),
                               layer.fmt, f"{layer.name}.{name}")


def test_quantize_nchw_rejects_weight_role():
    q = mq.QTensor(3, 3, 8, 8, 4, mq.MQ_ROLE_WEIGHT, "cuda")
    with pytest.raises(mq.MQError):
        mq.mq_quantize_nchw(torch.zeros(8, 8, 3, 3, device="cuda"), q, 0, 0,
                            mq.quantize_workspace("cuda"))


# ---- several tensors in one launch pair (mq_quantize_batch) ---------------------------------

def _oracle_for(layout, a, fmt, rnd, seed):
    if layout == mq.MQ_SRC_NCHW:
        return oracle.quantize(oracle.nchw_to_cbf(a), fmt, rnd, seed)
    if layout == mq.MQ_SRC_OIHW:
        return oracle.quantize(oracle.oihw_to_tap_major(a), fmt, rnd, seed)
    return oracle.quantize(a, fmt, rnd, seed)


BATCHES = {
    # a layer's forward pass: X from NCHW and W from OIHW together
    "x_w": [(mq.MQ_SRC_NCHW, (32, 64, 14, 14), mq.MQ_ROLE_ACT, 0),
            (mq.MQ_SRC_OIHW, (64, 64, 3, 3), mq.MQ_ROLE_WEIGHT, 0)],
    # every source order and both roundings, ragged shapes
    "mixed": [(mq.MQ_SRC_NCHW, (5, 9, 7, 11), mq.MQ_ROLE_ACT, 0),
              (mq.MQ_SRC_OIHW, (17, 13, 3, 3), mq.MQ_ROLE_WEIGHT, 0),
              (mq.MQ_SRC_DENSE, (6, 7, 20, 12), mq.MQ_ROLE_GRAD, 1),
              (mq.MQ_SRC_NCHW, (16, 8, 9, 9), mq.MQ_ROLE_GRAD, 1)],
    "one": [(mq.MQ_SRC_DENSE, (3, 5, 13, 18), mq.MQ_ROLE_ACT, 1)],
}


def _batch_tensors(name, fmt):
    out = []
    for i, (layout, shape, role, rnd) in enumerate(BATCHES[name]):
        a = workloads.random_array(shape, seed=300 + 7 * i, dist="relu" if rnd == 0 else "normal")
        a.reshape(-1)[3::11] = -0.0  # negative zeros inside squares with a non-zero scale
        if layout == mq.MQ_SRC_NCHW:
            n, c, h, w_ = shape
            qshape = (h, w_, c, n)
        elif layout == mq.MQ_SRC_OIHW:
            co, ci, kh, kw = shape
            qshape = (kh, kw, co, ci)
        else:
            qshape = shape
        out.append((layout, a, qshape, role, rnd, 1000 + i))
    return out


@pytest.mark.parametrize("fmt", [4, 6])
@pytest.mark.parametrize("name", sorted(BATCHES))
def test_quantize_batch_matches_single_calls(name, fmt):
    log("quantize_batch", name, fmt)
    items = _batch_tensors(name, fmt)
    keep, jobs = [], []
    for layout, a, qshape, role, rnd, seed in items:
        t = to_dev(a)
        q = mq.QTensor(*qshape, fmt, role)
        ws = mq.quantize_workspace()
        keep.append((t, q, ws))
        jobs.append(mq.quant_job(t, layout, q, rnd, seed, ws))
    mq.mq_quantize_batch(jobs)
    torch.cuda.synchronize()
    for (layout, a, qshape, role, rnd, seed), (_, q, _) in zip(items, keep):
        assert_quant_equal(q, _oracle_for(layout, a, fmt, rnd, seed), fmt,
                           f"batch {name} layout {layout} {qshape}")


def test_quantize_batch_amax_ready_and_special_values():
    """A job whose partial maxima come from a relayout, next to jobs holding NaN and zeros."""
    shape = (8, 12, 9, 10)
    x = workloads.random_array(shape, seed=5)
    nan = SPECIAL["nan"](shape)
    zeros = np.zeros((16, 4, 3, 3), np.float32)
    tx, tn, tz = to_dev(x), to_dev(nan), to_dev(zeros)
    ws = [mq.quantize_workspace() for _ in range(3)]
    xc = torch.empty(x.size, dtype=torch.float32, device="cuda")
    mq.mq_relayout_cbf(tx, xc, 8, 12, 9, 10, 0, amax_ws=ws[0])
    qx = mq.QTensor(9, 10, 12, 8, 4, mq.MQ_ROLE_ACT)
    qn = mq.QTensor(9, 10, 12, 8, 4, mq.MQ_ROLE_GRAD)
    qz = mq.QTensor(3, 3, 16, 4, 4, mq.MQ_ROLE_WEIGHT)
    mq.mq_quantize_batch([
        mq.quant_job(tx, mq.MQ_SRC_NCHW, qx, 0, 0, ws[0], mq.MQ_QUANTIZE_AMAX_READY),
        mq.quant_job(tn, mq.MQ_SRC_NCHW, qn, 1, 3, ws[1]),
        mq.quant_job(tz, mq.MQ_SRC_OIHW, qz, 0, 0, ws[2])])
    torch.cuda.synchronize()
    assert_quant_equal(qx, oracle.quantize(oracle.nchw_to_cbf(x), 4, 0, 0), 4, "amax ready")
    assert_quant_equal(qn, oracle.quantize(oracle.nchw_to_cbf(nan), 4, 1, 3), 4, "nan")
    assert_quant_equal(qz, oracle.quantize(oracle.oihw_to_tap_major(zeros), 4, 0, 0), 4, "zeros")


# ---- weights straight from OIHW (mq_quantize_weight) -------------------------------------

WEIGHT_SHAPES = [  # (Cout, Cin, Kh, Kw): small (one launch) and large (amax pass + gather)
    (1, 1, 1, 1), (5, 3, 3, 3), (16, 16, 3, 3), (24, 20, 3, 3), (64, 64, 3, 3), (17, 13, 1, 1),
    (36, 70, 5, 5), (128, 128, 3, 3), (130, 67, 3, 3), (256, 64, 1, 1),
]


@pytest.mark.parametrize("fmt", [4, 6])
@pytest.mark.parametrize("rnd", [0, 1])
@pytest.mark.parametrize("wshape", WEIGHT_SHAPES)
def test_quantize_weight_from_oihw(wshape, fmt, rnd):
    Co, Ci, Kh, Kw = wshape
    log("quantize_weight", wshape, fmt, rnd)
    w = workloads.random_array(wshape, seed=Co * 7 + Ci, dist="kaiming", fan_in=Ci * Kh * Kw)
    seed = 99 + rnd
    q = mq.QTensor(Kh, Kw, Co, Ci, fmt, mq.MQ_ROLE_WEIGHT, "cuda")
    ws = mq.quantize_workspace("cuda")
    mq.mq_quantize_weight(to_dev(w), q, rnd, seed, ws)
    torch.cuda.synchronize()
    ref = oracle.quantize(oracle.oihw_to_tap_major(w), fmt, rnd, seed)
    assert_quant_equal(q, ref, fmt, f"{wshape} {fmt} {rnd}")


@pytest.mark.parametrize("wshape", [(64, 64, 3, 3), (128, 128, 3, 3)])
def test_quantize_weight_special_values(wshape):
    Co, Ci, Kh, Kw = wshape
    negz = workloads.random_array(wshape, 6)
    negz.reshape(-1)[1::3] = -0.0
    for name, w in (("zeros", np.zeros(wshape, np.float32)),
                    ("inf", _with(workloads.random_array(wshape, 5), (1, 2, 0, 1), np.inf)),
                    ("neg_zero_elements", negz)):
        q = mq.QTensor(Kh, Kw, Co, Ci, 4, mq.MQ_ROLE_WEIGHT, "cuda")
        mq.mq_quantize_weight(to_dev(w), q, 0, 0, mq.quantize_workspace("cuda"))
        torch.cuda.synchronize()
        ref = oracle.quantize(oracle.oihw_to_tap_major(w), 4, 0, 0)
        assert_quant_equal(q, ref, 4, f"{wshape} {name}")


def test_quantize_weight_rejects_wrong_role():
    q = mq.QTensor(3, 3, 8, 8, 4, mq.MQ_ROLE_ACT, "cuda")
    w = torch.zeros(8, 8, 3, 3, device="cuda")
    with pytest.raises(mq.MQError):
        mq.mq_quantize_weight(w, q, 0, 0, mq.quantize_workspace("cuda"))
