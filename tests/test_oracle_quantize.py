"""Pins of the oracle's square-block quantizer (CPU only).

Checked against hand-derived worked squares (tests/golden/), closed-form invariants of the NVFP4 /
NVFP6 recipe (onedev.kr MicroQonv digest, section "How it differs": tensor scale, E4M3 block scale
per 4x4 square, element rounding; RNE for weights/activations, stochastic rounding for
gradients), and statistics of the stochastic rounding.
"""
import os
import zlib

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            d[k.strip()] = v.split()
    return d


@pytest.mark.parametrize("name", ["quantize_fp4_square.txt", "quantize_fp4_subnormal_scale.txt",
                                  "quantize_fp6_square.txt"])
def test_golden_worked_squares(name):
    g = _read_golden(name)
    fmt = int(g["fmt"][0])
    rnd = oracle.RNE if g["round"][0] == "rne" else oracle.SR
    shape = tuple(int(v) for v in g["shape"])
    x = np.array([float(v) for v in g["x"]], np.float32).reshape(shape)
    codes, scales, T = oracle.quantize(x, fmt, rnd)
    assert T == np.float32(float(g["T"][0]))
    assert list(scales) == [int(v, 0) for v in g["scales"]]
    assert list(codes.reshape(-1)) == [int(v, 0) for v in g["codes"]]
    packed = oracle.pack(codes, fmt)
    if "packed" in g:
        assert list(packed) == [int(v, 0) for v in g["packed"]]
    # FP6 layout: element e of a square is bits [6e, 6e+6) of its little-endian 96-bit word
    for t in range(codes.shape[0]):
        nb = 8 if fmt == 4 else 12
        word = int.from_bytes(bytes(packed[nb * t: nb * (t + 1)]), "little")
        bits = 4 if fmt == 4 else 6
        assert word == sum(int(c) << (bits * e) for e, c in enumerate(codes[t]))


def _grid(fmt):
    return np.array([oracle.elem_value(fmt, c) for c in range(8 if fmt == 4 else 32)])


def _square_view(x):
    """[O0][O1][R][S] -> per-square element arrays [nsq, 16] (padded with NaN) in the square
    order of the library: t = ((o0*O1 + o1)*R4 + r/4)*S4 + s/4, e = (r%4)*4 + s%4."""
    O0, O1, R, S = x.shape
    R4, S4 = -(-R // 4), -(-S // 4)
    pad = np.full((O0, O1, R4 * 4, S4 * 4), np.nan, np.float64)
    pad[:, :, :R, :S] = x
    v = pad.reshape(O0, O1, R4, 4, S4, 4).transpose(0, 1, 2, 4, 3, 5)
    return v.reshape(-1, 16)


CASES = [
    ((3, 2, 9, 6), "relu", 4),
    ((2, 3, 8, 8), "t3", 4),
    ((1, 4, 13, 7), "silu", 6),
    ((2, 2, 16, 33), "normal", 6),
    ((3, 3, 5, 2), "normal", 4),
    ((1, 1, 1, 1), "normal", 4),
]


@pytest.mark.parametrize("shape,dist,fmt", CASES)
def test_rne_invariants(shape, dist, fmt):
    x = workloads.random_array(shape, seed=zlib.crc32(repr((shape, dist)).encode()) % 1000,
                               dist=dist)
    codes, scales, T = oracle.quantize(x, fmt, oracle.RNE)
    grid = _grid(fmt)
    emax = grid[-1]
    sbit = 8 if fmt == 4 else 32
    # tensor scale: T * 448 * emax reproduces amax to within an fp32 rounding
    amax = float(np.abs(x).max())
    assert abs(float(T) * 448 * emax - amax) <= amax * 2.0 ** -23
    sq = _square_view(x)
    real = ~np.isnan(sq)
    assert (codes[~real] == 0).all(), "padded slots must hold code 0"
    assert (scales <= 0x7E).all()
    B = np.array([oracle.e4m3_value(int(s)) for s in scales])
    zero_sq = scales == 0
    assert (codes[zero_sq] == 0).all()
    mag = (codes & (sbit - 1)).astype(np.int64)
    E = np.where(codes & sbit, -1, 1) * grid[mag]
    with np.errstate(invalid="ignore", divide="ignore"):
        q = sq / (B[:, None] * float(T))  # exact-real quotient (double)
    ok = real & ~zero_sq[:, None]
    aq = np.abs(q[ok])
    e_ok = E[ok]
    # signs follow the input
    assert (np.signbit(e_ok) == np.signbit(sq[ok])).all()
    # nearest grid point: error at most half the local grid step (+ fp32 quotient slack)
    idx = np.clip(np.searchsorted(grid, aq, side="right") - 1, 0, len(grid) - 2)
    step = grid[idx + 1] - grid[idx]
    inside = aq <= emax
    err = np.abs(np.abs(e_ok) - aq)
    assert (err[inside] <= step[inside] / 2 + aq[inside] * 2.0 ** -22).all()
    assert (np.abs(e_ok[~inside]) == emax).all(), "beyond the largest element it saturates"
    # the square maximum of a normal-scale square lands on the top codes
    normal = (scales >= 8) & ~zero_sq
    for t in np.nonzero(normal)[0]:
        j = np.nanargmax(np.abs(sq[t]))
        top = {7} if fmt == 4 else {30, 31}
        assert int(mag[t, j]) in top
    # dequantized values reproduce the input within the grid bound
    xh = oracle.dequant(codes, scales, T, shape, fmt)
    assert np.all(np.abs(xh - x) <= np.abs(x) * 0.25 + float(T) * 448 * 0.5 + 1e-30)


@pytest.mark.parametrize("fmt", [4, 6])
def test_scale_invariance_by_powers_of_two(fmt):
    x = workloads.random_array((2, 2, 12, 9), seed=3, dist="t3")
    c0, s0, T0 = oracle.quantize(x, fmt, oracle.RNE)
    for k in (-20, -3, 5, 30):
        c1, s1, T1 = oracle.quantize(x * np.float32(2.0 ** k), fmt, oracle.RNE)
        assert (c0 == c1).all() and (s0 == s1).all()
        assert T1 == np.float32(T0 * 2.0 ** k)
    c2, s2, _ = oracle.quantize(x * np.float32(2.0 ** -3), fmt, oracle.SR, seed=9)
    c3, s3, _ = oracle.quantize(x, fmt, oracle.SR, seed=9)
    assert (c2 == c3).all() and (s2 == s3).all()


def test_square_locality():
    """Changing one element (not the tensor max) only changes its own 4x4 square."""
    x = workloads.random_array((2, 3, 10, 11), seed=4)
    x[0, 0, 0, 0] = 50.0  # pin the tensor max
    c0, s0, T0 = oracle.quantize(x, 4, oracle.RNE)
    rng = np.random.default_rng(0)
    for _ in range(20):
        o0, o1, r, s = rng.integers(0, 2), rng.integers(0, 3), rng.integers(0, 10), rng.integers(0, 11)
        if (o0, o1, r, s) == (0, 0, 0, 0):
            continue
        y = x.copy()
        y[o0, o1, r, s] = 7.5
        c1, s1, T1 = oracle.quantize(y, 4, oracle.RNE)
        assert T1 == T0
        t = ((o0 * 3 + o1) * 3 + r // 4) * 3 + s // 4
        diff = np.nonzero((c0 != c1).any(1) | (s0 != s1))[0]
        assert set(diff) <= {t} and t in diff


def test_zero_and_nonfinite_tensors():
    z = np.zeros((1, 2, 5, 6), np.float32)
    c, s, T = oracle.quantize(z, 4, oracle.RNE)
    assert T == 0 and (s == 0).all() and (c == 0).all()
    for bad in (np.nan, np.inf, -np.inf):
        y = workloads.random_array((1, 2, 5, 6), seed=1)
        y[0, 1, 3, 2] = bad
        for fmt in (4, 6):
            c, s, T = oracle.quantize(y, fmt, oracle.RNE)
            assert np.isnan(T) and np.float32(T).view(np.uint32) == 0x7FC00000
            assert (s == 0x7F).all() and (c == 0).all()
            xh = oracle.dequant(c, s, T, y.shape, fmt)
            assert np.isnan(xh).all()
    # a square of zeros in a non-zero tensor: scale 0, codes 0 (even for -0.0)
    y = workloads.random_array((1, 1, 8, 8), seed=2)
    y[0, 0, 4:8, 0:4] = 0.0
    y[0, 0, 5, 1] = -0.0
    c, s, T = oracle.quantize(y, 4, oracle.RNE)
    assert s[2] == 0 and (c[2] == 0).all()


def test_negative_zero_and_tiny_keep_sign():
    x = np.array([[[[6.0, -0.0, -1e-3, 1e-3]]]], np.float32)
    c, s, T = oracle.quantize(x, 4, oracle.RNE)
    assert list(c[0, :4]) == [7, 8, 8, 0]


@pytest.mark.parametrize("fmt", [4, 6])
def test_sr_neighbours_and_unbiased(fmt):
    x = workloads.random_array((1, 2, 8, 8), seed=11)
    grid = _grid(fmt)
    sbit = 8 if fmt == 4 else 32
    seeds = range(1, 3001)
    acc = np.zeros(x.shape)
    c_rne, s_rne, T_rne = oracle.quantize(x, fmt, oracle.RNE)
    for sd in seeds:
        c, s, T = oracle.quantize(x, fmt, oracle.SR, seed=sd)
        assert (s == s_rne).all() and T == T_rne  # scales do not depend on the rounding
        acc += oracle.dequant(c, s, T, x.shape, fmt)
    mean = acc / len(seeds)
    # per element: E[dequant] = x up to the 2^-16 probability grid; the noise of the sample
    # mean is at most step * D / (2 sqrt(S))
    B = np.array([oracle.e4m3_value(int(v)) for v in s_rne])
    D = B * float(T_rne)
    sq = _square_view(x)
    step_max = np.diff(grid).max()
    tol_sq = D[:, None] * step_max * (5 / (2 * np.sqrt(len(seeds))) + 2.0 ** -16) + 1e-12
    err_sq = np.abs(_square_view(mean) - sq)
    real = ~np.isnan(sq)
    # (elements beyond the largest grid value saturate deterministically, so they are biased)
    unsat = real & (np.abs(sq / D[:, None]) <= grid[-1])
    assert unsat.sum() > 100
    assert (err_sq[unsat] <= np.broadcast_to(tol_sq, sq.shape)[unsat]).all()
    # every SR code is one of the two grid neighbours of |q|
    c, s, T = oracle.quantize(x, fmt, oracle.SR, seed=77)
    q = np.abs(sq / D[:, None])
    E = grid[(c & (sbit - 1)).astype(np.int64)]
    lo_i = np.clip(np.searchsorted(grid, q, side="right") - 1, 0, len(grid) - 1)
    hi_i = np.minimum(lo_i + 1, len(grid) - 1)
    okm = real
    assert ((E[okm] == grid[lo_i[okm]]) | (E[okm] == grid[hi_i[okm]])).all()


def test_sr_uses_per_element_draws():
    """Two squares holding identical values round differently (their counters differ), and the
    same seed reproduces the same codes."""
    v = np.full((1, 1, 4, 4), 0.3, np.float32)
    x = np.concatenate([v, v], axis=3)
    x[0, 0, 0, 0] = x[0, 0, 0, 4] = 6.0
    c1, _, _ = oracle.quantize(x, 4, oracle.SR, seed=5)
    c2, _, _ = oracle.quantize(x, 4, oracle.SR, seed=5)
    assert (c1 == c2).all()
    assert (c1[0] != c1[1]).any()


@pytest.mark.parametrize("fmt", [4, 6])
def test_pack_roundtrip(fmt):
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16 if fmt == 4 else 64, size=(37, 16), dtype=np.uint8)
    p = oracle.pack(codes, fmt)
    assert p.size == 37 * (8 if fmt == 4 else 12)
    assert (oracle.unpack(p, 37, fmt) == codes).all()
