"""Pins of the oracle's fp32 operation order in the square-block quantizer (CPU only).

The recipe (onedev.kr MicroQonv digest, section "How it differs") writes the tensor scale as
amax / (448 * emax), the square-scale quotient as bmax / (T * emax) and the element quotient as
x / (B * T). The reading taken is fp32 with one rounding per operation in that order. The golden
rows tests/golden/quantize_order_fp{4,6}.txt were derived from those formulas in exact rational
arithmetic (tests/golden/derive_order_squares.py, which uses neither the oracle nor the GPU
library), with a non-power-of-two T and with square maxima and elements placed next to E4M3 and
element-grid rounding midpoints, so that (amax/448)/emax, (bmax/T)/emax, bmax*(1/(T*emax)),
(x/B)/T and x*(1/(B*T)) each change the tensor scale, a square scale or a code.
"""
import importlib.util
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _derivation():
    spec = importlib.util.spec_from_file_location(
        "derive_order_squares", os.path.join(GOLDEN, "derive_order_squares.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


D = _derivation()


def _read(fmt):
    g = {}
    with open(os.path.join(GOLDEN, f"quantize_order_fp{fmt}.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(":", 1)
                g[k.strip()] = v.split()
    shape = tuple(int(v) for v in g["shape"])
    x = np.array([float.fromhex(v) for v in g["x"]], np.float32).reshape(shape)
    T_bits = int(g["T_bits"][0], 0)
    scales = [int(v, 0) for v in g["scales"]]
    codes = [int(v, 0) for v in g["codes"]]
    return x, T_bits, scales, codes


def _flat(result):
    T, scales, codes = result
    return D.bits(T), list(scales), [c for sq in codes for c in sq]


@pytest.mark.parametrize("fmt", [4, 6])
def test_oracle_matches_order_squares(fmt):
    x, T_bits, scales, codes = _read(fmt)
    c, s, T = oracle.quantize(x, fmt, oracle.RNE)
    assert int(np.float32(T).view(np.uint32)) == T_bits, "tensor scale bits"
    assert list(s) == scales
    assert list(c.reshape(-1)) == codes


@pytest.mark.parametrize("fmt", [4, 6])
def test_order_squares_follow_the_written_formulas(fmt):
    """The stored outputs are what the formulas give in exact rationals with fp32 roundings."""
    x, T_bits, scales, codes = _read(fmt)
    xs = D.read_x(os.path.join(GOLDEN, f"quantize_order_fp{fmt}.txt"))
    assert [float(v) for row in xs for v in row] == [float(v) for v in x.reshape(-1)]
    assert _flat(D.quantize_row(xs, fmt)) == (T_bits, scales, codes)


@pytest.mark.parametrize("fmt", [4, 6])
@pytest.mark.parametrize("variant", D.STEPS)
def test_every_reassociation_changes_the_order_squares(fmt, variant):
    """Each plausible re-association of one step gives other bits, so an oracle that computed
    it would fail test_oracle_matches_order_squares."""
    xs = D.read_x(os.path.join(GOLDEN, f"quantize_order_fp{fmt}.txt"))
    _, T_bits, scales, codes = _read(fmt)
    assert _flat(D.quantize_row(xs, fmt, variant)) != (T_bits, scales, codes)


def test_fp32_rounding_helper():
    """The exact-rational fp32 rounding agrees with numpy's float32 cast (a library special
    case) on doubles near ties, subnormals and powers of two."""
    from fractions import Fraction as F
    rng = np.random.default_rng(5)
    vals = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 30, 2000))
    for e in (-149, -127, -126, -1, 0, 23, 60):
        base = 2.0 ** e
        vals += [base, base * (1 + 2.0 ** -24), base * (1 - 2.0 ** -25), base * (1 + 3 * 2.0 ** -24)]
    for v in vals:
        assert float(D.f32(F(v))) == float(np.float32(v)), v
