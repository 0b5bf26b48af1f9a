"""Pins of the oracle's number formats against library casts and closed forms (CPU only).

The formats are the ones the MicroQonv pages name (onedev.kr digest, section "How it differs":
E4M3 block scales and E2M1 elements; section "How it is used": E2M3 elements for NVFP6). The
pages print no tables, so the pins are torch's float8_e4m3fn type (a library implementation of
E4M3) and numpy's round-half-to-even on exactly scaled values.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _floats_in(lo: float, hi: float) -> np.ndarray:
    """Every float32 in [lo, hi) (lo, hi >= 0)."""
    a = np.array([lo, hi], np.float32).view(np.uint32)
    return np.arange(a[0], a[1], dtype=np.uint32).view(np.float32)


def _chunks(lo, hi, size=1 << 24):
    a = np.array([lo, hi], np.float32).view(np.uint32)
    start, stop = int(a[0]), int(a[1])
    for s in range(start, stop, size):
        yield np.arange(s, min(s + size, stop), dtype=np.uint32).view(np.float32)


# ---- E4M3 ----------------------------------------------------------------------------------

def test_e4m3_decode_matches_torch_float8():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = np.array([oracle.e4m3_value(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert (nan == np.isnan(got)).all()
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert (got[~nan] == ref[~nan]).all()
    # sign symmetric, largest finite value 448, smallest subnormal 2^-9
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e4m3_cast_exhaustive_matches_torch():
    """CastE4M3 = round-to-nearest-even with subnormals: every float32 in [2^-12, 448]."""
    for a in _chunks(2.0 ** -12, 448.0):
        ref = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = oracle.e4m3_cast(a)
        bad = np.nonzero(ref != got)[0]
        assert bad.size == 0, (a[bad[:5]], ref[bad[:5]], got[bad[:5]])
    assert oracle.e4m3_cast(np.array([448.0], np.float32))[0] == 0x7E


def test_e4m3_cast_small_and_saturating():
    tiny = _floats_in(0.0, 2.0 ** -12)[:: 4099]
    assert (oracle.e4m3_cast(tiny) == 0).all()
    # 2^-10 is the midpoint between 0 and the smallest subnormal 2^-9: ties to even (0)
    v = np.array([2.0 ** -10, np.nextafter(np.float32(2.0 ** -10), np.float32(1)), 2.0 ** -9],
                 np.float32)
    assert list(oracle.e4m3_cast(v)) == [0, 1, 1]
    # (448, 464) rounds to 448 in torch too; above that torch gives NaN, the oracle saturates
    mid = _floats_in(448.0, 464.0)[::97]
    ref = torch.from_numpy(mid).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ref == 0x7E).all() and (oracle.e4m3_cast(mid) == 0x7E).all()
    big = np.array([464.0, 1e6, 3e38, np.inf], np.float32)
    assert (oracle.e4m3_cast(big) == 0x7E).all()
    assert oracle.e4m3_cast(np.array([np.nan], np.float32))[0] == 0x7F


# ---- element grids -------------------------------------------------------------------------

def test_element_grids_are_e4m3_subsets():
    """E2M1 and E2M3 magnitudes are exact E4M3 values (same exponent field semantics)."""
    e4 = {oracle.e4m3_value(c) for c in range(127)}
    g4 = [oracle.elem_value(4, c) for c in range(8)]
    g6 = [oracle.elem_value(6, c) for c in range(32)]
    assert all(v in e4 for v in g4) and all(v in e4 for v in g6)
    assert g4 == sorted(g4) and g6 == sorted(g6)
    assert max(g4) == 6.0 and max(g6) == 7.5 and g4[1] == 0.5 and g6[1] == 0.125
    # the sign bit mirrors
    assert [oracle.elem_value(4, c | 8) for c in range(8)] == [-v for v in g4]
    assert [oracle.elem_value(6, c | 32) for c in range(32)] == [-v for v in g6]
    # E2M3 grid: k/8 below 1, then 8 steps per binade up to 7.5
    assert g6 == [k / 8 for k in range(8)] + [1 + k / 8 for k in range(8)] \
        + [2 + k / 4 for k in range(8)] + [4 + k / 2 for k in range(8)]


def _e2m1_pin(a: np.ndarray) -> np.ndarray:
    """Nearest E2M1 magnitude code, ties to even, from round-half-even on exact rescalings:
    codes 0..4 are 2a on [0,2], codes 4..6 are a+2 on [2,4], codes 6..7 are a/2+4 above."""
    a64 = a.astype(np.float64)
    c = np.where(a64 < 2, np.round(2 * a64), np.where(a64 < 4, np.round(a64) + 2,
                                                      np.round(a64 / 2) + 4))
    return np.minimum(c, 7).astype(np.uint8)


def _e2m3_pin(a: np.ndarray) -> np.ndarray:
    """Nearest E2M3 magnitude code: below 1 it is round-half-even(8a); on [1, 7.5] the E2M3 grid
    equals the E4M3 grid, so torch's float8_e4m3fn cast rounds it; above 7.75 it saturates."""
    grid = np.array([oracle.elem_value(6, c) for c in range(32)])
    sub = np.round(a.astype(np.float64) * 8)
    f8 = torch.from_numpy(np.minimum(a, np.float32(7.5))).to(torch.float8_e4m3fn).double().numpy()
    hic = np.searchsorted(grid, f8)
    return np.where(a < 1, sub, hic).astype(np.uint8)


@pytest.mark.parametrize("fmt", [4, 6])
def test_element_rne_exhaustive(fmt):
    """Every float32 in [2^-7, 16): the oracle's nearest-even grid rounding equals the pin."""
    pin = _e2m1_pin if fmt == 4 else _e2m3_pin
    for a in _chunks(2.0 ** -7, 16.0):
        got = oracle.elem_rne(fmt, a)
        ref = pin(a)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (a[bad[:5]], got[bad[:5]], ref[bad[:5]])
    tiny = _floats_in(0.0, 2.0 ** -7)[:: 1009]
    assert (oracle.elem_rne(fmt, tiny) == 0).all()
    assert (oracle.elem_rne(fmt, np.array([16.0, 1e30, np.inf], np.float32)) ==
            (7 if fmt == 4 else 31)).all()


def test_element_rne_ties_to_even_code():
    mids4 = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    assert list(oracle.elem_rne(4, mids4)) == [0, 2, 2, 4, 4, 6, 6]
    mids6 = np.array([1 / 16, 3 / 16, 15 / 16, 1.0625, 1.9375, 2.125, 3.875, 5.25, 7.25],
                     np.float32)
    assert list(oracle.elem_rne(6, mids6)) == [0, 2, 8, 8, 16, 16, 24, 26, 30]


# ---- stochastic rounding -------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [4, 6])
def test_sr_probability_is_exact_fraction(fmt):
    """Over all 65536 values of u16 the number of round-ups is ceil(frac * 2^16), with frac the
    exact rational position of a between its grid neighbours."""
    from fractions import Fraction
    grid = [oracle.elem_value(fmt, c) for c in range(8 if fmt == 4 else 32)]
    rng = np.random.default_rng(5)
    a = np.concatenate([rng.uniform(0, grid[-1], 300).astype(np.float32),
                        np.array(grid[:-1], np.float32),
                        np.array([np.nextafter(np.float32(g), np.float32(0)) for g in grid[1:]],
                                 np.float32)])
    u = np.arange(65536, dtype=np.uint32)
    for ai in a:
        codes = oracle.elem_sr(fmt, np.full(65536, ai, np.float32), u)
        lo = max(i for i, g in enumerate(grid) if g <= float(ai))
        assert set(np.unique(codes)) <= {lo, lo + 1}
        frac = (Fraction(float(ai)) - Fraction(grid[lo])) / (Fraction(grid[lo + 1]) - Fraction(grid[lo]))
        ups = int((codes == lo + 1).sum())
        assert ups == math.ceil(frac * 65536)
        # the round-ups are exactly the smallest u16 values
        assert (codes[:ups] == lo + 1).all() and (codes[ups:] == lo).all()
    sat = oracle.elem_sr(fmt, np.full(4, grid[-1] * 1.01, np.float32), u[:4])
    assert (sat == len(grid) - 1).all()


# Known-answer vectors of Philox4x32-10 distributed with the Random123 library that accompanies
# Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11):
# (counter, key) -> output, all as 32-bit words.
PHILOX4X32_10_KAT = [
    ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
    ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
    ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
     [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
]


@pytest.mark.parametrize("ctr,key,out", PHILOX4X32_10_KAT)
def test_philox_known_answers(ctr, key, out):
    got = oracle.philox4x32_10(ctr, np.array(key, np.uint32))
    assert [int(v) for v in got] == out


def test_sr_u16_slices_philox_words():
    """The SR draw of element e of square t is 16-bit half (e & 1) of Philox word (e & 7) >> 1
    for counter j = 2t + (e >> 3), key = (seed low, seed high)."""
    seed = 0x0123456789ABCDEF
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32)
    for t in (0, 1, 5, (1 << 31) + 3):
        words = [oracle.philox4x32_10([(2 * t + h) & 0xFFFFFFFF, (2 * t + h) >> 32, 0, 0], key)
                 for h in (0, 1)]
        e = np.arange(16, dtype=np.int32)
        u = oracle.sr_u16(seed, np.full(16, t, np.int64), e)
        want = [(int(words[k >> 3][(k & 7) >> 1]) >> (16 * (k & 1))) & 0xFFFF for k in range(16)]
        assert [int(v) for v in u] == want


def test_sr_uniforms_statistics():
    """u16 slices are uniform and the 16 elements of a square see distinct draws."""
    t = np.repeat(np.arange(1 << 16, dtype=np.int64), 16)
    e = np.tile(np.arange(16, dtype=np.int32), 1 << 16)
    u = oracle.sr_u16(12345, t, e)
    assert u.max() < 65536
    counts = np.bincount((u >> 8).astype(np.int64), minlength=256)
    exp = u.size / 256
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 400  # 255 dof: mean 255, sd ~22.6
    m = u.reshape(-1, 16).astype(np.float64)
    c = np.corrcoef(m.T)
    assert np.abs(c - np.eye(16)).max() < 0.02
    # different seeds give unrelated streams
    u2 = oracle.sr_u16(12346, t, e)
    assert (u == u2).mean() < 0.001
    # avalanche: flipping one counter bit flips about half the output bits
    k = np.array([7, 9], np.uint32)
    o1 = oracle.philox4x32_10([1, 0, 0, 0], k)
    o2 = oracle.philox4x32_10([3, 0, 0, 0], k)
    flips = sum(bin(int(a) ^ int(b)).count("1") for a, b in zip(o1, o2))
    assert 40 < flips < 88
