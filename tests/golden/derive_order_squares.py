"""Exact-rational derivation of the operation-order worked squares (test infrastructure).

The NVFP4 / NVFP6 recipe of the onedev.kr MicroQonv digest, section "How it differs", writes
three quotients:

    T = max|X| / (max B_sf * max B_ef)          tensor scale, max B_sf = 448 (E4M3)
    B = CastE4M3(max|X_i| / (T * max B_ef))      per 4x4 square
    code = Round(X_i / (B * T))                  per element

with max B_ef = 6 (E2M1) or 7.5 (E2M3). The reading taken (fp32, every operation rounded once,
in the written order, IEEE division) is fixed by these squares: they are chosen so that each
plausible re-association gives a different tensor scale, square scale or code:

    "T/448/emax"    T = (amax / 448) / emax            instead of amax / (448 * emax)
    "bmax/T/emax"   s = (bmax / T) / emax              instead of bmax / (T * emax)
    "bmax*recip"    s = bmax * (1 / (T * emax))        (a reciprocal instead of the division)
    "x/B/T"         q = (x / B) / T                    instead of x / (B * T)
    "x*recip"       q = x * (1 / (B * T))              (a reciprocal instead of the division)

Everything here is exact rational arithmetic (fractions.Fraction) with an explicit
round-to-nearest-even to fp32 after every operation; E4M3 and the element grids are decoded from
their bit fields. It uses neither the oracle nor the GPU library. `python derive_order_squares.py`
writes quantize_order_fp4.txt and quantize_order_fp6.txt next to it; the oracle tests check the
oracle against those files and re-run this derivation to check that the files are what the
formulas give and that every re-association above changes them.
"""
from __future__ import annotations

import os
import struct
from fractions import Fraction as F

HERE = os.path.dirname(os.path.abspath(__file__))

STEPS = ("T/448/emax", "bmax/T/emax", "bmax*recip", "x/B/T", "x*recip")


# ---- fp32 as exact rationals -------------------------------------------------------------

def f32(r: F) -> F:
    """Round a rational to the nearest fp32 value, ties to even (no overflow in this use)."""
    if r == 0:
        return F(0)
    neg = r < 0
    a = -r if neg else r
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    # now 2^e <= a < 2^(e+1)
    ulp = F(2) ** (e - 23) if e >= -126 else F(2) ** -149
    n = a / ulp
    q, rem = divmod(n.numerator, n.denominator)
    if 2 * rem > n.denominator or (2 * rem == n.denominator and q % 2 == 1):
        q += 1
    v = q * ulp
    return -v if neg else v


def next_up(v: F) -> F:
    """The next fp32 value above a positive fp32 value."""
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if F(2) ** e > v:
        e -= 1
    return v + (F(2) ** (e - 23) if e >= -126 else F(2) ** -149)


def next_down(v: F) -> F:
    e = v.numerator.bit_length() - v.denominator.bit_length()
    if F(2) ** e > v:
        e -= 1
    if v == F(2) ** e and e > -126:
        e -= 1  # the step below a power of two is half as large
    return v - (F(2) ** (e - 23) if e >= -126 else F(2) ** -149)


def to_hex(v: F) -> str:
    return float(v).hex()  # fp32 values are exact doubles


def bits(v: F) -> int:
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


# ---- formats, decoded from their bit fields -----------------------------------------------

def e4m3_table():
    """Finite non-negative E4M3 values, codes 0x00..0x7E: s|eeee|mmm, bias 7, subnormal m/2^9."""
    out = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        out.append(F(m, 512) if e == 0 else (1 + F(m, 8)) * F(2) ** (e - 7))
    return out


def elem_table(fmt: int):
    """Element magnitudes: E2M1 (s|ee|m) or E2M3 (s|ee|mmm), bias 1, subnormal m/2^mant."""
    mant = 1 if fmt == 4 else 3
    out = []
    for c in range(1 << (2 + mant)):
        e, m = c >> mant, c & ((1 << mant) - 1)
        out.append(F(m, 1 << mant) if e == 0 else (1 + F(m, 1 << mant)) * F(2) ** (e - 1))
    return out


E4M3 = e4m3_table()


def nearest_even(table, a: F) -> int:
    """Index of the entry nearest to a >= 0, ties to the even index, saturating at the top."""
    if a >= table[-1]:
        return len(table) - 1
    hi = next(i for i, v in enumerate(table) if v > a)
    lo = hi - 1
    mid = (table[lo] + table[hi]) / 2
    if a < mid:
        return lo
    if a > mid:
        return hi
    return lo if lo % 2 == 0 else hi


def emax_of(fmt: int) -> F:
    return F(6) if fmt == 4 else F(15, 2)


# ---- the recipe with one step possibly re-associated --------------------------------------

def tensor_scale(amax: F, fmt: int, variant: str | None = None) -> F:
    if variant == "T/448/emax":
        return f32(f32(amax / 448) / emax_of(fmt))
    return f32(amax / (448 * emax_of(fmt)))  # 448 * emax = 2688 or 3360, exact


def square_scale(bmax: F, T: F, fmt: int, variant: str | None = None) -> int:
    emax = emax_of(fmt)
    if variant == "bmax/T/emax":
        s = f32(f32(bmax / T) / emax)
    elif variant == "bmax*recip":
        s = f32(bmax * f32(1 / f32(T * emax)))
    else:
        s = f32(bmax / f32(T * emax))
    return nearest_even(E4M3, s)


def element_code(x: F, B: F, T: F, fmt: int, variant: str | None = None) -> int:
    if variant == "x/B/T":
        q = f32(f32(x / B) / T)
    elif variant == "x*recip":
        q = f32(x * f32(1 / f32(B * T)))
    else:
        q = f32(x / f32(B * T))
    mag = nearest_even(elem_table(fmt), abs(q))
    sign = 8 if fmt == 4 else 32
    return mag | (sign if x < 0 else 0)


def quantize_row(xs, fmt: int, variant: str | None = None):
    """One row of 4x4 squares: xs is [4][4*nsq] (rows r, columns s). Returns (T, scales,
    codes per square in element order e = 4*r + s%4). Non-zero finite values only matter."""
    nsq = len(xs[0]) // 4
    amax = max(abs(v) for row in xs for v in row)
    T = tensor_scale(amax, fmt, variant)
    scales, codes = [], []
    for t in range(nsq):
        sq = [xs[r][4 * t + c] for r in range(4) for c in range(4)]
        bmax = max(abs(v) for v in sq)
        b = square_scale(bmax, T, fmt, variant) if bmax > 0 else 0
        scales.append(b)
        B = E4M3[b]
        codes.append([element_code(v, B, T, fmt, variant) if B > 0 else 0 for v in sq])
    return T, scales, codes


# ---- the search for discriminating values ---------------------------------------------------

def _scan(center: F, radius: int):
    """fp32 values within `radius` steps of the fp32 value nearest `center` (nearest first)."""
    c = f32(center)
    yield c
    up, down = c, c
    for _ in range(radius):
        up, down = next_up(up), next_down(down)
        yield up
        yield down


def find_bmax(T: F, fmt: int, variant: str):
    """A square max whose E4M3 scale changes under `variant` (near a midpoint of the E4M3 grid),
    or None."""
    TE = f32(T * emax_of(fmt))
    for k in range(56, 104):  # E4M3 codes of the binades [2^-1, 2^5)
        mid = (E4M3[k] + E4M3[k + 1]) / 2
        for b in _scan(mid * TE, 3):
            if square_scale(b, T, fmt) != square_scale(b, T, fmt, variant):
                return b
    return None


def find_amax(fmt: int):
    """The first fp32 amax at or above 1.7 whose tensor scale depends on the order and for whose
    T both scale re-associations have a discriminating square max. Returns (amax, b1, b2)."""
    a = f32(F(17, 10))
    while True:
        if tensor_scale(a, fmt) != tensor_scale(a, fmt, "T/448/emax"):
            T = tensor_scale(a, fmt)
            b1 = find_bmax(T, fmt, "bmax/T/emax")
            b2 = find_bmax(T, fmt, "bmax*recip") if b1 is not None else None
            if b2 is not None:
                return a, b1, b2
        a = next_up(a)


def find_elements(B: F, T: F, fmt: int, variant: str, radius: int = 3):
    """Element values whose code changes under `variant`: near midpoints of the element grid."""
    grid = elem_table(fmt)
    D = f32(B * T)
    found = []
    for k in range(1, len(grid) - 1):
        mid = (grid[k] + grid[k + 1]) / 2
        for x in _scan(mid * D, radius):
            if element_code(x, B, T, fmt) != element_code(x, B, T, fmt, variant):
                found.append(x)
                break
    return found


def find_quotient_square(T: F, fmt: int, variant: str, want: int = 4):
    """A square scale B (not a power of two, so that B*T rounds) and up to `want` element values
    whose codes change under `variant`; the scale with the most such values wins."""
    best = (None, [])
    for code in range(0x30, 0x50):  # E4M3 binades [2^-1, 2^3)
        if code & 7 == 0:
            continue
        B = E4M3[code]
        xs = find_elements(B, T, fmt, variant)
        if len(xs) > len(best[1]):
            best = (B, xs)
        if len(xs) >= want:
            break
    if best[0] is None:
        raise RuntimeError(f"no discriminating element for {variant}")
    return best[0], best[1][:want]


def build_case(fmt: int):
    """A 4 x 20 row of five squares: square 0 holds the tensor max; squares 1 and 2 each hold a
    square max that one scale re-association moves across an E4M3 rounding midpoint; squares 3
    and 4 have scales that are not powers of two (so B*T rounds) and elements that one quotient
    re-association each moves across element-grid midpoints (some negated)."""
    amax, b1, b2 = find_amax(fmt)
    T = tensor_scale(amax, fmt)
    TE = f32(T * emax_of(fmt))
    xs = [[F(0)] * 20 for _ in range(4)]
    xs[0][0] = amax
    xs[1][4] = b1
    xs[2][9] = b2
    for t, variant in ((3, "x/B/T"), (4, "x*recip")):
        B, elems = find_quotient_square(T, fmt, variant)
        bmax = f32(B * TE)
        assert E4M3[square_scale(bmax, T, fmt)] == B
        xs[0][4 * t] = bmax
        slots = [(r, 4 * t + c) for r in range(4) for c in range(4) if (r, c) != (0, 0)]
        for i, v in enumerate(elems):
            r, c = slots[3 * i + 1]  # spread over the square
            xs[r][c] = -v if i % 2 == 1 else v
    return xs


def describe(xs, fmt: int):
    """Golden-file lines: derivation comments, inputs and expected outputs."""
    T, scales, codes = quantize_row(xs, fmt)
    emax = emax_of(fmt)
    TE = f32(T * emax)
    lines = [
        f"# Operation-order square row, NVFP{fmt} ({'E2M1' if fmt == 4 else 'E2M3'} elements), "
        f"round-to-nearest. Derived in exact rationals",
        "# with an fp32 rounding after every operation by derive_order_squares.py (no oracle, no "
        "GPU) from the recipe of the",
        "# onedev.kr MicroQonv digest, section \"How it differs\": T = amax / (448 * emax), "
        "B = CastE4M3(bmax / (T * emax)),",
        f"# code = Round(x / (B * T)), emax = {float(emax)}; the reading: fp32, written order, "
        "IEEE division, ties to even.",
        f"# amax = {to_hex(xs[0][0])}: T = fp32(amax / {448 * emax}) = {to_hex(T)} "
        f"(bits {bits(T):#010x}); (amax / 448) / emax would give "
        f"{to_hex(tensor_scale(xs[0][0], fmt, 'T/448/emax'))}",
        f"# T * emax = {to_hex(TE)}",
    ]
    nsq = len(xs[0]) // 4
    for t in range(nsq):
        sq = [xs[r][4 * t + c] for r in range(4) for c in range(4)]
        bmax = max(abs(v) for v in sq)
        s = f32(bmax / TE)
        lines.append(f"# square {t}: bmax = {to_hex(bmax)}, bmax / (T * emax) = {to_hex(s)} -> "
                     f"scale {scales[t]:#04x} ({float(E4M3[scales[t]])}); "
                     f"bmax/T/emax -> {square_scale(bmax, T, fmt, 'bmax/T/emax'):#04x}, "
                     f"reciprocal -> {square_scale(bmax, T, fmt, 'bmax*recip'):#04x}")
        B = E4M3[scales[t]]
        D = f32(B * T)
        for e, v in enumerate(sq):
            if v == 0 or v == bmax:
                continue
            q = f32(v / D)
            lines.append(f"#   e{e}: x = {to_hex(v)}, x / (B*T) = {to_hex(q)} -> code "
                         f"{codes[t][e]:#04x}; x/B/T -> "
                         f"{element_code(v, B, T, fmt, 'x/B/T'):#04x}, reciprocal -> "
                         f"{element_code(v, B, T, fmt, 'x*recip'):#04x}")
    flat = [v for row in xs for v in row]
    lines += [
        f"fmt: {fmt}",
        "round: rne",
        f"shape: 1 1 4 {len(xs[0])}",
        "x: " + " ".join(to_hex(v) for v in flat),
        f"T_bits: {bits(T):#010x}",
        "scales: " + " ".join(f"{s:#04x}" for s in scales),
        "codes: " + " ".join(f"{c:#04x}" for sq in codes for c in sq),
    ]
    return lines


def read_x(path: str):
    """The input row of a golden file as exact rationals [4][S]."""
    with open(path) as f:
        for line in f:
            if line.startswith("x:"):
                vals = [F(float.fromhex(v)) for v in line.split(":", 1)[1].split()]
                n = len(vals) // 4
                return [vals[n * r:n * (r + 1)] for r in range(4)]
    raise ValueError(f"{path}: no x line")


def main():
    for fmt in (4, 6):
        xs = build_case(fmt)
        path = os.path.join(HERE, f"quantize_order_fp{fmt}.txt")
        with open(path, "w") as f:
            f.write("\n".join(describe(xs, fmt)) + "\n")
        print(path)


if __name__ == "__main__":
    main()
