"""Exact-rational brute force for tiny inputs, independent of the oracle.

Everything here works on fractions.Fraction values and emulates each IEEE
rounding explicitly (round half to even at a given significand width), so it
shares no arithmetic with numpy's float32/float64 operations that the oracle
relies on.  Used only to pin the oracle on tiny inputs.
"""
from __future__ import annotations

from decimal import Decimal, getcontext
from fractions import Fraction
from typing import List, Sequence, Tuple

# (significand bits incl. hidden bit, minimum normal exponent, maximum exponent)
BINARY16 = (11, -14, 15)
BINARY32 = (24, -126, 127)
BINARY64 = (53, -1022, 1023)


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_rne(x: Fraction, fmt=BINARY32) -> Fraction:
    """Round an exact rational to the nearest value of a binary format (ties to even)."""
    p, emin, emax = fmt
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(Fraction(x))
    e = max(_floor_log2(a), emin)
    ulp = Fraction(2) ** (e - p + 1)
    m = a / ulp
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    res = n * ulp
    if res >= Fraction(2) ** (emax + 1):
        raise OverflowError("rounded value overflows the format")
    return sign * res


def rint_even(x: Fraction) -> int:
    """Nearest integer, halves to even."""
    n = x.numerator // x.denominator
    r = x - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def f16_to_fraction(h) -> Fraction:
    """Exact value of an fp16 number given as a Python float or numpy scalar."""
    return Fraction(float(h))


def quantize_group(ws: Sequence[Fraction], qmax: int = 15,
                   symmetric: bool = False) -> Tuple[Fraction, Fraction, List[int]]:
    """One group, each binary32 operation rounded explicitly:
    step = r32(r32(max - min) / qmax), zero = rint(r32(-min / step)),
    q = clamp(rint(r32(w / step)) + zero, 0, qmax).
    Symmetric: step = r32(max|w| / h) and zero = h with h = (qmax + 1) / 2."""
    mn, mx = min(ws), max(ws)
    if symmetric:
        h = (qmax + 1) // 2
        step = round_rne(max(abs(mn), abs(mx)) / h)
        if step == 0:
            step = Fraction(1)
        zero = Fraction(h)
        q = [int(min(max(rint_even(round_rne(w / step)) + zero, 0), qmax)) for w in ws]
        return step, zero, q
    step = round_rne(round_rne(mx - mn) / qmax)
    if step == 0:
        step = Fraction(1)
    zero = Fraction(rint_even(round_rne(-mn / step)))
    q = []
    for w in ws:
        v = rint_even(round_rne(w / step)) + zero
        q.append(int(min(max(v, 0), qmax)))
    return step, zero, q


def fake_quant_row(w_row: Sequence[Fraction], s_row: Sequence[Fraction], group: int = 128,
                   qmax: int = 15, symmetric: bool = False):
    """Quantize-dequantize one weight row: ws = r32(w s), group quantization,
    t = r32((q - zero) step), wq = r16(t * r32(1/s)).  Returns (wq, codes)."""
    ws = [round_rne(w * s) for w, s in zip(w_row, s_row)]
    wq: List[Fraction] = []
    codes: List[int] = []
    for g0 in range(0, len(ws), group):
        step, zero, q = quantize_group(ws[g0:g0 + group], qmax, symmetric)
        for j, qq in enumerate(q):
            t = round_rne((qq - zero) * step)
            inv_s = round_rne(Fraction(1) / s_row[g0 + j])
            wq.append(round_rne(t * inv_s, BINARY16))
        codes.extend(q)
    return wq, codes


def mse_exact(X: Sequence[Sequence[Fraction]], W: Sequence[Sequence[Fraction]],
              Wq: Sequence[Sequence[Fraction]]) -> Fraction:
    """Exact mean over tokens and outputs of (x . (wq - w))^2."""
    total = Fraction(0)
    for x in X:
        for w, wq in zip(W, Wq):
            d = sum((xi * (b - a) for xi, a, b in zip(x, w, wq)), Fraction(0))
            total += d * d
    return total / (len(X) * len(W))


def mean_abs_exact(col: Sequence[Fraction]) -> Fraction:
    return sum((abs(v) for v in col), Fraction(0)) / len(col)


def pow_decimal(base: Fraction, alpha: Fraction, digits: int = 60) -> Fraction:
    """base ** alpha to `digits` significant digits via Decimal exp/ln."""
    getcontext().prec = digits
    b = Decimal(base.numerator) / Decimal(base.denominator)
    a = Decimal(alpha.numerator) / Decimal(alpha.denominator)
    if a == 0:
        return Fraction(1)
    v = (a * b.ln()).exp()
    return Fraction(v)
