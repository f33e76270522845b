"""Exact rational model of the decode step, for pinning the CPU oracle (test helper).

Every real-valued quantity is a ``fractions.Fraction``; IEEE rounding to binary32 / binary16
and round-half-to-even to an integer are written here from their definitions (nearest
representable value, ties to the even significand), independent of the oracle's C code and of
any floating-point unit. Used only on tiny states (D <= 16).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def rne_int(x: Fraction) -> int:
    """Round to the nearest integer, ties to even."""
    fl = x.numerator // x.denominator
    r = x - fl
    if r > Fraction(1, 2):
        return fl + 1
    if r < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def _ilog2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_binary(x: Fraction, p: int, emin: int, emax: int):
    """Nearest IEEE value with p significand bits, minimum normal exponent emin and maximum
    exponent emax (ties to even); returns a Fraction, or +-inf (float) on overflow."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = max(_ilog2(a), emin)
    quantum = Fraction(2) ** (e - (p - 1))
    n = rne_int(a / quantum)
    val = n * quantum
    if val >= Fraction(2) ** (emax + 1):
        return sign * float("inf")
    return sign * val


def f32(x: Fraction):
    return round_binary(x, 24, -126, 127)


def f16(x: Fraction):
    return round_binary(x, 11, -14, 15)


def f16_bits(x: Fraction) -> int:
    """binary16 bit pattern of the (already representable or infinite) value x."""
    return int(np.array([float(x)], np.float64).astype(np.float16).view(np.uint16)[0])


def quant_row_exact(xf: list[Fraction]):
    """INT8 row rule on binary32 values xf: m = max|x|, s = f32(m/127), c = rne(f32(x/s)),
    clamped to [-127, 127]; m == 0 -> s = 0, c = 0."""
    m = max(abs(x) for x in xf)
    if m == 0:
        return [0] * len(xf), Fraction(0)
    s = f32(m / 127)
    codes = [max(-127, min(127, rne_int(f32(x / s)))) for x in xf]
    return codes, s


def step_exact(D, fmt, mask, S32, h, c, s, q, k, v, alpha, beta):
    """One unit, exact. fmt 0: S32 float32 [D, D]; fmt 1: mask [D], h uint16 [D, D],
    c int8 [D, D], s float32 [D]. alpha: scalar or [D]. Returns a dict with
    ``out`` (float32 [D]) and the new state in the unit's format, plus ``X`` (exact)."""
    F = Fraction
    a = [F(float(alpha))] * D if np.ndim(alpha) == 0 else [F(float(x)) for x in alpha]
    qq = [F(float(x)) for x in q]
    kk = [F(float(x)) for x in k]
    vv = [F(float(x)) for x in v]
    bb = F(float(beta))
    if fmt == 0:
        Sh = [[F(float(S32[i, j])) for j in range(D)] for i in range(D)]
    else:
        hf = h.view(np.float16).astype(np.float64)
        Sh = [[F(float(hf[i, j])) if mask[i] else int(c[i, j]) * F(float(s[i]))
               for j in range(D)] for i in range(D)]
    Sp = [[a[i] * Sh[i][j] for j in range(D)] for i in range(D)]
    u = [sum(kk[i] * Sp[i][j] for i in range(D)) for j in range(D)]
    delta = [bb * (vv[j] - u[j]) for j in range(D)]
    X = [[Sp[i][j] + kk[i] * delta[j] for j in range(D)] for i in range(D)]
    o = [sum(qq[i] * X[i][j] for i in range(D)) for j in range(D)]
    res = {"X": X, "out": np.array([float(f32(x)) for x in o], np.float32)}
    Xf = [[f32(X[i][j]) for j in range(D)] for i in range(D)]
    if fmt == 0:
        res["S32"] = np.array([[float(x) for x in row] for row in Xf], np.float32)
        return res
    hn = np.zeros((D, D), np.uint16)
    cn = np.zeros((D, D), np.int8)
    sn = np.zeros(D, np.float32)
    for i in range(D):
        if mask[i]:
            hn[i] = [f16_bits(f16(x)) for x in Xf[i]]
        else:
            codes, sc = quant_row_exact(Xf[i])
            cn[i] = codes
            sn[i] = float(sc)
    res.update(h=hn, c=cn, s=sn)
    return res
