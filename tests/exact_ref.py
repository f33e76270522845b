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
    clamped to [-127, 127]; s == 0 (m == 0, or m/127 below half the smallest subnormal) ->
    c = 0."""
    m = max(abs(x) for x in xf)
    s = f32(m / 127)
    if s == 0:
        return [0] * len(xf), Fraction(0)
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


# ------------------------------------------------------------------------------------------
# STEPQuant-style state (the STEPQuant page, appendix Table C2 steps 1-6; the fit's formulas
# are this repository's reading of the page's description): pivot rows in binary16, integer
# rows of b in {8, 6, 4} bits with a binary16 row factor each and one binary16 column-scale
# vector per unit, fitted from the new state X (rounded once to binary32) over the non-pivot
# rows N with squared row-impact weights w_i:
#   cs_j = the binary16 value nearest to sqrt(sum_N w_i^2 X_ij^2 / sum_N w_i^2)
#          (all w_i = 0 on N: every weight 1)
#   rf_i = f16(f32(max over j with cs_j > 0 of f32(|X_ij| / cs_j) / qmax)),  qmax = 2^(b-1) - 1
#   code = clamp(rne(f32(X_ij / (rf_i cs_j))), -qmax, qmax), 0 where rf_i cs_j = 0
# Here every quantity is exact (Fraction) up to the roundings the statement names; the square
# root is rounded to binary16 directly from the exact ratio, by comparing squares.
# ------------------------------------------------------------------------------------------
def _isqrt_floor(x: Fraction) -> int:
    """Largest integer n >= 0 with n^2 <= x."""
    from math import isqrt
    return isqrt(x.numerator // x.denominator)


def sqrt_round_binary(R: Fraction, p: int, emin: int, emax: int):
    """The IEEE value with p significand bits nearest to sqrt(R) (R >= 0), ties to even, from
    the exact R: n = floor(sqrt(R) / quantum) by an integer square root, then the half-way
    point compared by squares. Returns (value, distance of sqrt(R) to the nearest tie point in
    units of the quantum, as a float, for callers that want to know how close it came)."""
    if R == 0:
        return Fraction(0), float("inf")
    e = _ilog2(R) // 2      # 2^(2e) <= R < 2^(2e+2) up to the floor: sqrt(R) in [2^e, 2^(e+1))
    while Fraction(2) ** (2 * e) > R:
        e -= 1
    while Fraction(2) ** (2 * e + 2) <= R:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (p - 1))
    n = _isqrt_floor(R / (quantum * quantum))
    mid2 = (Fraction(2 * n + 1, 2) * quantum) ** 2
    if R > mid2:
        n += 1
    elif R == mid2 and n % 2 == 1:
        n += 1
    val = n * quantum
    if val >= Fraction(2) ** (emax + 1):
        return float("inf"), float("inf")
    # how far sqrt(R) lies from the tie point (n_floor + 1/2) quantum, relative to the quantum
    import math
    s = math.sqrt(float(R / (quantum * quantum)))
    return val, abs(s - (math.floor(s) + 0.5))


def f16_value(bits) -> Fraction:
    return Fraction(float(np.array([bits], np.uint16).view(np.float16)[0]))


def stq_step_exact(D, bits, w, h, c, rf, cs, q, k, v, alpha, beta, cs_near_tie=None):
    """One STEPQuant-style unit, exact. bits [D] (16 = pivot, 8, 6, 4), w [D] float32 row-impact
    scores, h uint16 [D, D], c int8 [D, D], rf uint16 [D], cs uint16 [D]; alpha scalar or [D].
    Returns dict(out float32 [D], h, c, rf, cs (new state), tie [D]: for each column, how close
    sqrt of its weighted mean square came to a binary16 tie, in quanta).
    cs_near_tie: optional dict j -> binary16 bits, used for column j instead of the exact value
    (for a column whose square root lies so close to a tie that binary64 evaluation may take the
    other side)."""
    F = Fraction
    a = [F(float(alpha))] * D if np.ndim(alpha) == 0 else [F(float(x)) for x in alpha]
    qq = [F(float(x)) for x in q]
    kk = [F(float(x)) for x in k]
    vv = [F(float(x)) for x in v]
    bb = F(float(beta))
    piv = [int(b) == 16 for b in bits]
    rfv = [f16_value(x) for x in rf]
    csv = [f16_value(x) for x in cs]
    Sh = [[f16_value(h[i, j]) if piv[i] else int(c[i, j]) * rfv[i] * csv[j] for j in range(D)]
          for i in range(D)]
    Sp = [[a[i] * Sh[i][j] for j in range(D)] for i in range(D)]
    u = [sum(kk[i] * Sp[i][j] for i in range(D)) for j in range(D)]
    delta = [bb * (vv[j] - u[j]) for j in range(D)]
    X = [[Sp[i][j] + kk[i] * delta[j] for j in range(D)] for i in range(D)]
    y = [sum(qq[i] * X[i][j] for i in range(D)) for j in range(D)]
    Xf = [[f32(X[i][j]) for j in range(D)] for i in range(D)]
    N = [i for i in range(D) if not piv[i]]
    w2 = {i: F(float(w[i])) ** 2 for i in N}
    if sum(w2.values()) == 0:
        w2 = {i: F(1) for i in N}
    sw = sum(w2.values())
    cs_new, tie = [], []
    for j in range(D):
        if not N:
            cs_new.append(F(0))
            tie.append(float("inf"))
            continue
        R = sum(w2[i] * Xf[i][j] ** 2 for i in N) / sw
        val, t = sqrt_round_binary(R, 11, -14, 15)
        if cs_near_tie and j in cs_near_tie:
            val = f16_value(cs_near_tie[j])
        cs_new.append(val)
        tie.append(t)
    hn, cn, rfn = stq_rows_exact(D, bits, Xf, cs_new)
    return {"out": np.array([float(f32(x)) for x in y], np.float32), "h": hn, "c": cn, "rf": rfn,
            "cs": np.array([f16_bits(x) for x in cs_new], np.uint16), "tie": np.array(tie)}


def stq_rows_exact(D, bits, Xf, cs_new):
    """The fit's second half: pivot values, row factors and codes of the binary32 state Xf
    (Fractions [D][D]) for the column scales cs_new (Fractions, binary16 values)."""
    hn = np.zeros((D, D), np.uint16)
    cn = np.zeros((D, D), np.int8)
    rfn = np.zeros(D, np.uint16)
    for i in range(D):
        if int(bits[i]) == 16:
            hn[i] = [f16_bits(f16(x)) for x in Xf[i]]
            continue
        qm = 2 ** (int(bits[i]) - 1) - 1
        m = max([f32(abs(Xf[i][j]) / cs_new[j]) for j in range(D) if cs_new[j] > 0], default=Fraction(0))
        r = f16(f32(m / qm))
        rfn[i] = f16_bits(r)
        for j in range(D):
            sc = r * cs_new[j]
            if sc > 0:
                cn[i, j] = max(-qm, min(qm, rne_int(f32(Xf[i][j] / sc))))
    return hn, cn, rfn
