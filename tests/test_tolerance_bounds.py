"""CPU checks of the error bounds the GPU tests take as tolerance windows (no GPU): the
STEPQuant-style fit's binary32 lane sums, the codes-held STEPQuant-style step's column sums
from int8 pieces of the row weights, and the fp32-state step's per-element bound.

The STEPQuant-style step sums each lane's rows of (w_i X_ij)^2 in binary32 (one binary32 value
per element, then one fused multiply-add per row, 8 rows per lane at d = 128 and d = 64) and adds
the 16 lane partials, divides by the sum of w_i^2 and takes the square root in binary64. At
d = 128 the value is w_i Y_ij = w_i X_ij / cs_j formed from the codes (its binary64 total is then
multiplied by cs_j^2, exactly); at d = 64 it is w_i X_ij rounded once. Either is within a few
ulps of the exact product, the same few ulps by which the device's X differs; emulated here as
one rounding. For positive terms the lane sum is within (8 + 2) u of the exact one (u = 2^-24),
so the column scale before its binary16 rounding is within 5u (relative) of the binary64 fit of
the same values. The GPU test allows a column scale to differ from the oracle's only where the
oracle's value lies within 1e-6 of a binary16 tie, which needs this 5u (3e-7) plus the few ulps
by which the device's X (or w Y) differs.
Here the device's arithmetic is emulated exactly (each binary32 product and fused
multiply-add rounded once from its exact rational value) on random and adversarial columns,
against exact sums.
"""
import math
from fractions import Fraction

import numpy as np

U = 2.0 ** -24
ROWS_PER_LANE = 8
LANES = 16


def _round32(q):
    """The binary32 value nearest the rational q, ties to even (one rounding)."""
    f = np.float32(float(q))
    best = None
    for g in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(g)) - q)
        even = (int(np.array(g, np.float32).view(np.uint32)) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, g)
    return best[1]


def _fma32(a, b, c):
    """fl32(a * b + c), rounded once from the exact value."""
    return _round32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def _device_scale(w, x):
    """w [128], x [128] (binary32): the column scale before its binary16 rounding, as the step
    forms it: partial l (a lane's row slot) holds rows l, l + 16, ..., l + 112 in that order, and
    the column thread adds the partials in index order."""
    parts = []
    for lane in range(LANES):
        acc = np.float32(0.0)
        for t in range(ROWS_PER_LANE):
            i = t * LANES + lane
            y = _round32(Fraction(float(w[i])) * Fraction(float(x[i])))
            acc = _fma32(y, y, acc)
        parts.append(float(acc))
    s = 0.0
    for p in parts:
        s += p
    sw = math.fsum(float(v) ** 2 for v in w)
    return math.sqrt(s / sw)


def _exact_scale(w, x):
    num = math.fsum((float(a) * float(b)) ** 2 for a, b in zip(w, x))
    sw = math.fsum(float(v) ** 2 for v in w)
    return math.sqrt(num / sw)


def _columns(rng):
    n = LANES * ROWS_PER_LANE
    yield rng.lognormal(0, 1, n).astype(np.float32), rng.normal(0, 0.1, n).astype(np.float32)
    w = rng.lognormal(0, 2, n).astype(np.float32)
    x = rng.normal(0, 1, n).astype(np.float32)
    x[rng.choice(n, 4, replace=False)] *= 300          # heavy rows
    yield w, x
    x = np.sort(np.abs(rng.normal(0, 1, n))).astype(np.float32)   # ascending, then descending
    yield np.ones(n, np.float32), x
    yield np.ones(n, np.float32), x[::-1].copy()
    x = (2.0 ** rng.uniform(-30, 30, n)).astype(np.float32)        # magnitudes spread wide
    yield rng.lognormal(0, 1, n).astype(np.float32), x
    x = np.full(n, np.float32(1.0) + np.float32(U) * 3, np.float32)   # equal terms, every add rounds
    yield np.ones(n, np.float32), x


def test_stq_binary32_lane_sums_stay_within_five_ulps_of_the_binary64_fit():
    rng = np.random.default_rng(20260)
    worst = 0.0
    for _ in range(40):
        for w, x in _columns(rng):
            exact = _exact_scale(w, x)
            if exact == 0.0:
                continue
            rel = abs(_device_scale(w, x) - exact) / exact
            worst = max(worst, rel)
            assert rel <= 5 * U, f"relative error {rel:.3g} above 5u"
    # the tolerance window of the GPU test holds this bound with room for the X differences
    assert 5 * U < 1e-6 / 2
    assert worst > 0.0


def _fp32_step_emulated(S, alpha, k, v, beta):
    """The fp32-state step in binary32, every operation rounded on its own (no fused
    multiply-add, sums in row order): S' = a S, u = sum_i k_i S'_i, delta = beta (v - u),
    X = S' + k delta^T."""
    n, D, _ = S.shape
    a = alpha.reshape(n, -1, 1) if alpha.ndim == 2 else alpha.reshape(n, 1, 1)
    Sp = (a.astype(np.float32) * S).astype(np.float32)
    u = np.zeros((n, D), np.float32)
    for i in range(D):
        u = (u + (k[:, i:i + 1] * Sp[:, i, :]).astype(np.float32)).astype(np.float32)
    delta = (beta.reshape(n, 1).astype(np.float32) * (v - u).astype(np.float32)).astype(np.float32)
    return (Sp + (k[:, :, None] * delta[:, None, :]).astype(np.float32)).astype(np.float32)


def test_fp32_state_error_bound_covers_binary32_arithmetic():
    """gpu_common.fp32_state_bound, the GPU tests' tolerance for the fp32-state step, holds for
    binary32 arithmetic in a plain order against the oracle's binary64 step, on GDN and KDA
    gates, on random states and on columns where v nearly cancels u."""
    import oracle
    from gpu_common import fp32_state_bound
    rng = np.random.default_rng(31)
    n, D = 6, 128
    for per_key in (False, True):
        for cancel in (False, True):
            S = rng.normal(0, 0.3, (n, D, D)).astype(np.float32)
            k = rng.normal(0, 1, (n, D))
            k = (k / np.linalg.norm(k, axis=1, keepdims=True)).astype(np.float32)
            q = rng.normal(0, 1, (n, D)).astype(np.float32)
            alpha = rng.uniform(0.2, 1.0, (n, D) if per_key else n).astype(np.float32)
            beta = rng.uniform(0.0, 1.0, n).astype(np.float32)
            v = rng.normal(0, 1, (n, D)).astype(np.float32)
            if cancel:   # v = the exact u, rounded: delta is all rounding
                a = alpha.reshape(n, -1, 1) if per_key else alpha.reshape(n, 1, 1)
                v = np.einsum("ni,nij->nj", k.astype(np.float64),
                              a.astype(np.float64) * S.astype(np.float64)).astype(np.float32)
            X_ref = S.copy()
            oracle.step_fp32(X_ref, q, k, v, alpha, beta)
            X = _fp32_step_emulated(S, alpha, k, v, beta)
            bound = fp32_state_bound(S, alpha, k, v, beta, X_ref)
            err = np.abs(X.astype(np.float64) - X_ref.astype(np.float64))
            assert (err <= bound).all(), f"per_key={per_key} cancel={cancel}: {(err > bound).sum()} above"
            assert err.max() > 0


# ---- the codes-held step's column sums: int8 pieces of the row weights on the matrix cores ----
def _pieces_sum(z, c):
    """u_j = sum_i z_i c_ij as the step forms it: z (binary32, one wave's rows) scaled by 2^S so
    that max |z| 2^S lies in [32, 64), split into four pieces P_k = rint of the remainder times
    128^k (each in [-64, 64]), exact integer sums A_k = sum_i P_k,i c_ij, then
    ((A_3 2^-7 + A_2) 2^-7 + A_1) 2^-7 + A_0 in binary32 (each step one rounding, the 2^-7
    products exact) and the result times 2^-S (exact)."""
    zm = max(abs(float(x)) for x in z)
    if zm == 0:
        return [0.0] * len(c[0])
    S = 6 - math.frexp(zm)[1]
    r = [Fraction(float(x)) * Fraction(2) ** S for x in z]
    P = []
    for _ in range(4):
        p = [round(x) for x in r]     # Python rounds halves to even, as v_rndne_f32 does
        assert all(abs(q) <= 64 for q in p)
        P.append(p)
        r = [(x - q) * 128 for x, q in zip(r, p)]
    out = []
    for j in range(len(c[0])):
        A = [sum(P[k][i] * int(c[i][j]) for i in range(len(z))) for k in range(4)]
        v = _round32(Fraction(A[3]) / 128 + A[2])
        v = _round32(Fraction(float(v)) / 128 + A[1])
        v = _round32(Fraction(float(v)) / 128 + A[0])
        out.append(Fraction(float(v)) / Fraction(2) ** S)
    return out


def test_piece_split_column_sums_stay_within_their_bound():
    """|u_j - exact| <= 3u sum_i |z_i c_ij| + 2^-27 max|z| sum_i |c_ij| (+ margin for the second
    order): the pieces keep each z_i to 2^-22 of the scaled unit (2^-27 of max|z|), the integer
    sums are exact and the recombination rounds three times. On these draws (GDN and KDA row
    weights, a row-factor outlier, a row of small codes) the error stays near the binary32
    summation error of the same sums."""
    rng = np.random.default_rng(11)
    worst = 0.0
    for trial in range(24):
        n = 32
        k = rng.standard_normal(n) / math.sqrt(128)
        gate = 1 / (1 + np.exp(-(rng.standard_normal(n) * (0 if trial % 2 else 3) + 2)))
        rf = np.abs(rng.standard_normal(n)) * 0.01 + 0.001
        rf[rng.integers(0, n)] *= (100 if trial % 3 == 0 else 8)
        z = (gate * rf * k).astype(np.float32)
        c = rng.integers(-127, 128, size=(n, 16))
        c[rng.integers(0, n)] = rng.integers(-2, 3, size=16)
        got = _pieces_sum(z, c)
        zmax = Fraction(float(np.abs(z).max()))
        for j in range(c.shape[1]):
            exact = sum(Fraction(float(z[i])) * int(c[i][j]) for i in range(n))
            sabs = sum(abs(Fraction(float(z[i])) * int(c[i][j])) for i in range(n))
            bound = 3 * Fraction(U) * sabs * (1 + 4 * Fraction(U)) + Fraction(2) ** -27 * zmax * sum(abs(int(x)) for x in c[:, j])
            err = abs(got[j] - exact)
            assert err <= bound, (trial, j, float(err), float(bound))
            if sabs:
                worst = max(worst, float(err / sabs))
    assert worst < 2e-6, worst   # the binary32 summation bound of 32 terms is ~34u = 2e-6
