"""Pins for the oracle's STEPQuant-style state (CPU only): pivot rows in FP16, integer rows of
4, 6 or 8 bits with FP16 row factors and one FP16 column-scale vector per unit fitted with
squared row-impact weights (the STEPQuant page, Table C2 steps 1-6; the fit's formulas are this
repository's reading, written out in oracle.c).

Pinned by a hand-derived 2x3 fixture (tests/golden/stq_3x3.json), exact rational
reconstruction, numpy's IEEE float16 on pivot rows, closed forms (a lone integer row codes every
entry at +-qmax, weight scaling changes nothing, zero weights mean equal weights), invariants of
the codes (range, half-step error where not clamped), the step's reduction to the
all-FP16 DAMP step when every row is a pivot, and the step over several units with integer rows
against an exact rational model of the fit (tests/exact_ref.py).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def test_hand_derived_fixture():
    g = json.load(open(os.path.join(HERE, "golden", "stq_3x3.json")))
    X = np.array(g["X"], np.float32)
    # the oracle's unit is D x D: embed the 2 x 3 block in a 3 x 3 unit whose last row is a pivot
    S = np.zeros((1, 3, 3), np.float32)
    S[0, :2, :] = X
    bits = np.array([[g["bits"][0], g["bits"][1], 16]], np.uint8)
    w = np.array([[1.0, 1.0, 0.0]], np.float32)
    h, c, rf, cs = oracle.stq_quantize(bits, w, S)
    assert _f16(cs[0]).tolist() == g["cs"]
    assert _f16(rf[0, :2]).tolist() == [m * 2.0 ** e for m, e in g["rf_units"]]
    assert c[0, :2].tolist() == g["codes"]
    assert rf[0, 2] == 0 and not c[0, 2].any()


def test_reconstruction_is_exact():
    rng = np.random.default_rng(3)
    D = 16
    S = (rng.standard_normal((2, D, D)) * 0.1).astype(np.float32)
    bits = rng.choice(np.array([16, 8, 6, 4], np.uint8), (2, D))
    w = rng.uniform(0, 2, (2, D)).astype(np.float32)
    h, c, rf, cs = oracle.stq_quantize(bits, w, S)
    R = oracle.stq_dequantize(bits, h, c, rf, cs)
    for u in range(2):
        for i in range(D):
            for j in range(0, D, 5):
                if bits[u, i] == 16:
                    want = Fraction(float(np.float16(S[u, i, j])))
                else:
                    want = int(c[u, i, j]) * Fraction(float(_f16(rf[u, i]))) * Fraction(float(_f16(cs[u, j])))
                assert Fraction(float(R[u, i, j])) == Fraction(float(np.float32(float(want))))


def test_pivot_rows_are_ieee_binary16():
    rng = np.random.default_rng(4)
    D = 16
    S = (rng.standard_normal((1, D, D)) * 10.0 ** rng.uniform(-6, 4, (1, D, 1))).astype(np.float32)
    bits = np.full((1, D), 16, np.uint8)
    bits[0, ::3] = 6
    h, c, rf, cs = oracle.stq_quantize(bits, np.ones((1, D), np.float32), S)
    piv = bits[0] == 16
    assert np.array_equal(h[0, piv], S[0, piv].astype(np.float16).view(np.uint16))
    assert not h[0, ~piv].any() and not c[0, piv].any() and not rf[0, piv].any()


def test_lone_integer_row_codes_at_qmax():
    # one integer row, every other row a pivot: cs_j = fp16(|x_j|), every |x_j| / cs_j is about 1,
    # so the row factor is about 1 / qmax and every non-zero entry codes at +-qmax
    D = 16
    rng = np.random.default_rng(5)
    for b, qm in ((8, 127), (6, 31), (4, 7)):
        S = (rng.standard_normal((1, D, D))).astype(np.float32)
        S[0, 3, 7] = 0.0
        bits = np.full((1, D), 16, np.uint8)
        bits[0, 3] = b
        h, c, rf, cs = oracle.stq_quantize(bits, np.ones((1, D), np.float32), S)
        want = np.sign(S[0, 3]).astype(int) * qm
        assert c[0, 3].tolist() == want.tolist()


def test_codes_stay_in_range_and_within_half_a_step():
    rng = np.random.default_rng(6)
    D, n = 32, 4
    S = (rng.standard_normal((n, D, D)) * 0.1).astype(np.float32)
    S[:, :, 5] *= 30          # a heavy column
    S[:, 2, :] *= 20          # a heavy row
    bits = rng.choice(np.array([16, 8, 6, 4], np.uint8), (n, D))
    w = rng.uniform(0.1, 3, (n, D)).astype(np.float32)
    h, c, rf, cs = oracle.stq_quantize(bits, w, S)
    for u in range(n):
        for i in range(D):
            if bits[u, i] == 16:
                continue
            qm = 2 ** (int(bits[u, i]) - 1) - 1
            assert np.abs(c[u, i].astype(int)).max() <= qm
            step = _f16(rf[u, i]) * _f16(cs[u])
            err = np.abs(S[u, i].astype(np.float64) - c[u, i] * step)
            unclamped = np.abs(c[u, i]) < qm
            assert np.all(err[unclamped] <= step[unclamped] / 2 * (1 + 1e-6) + 1e-30)


def test_weights_scale_free_and_zero_weights_mean_equal():
    rng = np.random.default_rng(7)
    D = 16
    S = (rng.standard_normal((1, D, D)) * 0.1).astype(np.float32)
    bits = rng.choice(np.array([8, 6, 4], np.uint8), (1, D))
    w = rng.uniform(0.5, 2, (1, D)).astype(np.float32)
    a = oracle.stq_quantize(bits, w, S)
    b = oracle.stq_quantize(bits, 4 * w, S)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    z = oracle.stq_quantize(bits, np.zeros((1, D), np.float32), S)
    o = oracle.stq_quantize(bits, np.ones((1, D), np.float32), S)
    assert all(np.array_equal(x, y) for x, y in zip(z, o))
    # pivot rows, whatever their impact score, do not enter the column scales
    bp = bits.copy()
    bp[0, 1] = 16
    wp = w.copy()
    wp[0, 1] = 50.0
    assert all(np.array_equal(x, y) for x, y in zip(oracle.stq_quantize(bp, wp, S), oracle.stq_quantize(bp, w, S)))
    # a row with zero impact does not enter the column scales
    w2 = w.copy()
    w2[0, 4] = 0.0
    S2 = S.copy()
    S2[0, 4] *= 1000
    assert np.array_equal(oracle.stq_quantize(bits, w2, S2)[3], oracle.stq_quantize(bits, w2, S)[3])


def test_step_with_every_row_a_pivot_is_the_all_fp16_damp_step():
    rng = np.random.default_rng(8)
    D, n = 16, 3
    S = (rng.standard_normal((n, D, D)) * 0.1).astype(np.float32)
    bits = np.full((n, D), 16, np.uint8)
    w = np.ones((n, D), np.float32)
    h, c, rf, cs = oracle.stq_quantize(bits, w, S)
    q = rng.standard_normal((n, D)).astype(np.float32)
    k = rng.standard_normal((n, D)).astype(np.float32)
    v = rng.standard_normal((n, D)).astype(np.float32)
    al = rng.uniform(0.2, 1, (n, D)).astype(np.float32)
    be = rng.uniform(0, 1, n).astype(np.float32)
    out, (h2, c2, rf2, cs2) = oracle.stq_step(bits, w, h, c, rf, cs, q, k, v, al, be)
    mask = np.ones((n, D), np.uint8)
    hd, cd, sd = oracle.quantize(mask, S)
    assert np.array_equal(hd, h)
    outd = oracle.step_quant(mask, hd, cd, sd, q, k, v, al, be)
    assert np.array_equal(out, outd) and np.array_equal(h2, hd)


def _stq_case(seed, n, D, per_key):
    """n units with their own precision maps (each has a pivot and rows of all three integer
    widths), their own row-impact scores (the last unit all zero: equal weights), a heavy row
    and a heavy column, packed by the oracle; plus one step's inputs."""
    rng = np.random.default_rng(seed)
    bits = np.empty((n, D), np.uint8)
    for u in range(n):
        kinds = np.array([16, 8, 6, 4] + list(rng.choice(np.array([16, 8, 6, 4], np.uint8), D - 4)), np.uint8)
        bits[u] = rng.permutation(kinds)
    w = rng.uniform(0.2, 3.0, (n, D)).astype(np.float32)
    w[-1] = 0.0
    S = (rng.standard_normal((n, D, D)) * 0.3).astype(np.float32)
    S[:, :, 3] *= 12.0
    S[:, 5, :] *= 7.0
    st = oracle.stq_quantize(bits, w, S)
    q = rng.standard_normal((n, D)).astype(np.float32)
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((n, D)).astype(np.float32)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((n, D)).astype(np.float32)
    al = (rng.uniform(0.3, 1.0, (n, D)) if per_key else rng.uniform(0.3, 1.0, n)).astype(np.float32)
    be = rng.uniform(0.1, 1.0, n).astype(np.float32)
    return bits, w, st, (q, k, v, al, be)


@pytest.mark.parametrize("per_key", [False, True])
def test_step_on_integer_rows_matches_exact_rationals_across_units(per_key):
    """The step over several units with mixed 8/6/4-bit rows, per-unit precision maps and row
    weights, both gate forms, against exact rational arithmetic of the fit's statement: every
    readout, pivot value, code, row factor and column scale bit for bit. A column whose square
    root lies within 1e-9 of a quantum of a binary16 tie (where binary64 evaluation could take
    the other side) takes the oracle's scale and is counted; there is none in these cases."""
    import exact_ref
    n, D = 4, 12
    bits, w, (h, c, rf, cs), (q, k, v, al, be) = _stq_case(11 + per_key, n, D, per_key)
    out, (h2, c2, rf2, cs2) = oracle.stq_step(bits, w, h, c, rf, cs, q, k, v, al, be)
    near = 0
    for u in range(n):
        ref = exact_ref.stq_step_exact(D, bits[u], w[u], h[u], c[u], rf[u], cs[u], q[u], k[u], v[u],
                                       al[u], be[u])
        ties = {j: int(cs2[u, j]) for j in np.nonzero(ref["tie"] < 1e-9)[0]}
        if ties:
            near += len(ties)
            ref = exact_ref.stq_step_exact(D, bits[u], w[u], h[u], c[u], rf[u], cs[u], q[u], k[u],
                                           v[u], al[u], be[u], cs_near_tie=ties)
        assert np.array_equal(cs2[u], ref["cs"]), f"unit {u}: column scales"
        assert np.array_equal(rf2[u], ref["rf"]), f"unit {u}: row factors"
        assert np.array_equal(c2[u], ref["c"]), f"unit {u}: codes"
        assert np.array_equal(h2[u], ref["h"]), f"unit {u}: pivot rows"
        assert np.array_equal(out[u], ref["out"]), f"unit {u}: readout"
        assert (c2[u][bits[u] != 16] != 0).any()
    assert near == 0


def test_fit_rows_for_given_column_scales_matches_exact_rationals():
    """oracle_stq_fit_rows (the fit's second half with the column scales given, which the GPU
    tests use to take the row factors and codes from the device's own column scales) against
    the exact rational rule, on states and column scales drawn at random (some scales 0), and
    against the whole fit when handed the fit's own column scales."""
    import exact_ref
    rng = np.random.default_rng(21)
    n, D = 3, 12
    bits = np.stack([rng.permutation(np.array([16, 8, 6, 4] + list(rng.choice(np.array([16, 8, 6, 4], np.uint8), D - 4)), np.uint8))
                     for _ in range(n)])
    X = (rng.standard_normal((n, D, D)) * 0.5).astype(np.float32)
    cs = np.abs(rng.standard_normal((n, D)) * 0.2).astype(np.float16)
    cs[0, 3] = 0
    csb = cs.view(np.uint16)
    h, c, rf = oracle.stq_fit_rows(bits, X, csb)
    for u in range(n):
        Xf = [[Fraction(float(X[u, i, j])) for j in range(D)] for i in range(D)]
        he, ce, rfe = exact_ref.stq_rows_exact(D, bits[u], Xf, [Fraction(float(x)) for x in cs[u]])
        assert np.array_equal(h[u], he) and np.array_equal(c[u], ce) and np.array_equal(rf[u], rfe)
    w = rng.uniform(0.5, 2, (n, D)).astype(np.float32)
    hq, cq, rfq, csq = oracle.stq_quantize(bits, w, X)
    h2, c2, rf2 = oracle.stq_fit_rows(bits, X, csq)
    assert np.array_equal(hq, h2) and np.array_equal(cq, c2) and np.array_equal(rfq, rf2)
