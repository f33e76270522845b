"""Pins for the oracle's binary16 conversion and INT8 row rule (CPU only).

FP16: the oracle's conversion is written from the IEEE 754 definition in C; here it must agree
with numpy's float16 cast (an IEEE round-to-nearest-even library routine) on random, tie,
subnormal and overflow inputs, and on every one of the 65,536 binary16 patterns when widening.
INT8: closed-form rows (absmax 127 gives scale 1 and the codes are plain half-to-even
roundings), invariants that any correct symmetric absmax quantizer satisfies, and the exact
rational model in ``exact_ref``.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import exact_ref


def _np_f16_bits(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def test_f16_random_scales_match_ieee_library():
    rng = np.random.default_rng(7)
    parts = [rng.standard_normal(20000).astype(np.float32) * np.float32(10.0 ** e)
             for e in range(-9, 6)]
    x = np.concatenate(parts)
    assert np.array_equal(oracle.f16_from_f32(x), _np_f16_bits(x))


def test_f16_ties_subnormals_overflow():
    # midpoints between consecutive finite binary16 values are exact in binary32
    allh = np.arange(0, 0x7c00, dtype=np.uint16)
    vals = allh.view(np.float16).astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:].astype(np.float64)) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64),
                          (vals[:-1].astype(np.float64) + vals[1:]) / 2)
    special = np.array([0.0, -0.0, 65504.0, 65519.996, 65520.0, 1e6, -1e6, np.inf, -np.inf,
                        2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 1e-30, -1e-30],
                       np.float32)
    x = np.concatenate([mids, -mids, special])
    assert np.array_equal(oracle.f16_from_f32(x), _np_f16_bits(x))


def test_f16_ties_to_even_closed_form():
    x = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2049.0, 2051.0, 65520.0, 2.0 ** -25],
                 np.float32)
    want = np.array([0x3C00, 0x3C02, 0x6800, 0x6802, 0x7C00, 0x0000], np.uint16)
    assert np.array_equal(oracle.f16_from_f32(x), want)


def test_f16_widen_every_pattern():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f32_from_f16(h)
    want = h.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_int8_closed_form_row():
    x = np.array([127, 0.5, 1.5, 2.5, -1.5, -2.5, 3.5, -0.5, 126.5, -126.5, -127], np.float32)
    c, s = oracle.quant_row(x)
    assert s == np.float32(1.0)
    assert c.tolist() == [127, 0, 2, 2, -2, -2, 4, 0, 126, -126, -127]


def test_int8_zero_row():
    c, s = oracle.quant_row(np.zeros(16, np.float32))
    assert s == 0.0 and not c.any()


def test_int8_invariants_random_rows():
    rng = np.random.default_rng(11)
    for t in range(2000):
        D = 128
        x = (rng.standard_normal(D) * rng.lognormal(0, 2)).astype(np.float32)
        if t % 7 == 0:
            x[rng.integers(D)] *= np.float32(50)          # an outlier column
        c, s = oracle.quant_row(x)
        m = np.abs(x).max()
        assert int(np.abs(c).max()) == 127                # the absmax entry maps to +-127
        assert np.all(np.sign(c) * np.sign(x) >= 0)        # signs preserved (or zero)
        err = np.abs(x.astype(np.float64) - c.astype(np.float64) * np.float64(s))
        assert np.all(err <= 0.5 * np.float64(s) * (1 + 1e-5))
        assert abs(np.float64(s) * 127 - m) <= 1e-6 * m
        order = np.argsort(x, kind="stable")
        assert np.all(np.diff(c[order].astype(int)) >= 0)  # monotone


def test_int8_matches_exact_rational_rule():
    rng = np.random.default_rng(12)
    for _ in range(300):
        D = 16
        x = (rng.standard_normal(D) * rng.lognormal(0, 1)).astype(np.float32)
        if rng.random() < 0.3:   # plant exact .5 ties of x/s: s = 1 rows
            x = (rng.integers(-254, 255, D) / 2).astype(np.float32)
            x[0] = 127.0
        c, s = oracle.quant_row(x)
        ce, se = exact_ref.quant_row_exact([Fraction(float(v)) for v in x])
        assert float(s) == float(se)
        assert c.tolist() == ce


def test_int8_rule_with_subnormal_scales_matches_exact_rationals():
    """Rows whose absmax is below 127 * 2^-126, so that the scale is a binary32 subnormal (down
    to rows of subnormal values themselves): the rule is the same, decided on the subnormal
    scale, and the largest entry still codes at +-127."""
    rng = np.random.default_rng(13)
    for amax in (127 * 2.0 ** -126, 1e-36, 1e-37, 2e-39, 3e-41, 2.0 ** -140, 2.0 ** -142):
        for _ in range(20):
            x = rng.standard_normal(16)
            x = (x / np.abs(x).max() * amax).astype(np.float32)
            c, s = oracle.quant_row(x)
            ce, se = exact_ref.quant_row_exact([Fraction(float(v)) for v in x])
            assert float(s) == float(se) and c.tolist() == ce
            assert 0 < s < 2.0 ** -126 or amax == 127 * 2.0 ** -126
            assert np.abs(c).max() == 127
    # absmax below 127 * 2^-150: m / 127 rounds to zero, so scale 0 and codes 0
    x = np.zeros(16, np.float32)
    x[[2, 5]] = np.float32(2.0 ** -149) * np.array([3, -60], np.float32)
    c, s = oracle.quant_row(x)
    assert s == 0 and not c.any()
    assert exact_ref.quant_row_exact([Fraction(float(v)) for v in x]) == ([0] * 16, 0)


def test_requantize_is_idempotent():
    rng = np.random.default_rng(13)
    X = (rng.standard_normal((20000, 128)) * rng.lognormal(0, 1, (20000, 1))).astype(np.float32)
    mask = np.zeros((20000 // 128 + 1, 128), np.uint8)
    n = 20000 // 128
    S = X[: n * 128].reshape(n, 128, 128)
    h, c, s = oracle.quantize(mask[:n], S)
    R = oracle.dequantize(mask[:n], h, c, s)
    h2, c2, s2 = oracle.quantize(mask[:n], R)
    assert np.array_equal(c, c2)
    ulp = np.spacing(s)
    assert np.all(np.abs(s2.astype(np.float64) - s) <= ulp)


@pytest.mark.parametrize("D", [4, 16])
def test_quantize_dequantize_fp16_rows(D):
    rng = np.random.default_rng(14)
    S = rng.standard_normal((3, D, D)).astype(np.float32)
    mask = (rng.random((3, D)) < 0.3).astype(np.uint8)
    h, c, s = oracle.quantize(mask, S)
    R = oracle.dequantize(mask, h, c, s)
    fp16 = mask.astype(bool)
    assert np.array_equal(R[fp16], S[fp16].astype(np.float16).astype(np.float32))
    assert np.array_equal(h[fp16], S[fp16].astype(np.float16).view(np.uint16))
    # INT8 rows reconstruct as code * scale rounded once to binary32
    for u in range(3):
        for i in range(D):
            if not mask[u, i]:
                want = (c[u, i].astype(np.float64) * np.float64(s[u, i])).astype(np.float32)
                assert np.array_equal(R[u, i], want)
