"""Pins for the oracle's budgeted row selection with a per-head FP16 row count (CPU only).

The DAMP abstracts choose high-risk key channels offline from quantization-error energy and
decay-based error retention, and keep them in FP16 under a fixed storage budget (9.9 bits per
state value). The oracle reads the error energy as the squared INT8 error of the row, the
retention as 1/(1 - abar), and hands the budget's FP16 rows to the best groups of g rows over
all heads. Pinned here by closed forms of the error (exact rationals), the budget's byte
identities (the r = 24 layout, uniform INT8, all-FP16 and the pages' 9.9 bits), a brute-force
search over every allocation on small problems, tie rules and output invariants.
"""
from fractions import Fraction
from itertools import product

import numpy as np
import pytest

import oracle


# ---- quantization-error energy of one row --------------------------------------------------
def test_error_is_zero_on_the_code_grid():
    # absmax 127 gives scale exactly 1, so integer rows are stored without error
    x = np.array([127, -3, 0, 42, -127, 1], np.float32)
    assert oracle.int8_row_error(x) == 0.0
    # and so is any row whose entries are code multiples of a power-of-two scale
    assert oracle.int8_row_error(x * np.float32(2.0 ** -9)) == 0.0


def test_error_closed_forms():
    # scale 1: 0.5 -> 0 and 2.5 -> 2 (ties to even), 1.5 -> 2, -0.25 -> 0
    assert oracle.int8_row_error(np.array([127, 0.5], np.float32)) == 0.25
    assert oracle.int8_row_error(np.array([127, 1.5, 2.5, -0.25], np.float32)) == 0.5625
    # zero row: scale 0, codes 0, no error
    assert oracle.int8_row_error(np.zeros(8, np.float32)) == 0.0


def test_error_matches_exact_rationals():
    rng = np.random.default_rng(5)
    for _ in range(50):
        x = (rng.standard_normal(16) * 10.0 ** rng.uniform(-6, 3)).astype(np.float32)
        c, s = oracle.quant_row(x)
        exact = sum((Fraction(float(a)) - Fraction(float(s)) * int(b)) ** 2 for a, b in zip(x, c))
        got = oracle.int8_row_error(x)
        assert abs(Fraction(got) - exact) <= exact * Fraction(1, 10 ** 14)
        # the error of a rounded code is at most half a scale step per entry
        assert got <= 16 * (float(s) / 2) ** 2 * (1 + 1e-12)


# ---- risk scores ---------------------------------------------------------------------------
def test_scores_average_slots_and_apply_retention():
    D, H = 8, 2
    rng = np.random.default_rng(6)
    S = rng.standard_normal((2, H, D, D)).astype(np.float32)
    abar = np.zeros((H, D), np.float32)
    abar[1] = 0.5
    score = oracle.risk_scores(S, abar)
    for h in range(H):
        for i in range(D):
            e = (oracle.int8_row_error(S[0, h, i]) + oracle.int8_row_error(S[1, h, i])) / 2
            assert score[h, i] == e / (1.0 - float(abar[h, i]))
    # gate 1/2: retention exactly 2
    assert np.array_equal(score[1], 2 * np.array([(oracle.int8_row_error(S[0, 1, i]) +
                                                  oracle.int8_row_error(S[1, 1, i])) / 2
                                                 for i in range(D)]))


def test_scores_scale_with_the_square_of_the_state():
    rng = np.random.default_rng(7)
    S = rng.standard_normal((3, 2, 16, 16)).astype(np.float32)
    abar = rng.uniform(0, 0.9, (2, 16)).astype(np.float32)
    assert np.array_equal(oracle.risk_scores(4 * S, abar), 16 * oracle.risk_scores(S, abar))


def test_scores_index_heads_and_rows():
    # one noisy row at (slot 1, head 2, row 5) in otherwise error-free states: only (2, 5) scores
    D, H = 8, 3
    S = np.zeros((2, H, D, D), np.float32)
    S[:, :, :, 0] = 127.0
    S[1, 2, 5, 1] = 0.5
    score = oracle.risk_scores(S, np.zeros((H, D), np.float32))
    nz = np.argwhere(score != 0)
    assert nz.tolist() == [[2, 5]] and score[2, 5] == 0.25 / 2


# ---- budget --------------------------------------------------------------------------------
def test_budget_byte_identities():
    D, H = 128, 32
    # r = 24 per head is 19,872 data bytes = 9.703125 bits per value
    assert oracle.budget_rows(D, H, 9.703125) == 24 * H
    # uniform INT8 with fp32 scales is 8.25 bits; all-FP16 is 16 bits
    assert oracle.budget_rows(D, H, 8.25) == 0
    assert oracle.budget_rows(D, H, 16.0) == D * H
    # the pages' 9.9 bits per value: 27.25 FP16 rows per head on average at D = 128
    assert oracle.budget_rows(D, H, 9.9) == 872
    # groups of g rows, a per-head cap, and a budget below uniform INT8
    assert oracle.budget_rows(D, H, 9.9, g=16) == 864
    assert oracle.budget_rows(D, H, 9.9, r_max=16) == 16 * H
    assert oracle.budget_rows(D, H, 8.0) == -1


# ---- allocation ----------------------------------------------------------------------------
def _ranking(sc):
    return sorted(range(len(sc)), key=lambda i: (-sc[i], i))


def _check_output(score, R, g, r_max, r, m):
    H, D = score.shape
    assert all(x % g == 0 and 0 <= x <= r_max for x in r)
    assert int(r.sum()) == min(R, H * (r_max // g) * g)
    for h in range(H):
        assert sorted(m[h].tolist()) == list(range(D))
        f16, i8 = m[h, :r[h]].tolist(), m[h, r[h]:].tolist()
        assert f16 == sorted(f16) and i8 == sorted(i8)
        assert sorted(f16) == sorted(_ranking(score[h].tolist())[:r[h]])


@pytest.mark.parametrize("g,r_max", [(1, 6), (2, 6), (2, 4), (3, 6)])
def test_allocation_against_exhaustive_search(g, r_max):
    rng = np.random.default_rng(100 + g * 10 + r_max)
    H, D = 3, 6
    for trial in range(20):
        score = rng.exponential(1.0, (H, D)) * rng.uniform(0.2, 5.0, (H, 1))
        if trial % 4 == 0:
            score = np.round(score, 1)          # planted ties
        prefix = [np.concatenate([[0.0], np.cumsum(sorted(score[h], reverse=True))]) for h in range(H)]
        for R in range(0, H * r_max + 1, g):
            best = max(sum(prefix[h][c[h]] for h in range(H))
                       for c in product(range(0, r_max + 1, g), repeat=H) if sum(c) <= R)
            r, m = oracle.allocate_rows(score, R, g, r_max)
            _check_output(score, R, g, r_max, r, m)
            kept = sum(score[h, m[h, :r[h]]].sum() for h in range(H))
            assert kept == pytest.approx(best, rel=1e-12)


def test_allocation_ties():
    H, D = 3, 8
    score = np.ones((H, D))
    r, m = oracle.allocate_rows(score, 8, g=2)
    # equal gains: groups go to the lower head first, rows to the lower index
    assert r.tolist() == [8, 0, 0]
    assert m[0, :8].tolist() == list(range(8))
    r, m = oracle.allocate_rows(score, 8, g=2, r_max=4)
    assert r.tolist() == [4, 4, 0]
    assert m[1, :4].tolist() == [0, 1, 2, 3]


def test_allocation_follows_the_retention_factor():
    # equal errors everywhere; slower gates (larger abar) on head 1 draw the FP16 rows there
    H, D = 2, 16
    S = np.random.default_rng(8).standard_normal((1, 1, D, D)).astype(np.float32)
    S = np.repeat(S, H, axis=1)
    abar = np.full((H, D), 0.2, np.float32)
    abar[1, 3:7] = 0.9
    r, m = oracle.allocate_rows(oracle.risk_scores(S, abar), 4)
    assert r.tolist() == [0, 4] and m[1, :4].tolist() == [3, 4, 5, 6]
