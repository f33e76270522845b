"""Pins for the oracle's decode step (CPU only).

What fixes the expected values, none of it the oracle itself:
  * a hand-worked 4x4 case (tests/golden/hand_4x4.json, all values dyadic and exact);
  * the exact rational model in ``exact_ref`` on random 4x4 / 8x8 / 16x16 units (bit-exact);
  * closed forms: alpha = 1, beta = 0 is the identity; beta = 1 with a unit key writes v into
    the key direction; a query orthogonal to the key reads S'^T q whatever v and beta are;
  * cross-format identities: a per-key gate vector of equal entries equals the scalar gate,
    all rows FP16 agrees with the fp32 state to FP16 precision, units are independent.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import exact_ref
from quantized_delta_rule_gdn_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _unit(rng, D, n=1):
    x = rng.standard_normal((n, D))
    return (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)


def _random_quant_unit(rng, D, n, frac_fp16=0.25):
    S = (rng.standard_normal((n, D, D)) * 0.3).astype(np.float32)
    mask = (rng.random((n, D)) < frac_fp16).astype(np.uint8)
    h, c, s = oracle.quantize(mask, S)
    return mask, h, c, s


def test_hand_worked_4x4():
    g = json.load(open(os.path.join(GOLD, "hand_4x4.json")))
    D = g["D"]
    mask = np.array([g["mask"]], np.uint8)
    c = np.array([g["codes_in"]], np.int8)
    s = np.array([g["scales_in"]], np.float32)
    h = np.zeros((1, D, D), np.uint16)
    h[0, 3] = np.array(g["fp16_row3_in"], np.float16).view(np.uint16)
    # the input reconstructs to S_hat exactly
    assert np.array_equal(oracle.dequantize(mask, h, c, s)[0], np.array(g["S_hat"], np.float32))
    out = oracle.step_quant(mask, h, c, s, g["q"], g["k"], g["v"], [g["alpha"]], [g["beta"]])
    assert out[0].tolist() == g["y"]
    assert c[0, :3].tolist() == g["codes_out_rows012"]
    for i, (num, den) in enumerate(g["scale_out_rationals"]):
        assert Fraction(float(s[0, i])) == exact_ref.f32(Fraction(num, den))
    assert h[0, 3].view(np.float16).astype(float).tolist() == g["fp16_row3_out"]
    # the same step on the fp32 state gives X exactly
    S = np.array([g["S_hat"]], np.float32)
    out32 = oracle.step_fp32(S, g["q"], g["k"], g["v"], [g["alpha"]], [g["beta"]])
    assert out32[0].tolist() == g["y"]
    assert (S[0] * 16).tolist() == g["X_num_over_16"]


@pytest.mark.parametrize("D,fmt,kda,seed", [(4, 1, 0, 1), (4, 0, 1, 2), (8, 1, 1, 3),
                                            (8, 0, 0, 4), (16, 1, 0, 5), (16, 1, 1, 6)])
def test_step_matches_exact_rational_model(D, fmt, kda, seed):
    rng = np.random.default_rng(seed)
    n = 2
    q, k = _unit(rng, D, n), _unit(rng, D, n)
    v = rng.standard_normal((n, D)).astype(np.float32)
    alpha = rng.uniform(0.05, 1, (n, D) if kda else n).astype(np.float32)
    beta = rng.uniform(0, 1, n).astype(np.float32)
    if fmt == 0:
        S = (rng.standard_normal((n, D, D)) * 0.3).astype(np.float32)
        S0 = S.copy()
        out = oracle.step_fp32(S, q, k, v, alpha, beta)
        for u in range(n):
            e = exact_ref.step_exact(D, 0, None, S0[u], None, None, None, q[u], k[u], v[u],
                                     alpha[u], beta[u])
            assert np.array_equal(out[u], e["out"])
            assert np.array_equal(S[u], e["S32"])
    else:
        mask, h, c, s = _random_quant_unit(rng, D, n)
        h0, c0, s0 = h.copy(), c.copy(), s.copy()
        out = oracle.step_quant(mask, h, c, s, q, k, v, alpha, beta)
        for u in range(n):
            e = exact_ref.step_exact(D, 1, mask[u], None, h0[u], c0[u], s0[u], q[u], k[u],
                                     v[u], alpha[u], beta[u])
            assert np.array_equal(out[u], e["out"])
            f = mask[u].astype(bool)
            assert np.array_equal(h[u][f], e["h"][f])
            assert np.array_equal(c[u][~f], e["c"][~f])
            assert np.array_equal(s[u][~f], e["s"][~f])


def test_identity_alpha1_beta0():
    """alpha = 1, beta = 0: X = S_hat, so requantization returns the same codes and FP16
    values, scales move by at most one ulp, and y = S_hat^T q."""
    rng = np.random.default_rng(21)
    D, n = 128, 6
    mask, h, c, s = _random_quant_unit(rng, D, n)
    R = oracle.dequantize(mask, h, c, s).astype(np.float64)
    q, k = _unit(rng, D, n), _unit(rng, D, n)
    v = rng.standard_normal((n, D)).astype(np.float32)
    h0, c0, s0 = h.copy(), c.copy(), s.copy()
    out = oracle.step_quant(mask, h, c, s, q, k, v, np.ones(n, np.float32), np.zeros(n, np.float32))
    f = mask.astype(bool)
    assert np.array_equal(h[f], h0[f])
    assert np.array_equal(c[~f], c0[~f])
    assert np.all(np.abs(s[~f].astype(np.float64) - s0[~f]) <= np.spacing(s0[~f]))
    want = np.einsum("uij,ui->uj", R, q.astype(np.float64))
    np.testing.assert_allclose(out, want, rtol=1e-6, atol=1e-7)


def test_unit_key_writes_value():
    """beta = 1, alpha = 1, k = e_m: row m of X becomes v exactly and every other row is kept.
    For a general unit k, X^T k = v up to the binary32 rounding of X."""
    rng = np.random.default_rng(22)
    D, n = 128, 4
    S = (rng.standard_normal((n, D, D)) * 0.3).astype(np.float32)
    S0 = S.copy()
    m = 37
    k = np.zeros((n, D), np.float32)
    k[:, m] = 1
    q = _unit(rng, D, n)
    v = rng.standard_normal((n, D)).astype(np.float32)
    oracle.step_fp32(S, q, k, v, np.ones(n, np.float32), np.ones(n, np.float32))
    assert np.array_equal(S[:, m], v)
    keep = np.arange(D) != m
    assert np.array_equal(S[:, keep], S0[:, keep])
    k = _unit(rng, D, n)
    S = S0.copy()
    oracle.step_fp32(S, q, k, v, np.ones(n, np.float32), np.ones(n, np.float32))
    got = np.einsum("uij,ui->uj", S.astype(np.float64), k.astype(np.float64))
    np.testing.assert_allclose(got, v, rtol=0, atol=2e-6)


def test_orthogonal_query_ignores_v_and_beta():
    """q orthogonal to k (exact dyadic Hadamard rows): y = S'^T q, independent of v and beta;
    with the key's row of S_hat zero, X = S' + beta k v^T exactly."""
    H2 = np.array([[1, 1], [1, -1]])
    Had = H2
    for _ in range(3):
        Had = np.kron(Had, H2)
    D = 16
    q = (Had[3] / 4.0).astype(np.float32)
    k = (Had[5] / 4.0).astype(np.float32)
    assert float(q.astype(np.float64) @ k) == 0.0
    rng = np.random.default_rng(23)
    S = (rng.standard_normal((1, D, D)) * 0.3).astype(np.float32)
    alpha = np.float32(0.75)
    outs = []
    for vs, b in ((1.0, 0.2), (-3.0, 0.9)):
        St = S.copy()
        v = (rng.standard_normal(D) * vs).astype(np.float32)
        outs.append(oracle.step_fp32(St, q, k, v, [alpha], [b]))
    assert np.array_equal(outs[0], outs[1])
    want = (float(alpha) * S[0].astype(np.float64)).T @ q.astype(np.float64)
    np.testing.assert_allclose(outs[0][0], want, rtol=1e-6, atol=1e-7)
    # S_hat^T k = 0 (k = e_m, row m zero), alpha = 1: X = S + beta k v^T exactly in binary32
    S2 = S.copy()
    S2[0, 9] = 0
    k2 = np.zeros(D, np.float32)
    k2[9] = 1
    v = np.array([0.5 * (j - 8) for j in range(D)], np.float32)
    St = S2.copy()
    oracle.step_fp32(St, q, k2, v, [1.0], [0.25])
    want = S2[0].copy()
    want[9] = 0.25 * v
    assert np.array_equal(St[0], want)


def test_constant_kda_gate_equals_gdn_gate():
    rng = np.random.default_rng(24)
    D, n = 128, 3
    mask, h, c, s = _random_quant_unit(rng, D, n)
    q, k = _unit(rng, D, n), _unit(rng, D, n)
    v = rng.standard_normal((n, D)).astype(np.float32)
    a = rng.uniform(0.1, 1, n).astype(np.float32)
    b = rng.uniform(0, 1, n).astype(np.float32)
    st1 = [x.copy() for x in (h, c, s)]
    st2 = [x.copy() for x in (h, c, s)]
    o1 = oracle.step_quant(mask, *st1, q, k, v, a, b)
    o2 = oracle.step_quant(mask, *st2, q, k, v, np.repeat(a[:, None], D, 1), b)
    assert np.array_equal(o1, o2)
    for x1, x2 in zip(st1, st2):
        assert np.array_equal(x1, x2)


def test_all_fp16_rows_track_fp32_state():
    rng = np.random.default_rng(25)
    D, n = 128, 3
    S = (rng.standard_normal((n, D, D)) * 0.3).astype(np.float32)
    mask = np.ones((n, D), np.uint8)
    h, c, s = oracle.quantize(mask, S)
    S16 = oracle.dequantize(mask, h, c, s)
    q, k = _unit(rng, D, n), _unit(rng, D, n)
    v = rng.standard_normal((n, D)).astype(np.float32)
    a = rng.uniform(0.1, 1, n).astype(np.float32)
    b = rng.uniform(0, 1, n).astype(np.float32)
    o16 = oracle.step_quant(mask, h, c, s, q, k, v, a, b)
    o32 = oracle.step_fp32(S16, q, k, v, a, b)
    assert np.array_equal(o16, o32)    # same S_hat, same X, readout before requantization
    assert np.array_equal(h, S16.astype(np.float16).view(np.uint16))


def test_units_independent_and_thread_count_invariant():
    rng = np.random.default_rng(26)
    D, n = 128, 9
    mask, h, c, s = _random_quant_unit(rng, D, n)
    q, k = _unit(rng, D, n), _unit(rng, D, n)
    v = rng.standard_normal((n, D)).astype(np.float32)
    a = rng.uniform(0.1, 1, (n, D)).astype(np.float32)
    b = rng.uniform(0, 1, n).astype(np.float32)
    A = [x.copy() for x in (h, c, s)]
    oa = oracle.step_quant(mask, *A, q, k, v, a, b, nthreads=1)
    B = [x.copy() for x in (h, c, s)]
    ob = oracle.step_quant(mask, *B, q, k, v, a, b, nthreads=4)
    assert np.array_equal(oa, ob)
    for x, y in zip(A, B):
        assert np.array_equal(x, y)
    u = 5
    C = [x[u:u + 1].copy() for x in (h, c, s)]
    oc = oracle.step_quant(mask[u:u + 1], *C, q[u:u + 1], k[u:u + 1], v[u:u + 1], a[u:u + 1],
                           b[u:u + 1])
    assert np.array_equal(oc[0], oa[u])
    for x, y in zip(C, A):
        assert np.array_equal(x[0], y[u])


def test_tiny_workload_free_run_is_finite_and_close_to_fp32():
    rows, S0, steps = synth.tiny()
    D, H = 16, 2
    mask = synth.rows_to_mask(rows, D)
    n = H
    S32 = S0.reshape(n, D, D).copy()
    h, c, s = oracle.quantize(mask, S32)
    for st in steps:
        o32 = oracle.step_fp32(S32, st.q, st.k, st.v, st.alpha, st.beta)
        oq = oracle.step_quant(mask, h, c, s, st.q, st.k, st.v, st.alpha, st.beta)
        assert np.all(np.isfinite(oq))
        rel = np.linalg.norm(oq - o32) / np.linalg.norm(o32)
        assert rel < 0.05
