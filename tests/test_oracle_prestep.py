"""Pins for the oracle's pre-step (CPU only): unit q and k, alpha = exp(-softplus(g)) and
beta = sigmoid(b), the inputs the decode step expects as a GDN / KDA layer makes them.
Pinned by closed forms (a 3-4-5 vector, logits of 0 and +-ln 3), invariants (unit norm,
direction, scale invariance), the zero vector, and numpy's log-add-exp / exp routines.
"""
import numpy as np

import oracle


def test_closed_forms():
    q = np.array([[3.0, 4.0], [0.0, 0.0]], np.float32)
    k = np.array([[0.0, -2.0], [5.0, 12.0]], np.float32)
    g = np.array([0.0, np.log(3.0)], np.float32)
    b = np.array([0.0, -np.log(3.0)], np.float32)
    qh, kh, a, bt = oracle.prestep(q, k, g, b)
    assert qh.tolist() == [[np.float32(0.6), np.float32(0.8)], [0.0, 0.0]]   # zero stays zero
    assert kh.tolist() == [[0.0, -1.0], [np.float32(5 / 13), np.float32(12 / 13)]]
    assert a[0] == 0.5 and bt[0] == 0.5
    # g = ln 3: alpha = 1/(1+3) = 1/4; b = -ln 3: beta = 1/(1+3)
    assert abs(a[1] - 0.25) <= 2 ** -24 and abs(bt[1] - 0.25) <= 2 ** -24


def test_unit_norm_direction_and_scale_invariance():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((50, 128)).astype(np.float32) * 10.0 ** rng.uniform(-3, 3, (50, 1)).astype(np.float32)
    k = rng.standard_normal((50, 128)).astype(np.float32)
    g = rng.standard_normal(50).astype(np.float32)
    b = rng.standard_normal(50).astype(np.float32)
    qh, kh, _, _ = oracle.prestep(q, k, g, b)
    for x, xh in ((q, qh), (k, kh)):
        nrm = np.linalg.norm(xh.astype(np.float64), axis=1)
        assert np.all(np.abs(nrm - 1) < 1e-6)
        cos = np.sum(x.astype(np.float64) * xh, axis=1) / np.linalg.norm(x.astype(np.float64), axis=1)
        assert np.all(np.abs(cos - 1) < 1e-6)
    q2, k2, _, _ = oracle.prestep(q * np.float32(2.0 ** 7), k * np.float32(2.0 ** -5), g, b)
    assert np.array_equal(q2, qh) and np.array_equal(k2, kh)


def test_gates_against_library_routines():
    g = np.concatenate([np.linspace(-60, 60, 241), [-1e-3, 1e-3]]).astype(np.float32)
    n = g.size
    z = np.zeros((n, 4), np.float32)
    _, _, a, bt = oracle.prestep(z, z, g, g)
    gd = g.astype(np.float64)
    want_a = np.exp(-np.logaddexp(0.0, gd))          # exp(-softplus(g))
    want_b = 1.0 / (1.0 + np.exp(-gd))               # sigmoid(b)
    np.testing.assert_allclose(a, want_a.astype(np.float32), rtol=2 ** -23, atol=0)
    np.testing.assert_allclose(bt, want_b.astype(np.float32), rtol=2 ** -23, atol=0)
    # alpha(g) + alpha(-g) = 1 and alpha(g) = beta(-g)
    _, _, a2, b2 = oracle.prestep(z, z, -g, -g)
    assert np.all(np.abs(a.astype(np.float64) + a2 - 1) <= 2 ** -23)
    assert np.array_equal(a, b2)


def test_per_key_gates():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 8)).astype(np.float32)
    g = rng.standard_normal((3, 8)).astype(np.float32)
    _, _, a, _ = oracle.prestep(q, q, g, np.zeros(3, np.float32))
    assert a.shape == (3, 8)
    _, _, a0, _ = oracle.prestep(q[:, :1].copy(), q[:, :1].copy(), g[:, 0].copy(), np.zeros(3, np.float32))
    # the per-key gate of channel 0 equals the scalar gate of the same logit
    assert np.array_equal(a[:, 0], a0)
