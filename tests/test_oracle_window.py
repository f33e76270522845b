"""Pins for the oracle's per-window requantization (CPU only).

The LeapQuant abstract: the low-bit state stays fixed for a window of tokens, the window's
updates are held in high precision, outputs come from both, and the state is quantized once at
the window's end. Pinned here by special cases that reduce to separately pinned paths: a window
of one token is the per-token step bit for bit; inside a window the readouts follow the fp32
recurrence from the reconstructed state up to fp32 rounding; an identity window returns the
stored codes unchanged; a flush after t tokens equals a window of t tokens; units in different
window phases do not interact. And by the property the page claims: fewer requantizations
accumulate less error against the exact recurrence.
"""
import numpy as np

import oracle
from quantized_delta_rule_gdn_amd import synth


def _state(seed, n, D, r, decay=synth.GDN):
    rng = np.random.default_rng(seed)
    S = synth.normal_states(rng, (n, D, D), 0.1)
    S[:, rng.choice(D, 2, replace=False), :] *= 6
    mask = np.zeros((n, D), np.uint8)
    for u in range(n):
        mask[u, rng.choice(D, r, replace=False)] = 1
    h, c, s = oracle.quantize(mask, S)
    return rng, mask, h, c, s


def _inputs(rng, n, D, decay, dtype="fp32"):
    inp = synth.step_inputs(rng, 1, n, D, decay, dtype)
    al = inp.alpha.reshape(n, D) if decay == synth.KDA else inp.alpha.reshape(n)
    return inp.q.reshape(n, D), inp.k.reshape(n, D), inp.v.reshape(n, D), al, inp.beta.reshape(n)


def test_window_of_one_is_the_per_token_step():
    for decay in (synth.GDN, synth.KDA):
        rng, mask, h, c, s = _state(1 + decay, 5, 16, 3, decay)
        win = oracle.Window(mask, h.copy(), c.copy(), s.copy(), 1)
        for _ in range(4):
            x = _inputs(rng, 5, 16, decay)
            o1 = win.step(*x)
            o2 = oracle.step_quant(mask, h, c, s, *x)
            assert np.array_equal(o1, o2)
            assert np.array_equal(win.h, h) and np.array_equal(win.c, c) and np.array_equal(win.s, s)
            assert not win.t.any()


def test_readouts_follow_the_fp32_recurrence_inside_a_window():
    D, n, W = 32, 4, 8
    rng, mask, h, c, s = _state(7, n, D, 4, synth.KDA)
    S32 = oracle.dequantize(mask, h, c, s)
    win = oracle.Window(mask, h.copy(), c.copy(), s.copy(), W)
    for t in range(W):
        x = _inputs(rng, n, D, synth.KDA)
        ow = win.step(*x)
        of = oracle.step_fp32(S32, *x)
        np.testing.assert_allclose(ow, of, rtol=1e-5, atol=1e-7)
        assert win.t.tolist() == [(t + 1) % W] * n
    # at the window's end the stored state is the fp32 state requantized (up to the codes that
    # its fp32 rounding moves)
    h2, c2, s2 = oracle.quantize(mask, S32)
    assert np.abs(win.c.astype(int) - c2.astype(int)).max() <= 1
    assert (win.c == c2).mean() > 0.999


def test_identity_window_keeps_the_stored_state():
    D, n, W = 16, 3, 5
    rng, mask, h, c, s = _state(9, n, D, 2)
    win = oracle.Window(mask, h.copy(), c.copy(), s.copy(), W)
    S0 = oracle.dequantize(mask, h, c, s).astype(np.float64)
    for _ in range(W):
        q, k, v, _, _ = _inputs(rng, n, D, synth.GDN)
        out = win.step(q, k, v, np.ones(n, np.float32), np.zeros(n, np.float32))
        np.testing.assert_allclose(out, np.einsum("nij,ni->nj", S0, q.astype(np.float64)), rtol=1e-6, atol=1e-9)
    assert np.array_equal(win.c, c) and np.array_equal(win.h, h) and np.array_equal(win.s, s)


def test_flush_after_t_tokens_is_a_window_of_t():
    D, n = 16, 4
    for t in (1, 3):
        rng, mask, h, c, s = _state(11 + t, n, D, 2, synth.KDA)
        xs = [_inputs(rng, n, D, synth.KDA) for _ in range(t)]
        a = oracle.Window(mask, h.copy(), c.copy(), s.copy(), 8)
        b = oracle.Window(mask, h.copy(), c.copy(), s.copy(), t)
        for x in xs:
            assert np.array_equal(a.step(*x), b.step(*x))
        assert not np.array_equal(a.c, b.c)     # b has stored its window, a not yet
        a.flush()
        assert np.array_equal(a.c, b.c) and np.array_equal(a.h, b.h) and np.array_equal(a.s, b.s)
        assert not a.t.any() and not b.t.any()


def test_units_in_different_phases_are_independent():
    D, n, W = 16, 2, 4
    rng, mask, h, c, s = _state(13, n, D, 2)
    xs = [_inputs(rng, n, D, synth.GDN) for _ in range(6)]
    both = oracle.Window(mask, h.copy(), c.copy(), s.copy(), W)
    both.step(*xs[0])
    both.t[1] = 0     # unit 1 drops its pending token: its window restarts one token later
    # unit 1 alone, with its own window object, from the same stored state
    one = oracle.Window(mask[1:], h[1:].copy(), c[1:].copy(), s[1:].copy(), W)
    for x in xs[1:]:
        ob = both.step(*x)
        oo = one.step(*(a[1:] for a in x))
        assert np.array_equal(ob[1:], oo)
    assert both.t.tolist() == [(1 + 5) % W, 5 % W]
    assert np.array_equal(both.c[1:], one.c)


def test_fewer_requantizations_accumulate_less_error():
    # slow decay (alpha = 0.98): requantization errors persist across many steps, the regime
    # where the page says per-token requantization accumulates error
    D, n, T = 32, 16, 64
    rng, mask, h, c, s = _state(17, n, D, 4)
    S_exact = oracle.dequantize(mask, h, c, s)
    wins = {W: oracle.Window(mask, h.copy(), c.copy(), s.copy(), W) for W in (1, 16)}
    for _ in range(T):
        q, k, v, _, b = _inputs(rng, n, D, synth.GDN)
        x = (q, k, v, np.full(n, 0.98, np.float32), b)
        oracle.step_fp32(S_exact, *x)
        for w in wins.values():
            w.step(*x)
    err = {W: np.linalg.norm(oracle.dequantize(mask, w.h, w.c, w.s) - S_exact) for W, w in wins.items()}
    assert err[16] < 0.5 * err[1], err
