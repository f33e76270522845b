"""CPU oracle for the GDN / KDA recurrent-state decode step (FP32, uniform INT8, DAMP).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()`` and by the CPU
baseline leg of ``bench.py``. The GPU library and its binding never import it, and it imports
nothing from them. The arithmetic lives in ``oracle.c`` (see its header for the sources and the
precision policy); this module only builds/loads that library and marshals numpy arrays.

Logical state representation of ``n`` units of a ``D x D`` state (rows = key channels):
    fp32:       S  float32 [n, D, D]
    quantized:  mask uint8 [n, D] (1 = FP16 row), h uint16 [n, D, D] (binary16 bits),
                c int8 [n, D, D], s float32 [n, D]
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra"]


def build() -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` next to it (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        Lg = ctypes.c_long
        L.oracle_f16_from_f32_n.argtypes = [P, P, Lg]
        L.oracle_f32_from_f16_n.argtypes = [P, P, Lg]
        L.oracle_quant_row.argtypes = [I, P, P, P]
        L.oracle_quantize.argtypes = [I, Lg, P, P, P, P, P, I]
        L.oracle_quantize.restype = I
        L.oracle_dequantize.argtypes = [I, Lg, P, P, P, P, P, I]
        L.oracle_dequantize.restype = I
        L.oracle_step.argtypes = [I, Lg, I, P, P, P, P, P, P, P, P, P, I, P, P, I]
        L.oracle_step.restype = I
        L.oracle_select_rows.argtypes = [I, I, Lg, P, P, I, P, P]
        L.oracle_select_rows.restype = I
        L.oracle_int8_row_error.argtypes = [I, P]
        L.oracle_int8_row_error.restype = ctypes.c_double
        L.oracle_risk_scores.argtypes = [I, I, Lg, P, P, P]
        L.oracle_risk_scores.restype = I
        L.oracle_budget_rows.argtypes = [I, I, ctypes.c_double, I, I]
        L.oracle_budget_rows.restype = Lg
        L.oracle_allocate_rows.argtypes = [I, I, P, Lg, I, I, P, P]
        L.oracle_allocate_rows.restype = I
        L.oracle_prestep.argtypes = [I, Lg, P, P, P, I, P, P, P, P, P]
        L.oracle_prestep.restype = I
        L.oracle_window_step.argtypes = [I, Lg, P, P, P, P, P, P, I, P, P, P, P, I, P, P, I]
        L.oracle_window_step.restype = I
        L.oracle_window_flush.argtypes = [I, Lg, P, P, P, P, P, P]
        L.oracle_window_flush.restype = I
        L.oracle_stq_quantize.argtypes = [I, Lg, P, P, P, P, P, P, P]
        L.oracle_stq_quantize.restype = I
        L.oracle_stq_dequantize.argtypes = [I, Lg, P, P, P, P, P, P]
        L.oracle_stq_dequantize.restype = I
        L.oracle_stq_step.argtypes = [I, Lg, P, P, P, P, P, P, P, P, P, P, P, P, P, P, I, P, P, P, I]
        L.oracle_stq_step.restype = I
        L.oracle_stq_fit_rows.argtypes = [I, Lg, P, P, P, P, P, P]
        L.oracle_stq_fit_rows.restype = I
        _lib = L
    return _lib


def default_threads() -> int:
    n = os.environ.get("OMP_NUM_THREADS")
    if n and n.isdigit() and int(n) > 0:
        return int(n)
    return max(1, min(16, os.cpu_count() or 1))


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def f16_from_f32(x) -> np.ndarray:
    x = _c(x, np.float32)
    h = np.empty(x.shape, np.uint16)
    lib().oracle_f16_from_f32_n(_p(x), _p(h), x.size)
    return h


def f32_from_f16(h) -> np.ndarray:
    h = _c(h, np.uint16)
    x = np.empty(h.shape, np.float32)
    lib().oracle_f32_from_f16_n(_p(h), _p(x), h.size)
    return x


def quant_row(x) -> tuple[np.ndarray, np.float32]:
    x = _c(x, np.float32)
    c = np.empty(x.shape, np.int8)
    s = np.zeros(1, np.float32)
    lib().oracle_quant_row(x.size, _p(x), _p(c), _p(s))
    return c, s[0]


def quantize(mask, S, nthreads: int | None = None):
    """fp32 states ``S[n, D, D]`` -> logical quantized representation ``(h, c, s)``."""
    S = _c(S, np.float32)
    n, D, _ = S.shape
    mask = _c(np.broadcast_to(mask, (n, D)), np.uint8)
    h = np.empty((n, D, D), np.uint16)
    c = np.empty((n, D, D), np.int8)
    s = np.empty((n, D), np.float32)
    rc = lib().oracle_quantize(D, n, _p(mask), _p(S), _p(h), _p(c), _p(s),
                               nthreads or default_threads())
    assert rc == 0
    return h, c, s


def dequantize(mask, h, c, s, nthreads: int | None = None) -> np.ndarray:
    h = _c(h, np.uint16)
    c = _c(c, np.int8)
    s = _c(s, np.float32)
    n, D, _ = c.shape
    mask = _c(np.broadcast_to(mask, (n, D)), np.uint8)
    S = np.empty((n, D, D), np.float32)
    rc = lib().oracle_dequantize(D, n, _p(mask), _p(h), _p(c), _p(s), _p(S),
                                 nthreads or default_threads())
    assert rc == 0
    return S


def _vecs(q, k, v, alpha, beta, n, D):
    q = _c(q, np.float32).reshape(n, D)
    k = _c(k, np.float32).reshape(n, D)
    v = _c(v, np.float32).reshape(n, D)
    alpha = _c(alpha, np.float32)
    per_key = 1 if alpha.size == n * D and D != 1 else 0
    alpha = alpha.reshape(n, D) if per_key else alpha.reshape(n)
    beta = _c(beta, np.float32).reshape(n)
    return q, k, v, alpha, per_key, beta


def step_fp32(S, q, k, v, alpha, beta, nthreads: int | None = None) -> np.ndarray:
    """One step on fp32 states ``S[n, D, D]`` (updated in place); returns the readout [n, D].
    ``alpha`` is [n] (GDN) or [n, D] (KDA)."""
    assert S.dtype == np.float32 and S.flags.c_contiguous
    n, D, _ = S.shape
    q, k, v, alpha, per_key, beta = _vecs(q, k, v, alpha, beta, n, D)
    out = np.empty((n, D), np.float32)
    rc = lib().oracle_step(D, n, 0, None, _p(S), None, None, None, _p(q), _p(k), _p(v),
                           _p(alpha), per_key, _p(beta), _p(out), nthreads or default_threads())
    assert rc == 0
    return out


def step_quant(mask, h, c, s, q, k, v, alpha, beta, nthreads: int | None = None) -> np.ndarray:
    """One step on the quantized representation (``h, c, s`` updated in place); returns the
    readout [n, D]. Uniform INT8 is ``mask`` all zero."""
    for a, t in ((h, np.uint16), (c, np.int8), (s, np.float32)):
        assert a.dtype == t and a.flags.c_contiguous
    n, D, _ = c.shape
    mask = _c(np.broadcast_to(mask, (n, D)), np.uint8)
    q, k, v, alpha, per_key, beta = _vecs(q, k, v, alpha, beta, n, D)
    out = np.empty((n, D), np.float32)
    rc = lib().oracle_step(D, n, 1, _p(mask), None, _p(h), _p(c), _p(s), _p(q), _p(k), _p(v),
                           _p(alpha), per_key, _p(beta), _p(out), nthreads or default_threads())
    assert rc == 0
    return out


def select_rows(S, abar, r: int):
    """Row selection for ``S[n_slots, H, D, D]`` with mean decay ``abar[H, D]``.
    Returns ``(rows int32 [H, r] ascending, score float64 [H, D])``."""
    S = _c(S, np.float32)
    n_slots, H, D, _ = S.shape
    abar = _c(np.broadcast_to(abar, (H, D)), np.float64)
    rows = np.empty((H, r), np.int32)
    score = np.empty((H, D), np.float64)
    rc = lib().oracle_select_rows(D, H, n_slots, _p(S), _p(abar), r, _p(rows), _p(score))
    assert rc == 0
    return rows, score


def int8_row_error(x) -> float:
    """Squared error of storing row ``x`` with the INT8 rule (binary64)."""
    x = _c(x, np.float32)
    return float(lib().oracle_int8_row_error(x.size, _p(x)))


def risk_scores(S, abar) -> np.ndarray:
    """Per (head, key row) risk score for calibration states ``S[n_slots, H, D, D]`` and mean
    gates ``abar[H, D]`` (float32); returns float64 [H, D]."""
    S = _c(S, np.float32)
    n_slots, H, D, _ = S.shape
    abar = _c(np.broadcast_to(abar, (H, D)), np.float32)
    score = np.empty((H, D), np.float64)
    rc = lib().oracle_risk_scores(D, H, n_slots, _p(S), _p(abar), _p(score))
    assert rc == 0
    return score


def budget_rows(D: int, H: int, bits_per_value: float, g: int = 1, r_max: int | None = None) -> int:
    return int(lib().oracle_budget_rows(D, H, float(bits_per_value), g, D if r_max is None else r_max))


def allocate_rows(score, R: int, g: int = 1, r_max: int | None = None):
    """Allocation of ``R`` FP16 rows over the heads of ``score[H, D]`` in groups of ``g``.
    Returns ``(r int32 [H], map int32 [H, D])``: map[h, :r[h]] are head h's FP16 rows ascending,
    the rest its INT8 rows ascending."""
    score = _c(score, np.float64)
    H, D = score.shape
    r = np.empty(H, np.int32)
    m = np.empty((H, D), np.int32)
    rc = lib().oracle_allocate_rows(D, H, _p(score), R, g, D if r_max is None else r_max, _p(r), _p(m))
    assert rc == 0
    return r, m


def prestep(q, k, g, b):
    """Pre-step of the layer inputs: ``q, k [n, D]`` (any float), gate logits ``g`` [n] or
    [n, D], beta logits ``b`` [n]. Returns fp32 ``(q_hat, k_hat, alpha, beta)``."""
    q = _c(q, np.float32)
    n, D = q.shape
    k = _c(k, np.float32).reshape(n, D)
    g = _c(g, np.float32)
    per_key = 1 if g.size == n * D and D != 1 else 0
    g = g.reshape(n, D) if per_key else g.reshape(n)
    b = _c(b, np.float32).reshape(n)
    qo, ko = np.empty((n, D), np.float32), np.empty((n, D), np.float32)
    ao = np.empty(g.shape, np.float32)
    bo = np.empty(n, np.float32)
    rc = lib().oracle_prestep(D, n, _p(q), _p(k), _p(g), per_key, _p(b), _p(qo), _p(ko), _p(ao), _p(bo))
    assert rc == 0
    return qo, ko, ao, bo


class Window:
    """Per-window requantization state of ``n`` units in the oracle: the quantized arrays
    ``(h, c, s)`` (updated in place at window ends), each unit's exact binary64 state within its
    window, and the number of tokens already applied in the current window."""

    def __init__(self, mask, h, c, s, W: int):
        for a, t in ((h, np.uint16), (c, np.int8), (s, np.float32)):
            assert a.dtype == t and a.flags.c_contiguous
        n, D, _ = c.shape
        self.mask = _c(np.broadcast_to(mask, (n, D)), np.uint8)
        self.h, self.c, self.s, self.W = h, c, s, W
        self.Sx = np.zeros((n, D, D), np.float64)
        self.t = np.zeros(n, np.int32)

    def step(self, q, k, v, alpha, beta, nthreads: int | None = None) -> np.ndarray:
        n, D, _ = self.c.shape
        q, k, v, alpha, per_key, beta = _vecs(q, k, v, alpha, beta, n, D)
        out = np.empty((n, D), np.float32)
        rc = lib().oracle_window_step(D, n, _p(self.mask), _p(self.h), _p(self.c), _p(self.s),
                                      _p(self.Sx), _p(self.t), self.W, _p(q), _p(k), _p(v),
                                      _p(alpha), per_key, _p(beta), _p(out),
                                      nthreads or default_threads())
        assert rc == 0
        return out

    def flush(self) -> None:
        n, D, _ = self.c.shape
        rc = lib().oracle_window_flush(D, n, _p(self.mask), _p(self.h), _p(self.c), _p(self.s),
                                       _p(self.Sx), _p(self.t))
        assert rc == 0


# ---- STEPQuant-style state -------------------------------------------------------------------
def stq_quantize(bits, w, S):
    """fp32 states ``S[n, D, D]`` -> ``(h, c, rf, cs)`` for per-row code widths ``bits[n, D]``
    (16 = pivot, 8, 6, 4) and row-impact scores ``w[n, D]``."""
    S = _c(S, np.float32)
    n, D, _ = S.shape
    bits = _c(np.broadcast_to(bits, (n, D)), np.uint8)
    w = _c(np.broadcast_to(w, (n, D)), np.float32)
    h = np.empty((n, D, D), np.uint16)
    c = np.empty((n, D, D), np.int8)
    rf = np.empty((n, D), np.uint16)
    cs = np.empty((n, D), np.uint16)
    rc = lib().oracle_stq_quantize(D, n, _p(bits), _p(w), _p(S), _p(h), _p(c), _p(rf), _p(cs))
    assert rc == 0
    return h, c, rf, cs


def stq_dequantize(bits, h, c, rf, cs):
    h, c = _c(h, np.uint16), _c(c, np.int8)
    rf, cs = _c(rf, np.uint16), _c(cs, np.uint16)
    n, D, _ = c.shape
    bits = _c(np.broadcast_to(bits, (n, D)), np.uint8)
    S = np.empty((n, D, D), np.float32)
    rc = lib().oracle_stq_dequantize(D, n, _p(bits), _p(h), _p(c), _p(rf), _p(cs), _p(S))
    assert rc == 0
    return S


def stq_step(bits, w, h, c, rf, cs, q, k, v, alpha, beta, nthreads: int | None = None,
             return_x: bool = False):
    """One step; returns ``(out [n, D], (h2, c2, rf2, cs2))`` (the inputs are not modified), and
    with ``return_x`` also the new states X rounded to binary32 [n, D, D]."""
    h, c = _c(h, np.uint16), _c(c, np.int8)
    rf, cs = _c(rf, np.uint16), _c(cs, np.uint16)
    n, D, _ = c.shape
    bits = _c(np.broadcast_to(bits, (n, D)), np.uint8)
    w = _c(np.broadcast_to(w, (n, D)), np.float32)
    q, k, v, alpha, per_key, beta = _vecs(q, k, v, alpha, beta, n, D)
    h2, c2, rf2, cs2 = np.empty_like(h), np.empty_like(c), np.empty_like(rf), np.empty_like(cs)
    out = np.empty((n, D), np.float32)
    X = np.empty((n, D, D), np.float32) if return_x else None
    rc = lib().oracle_stq_step(D, n, _p(bits), _p(w), _p(h), _p(c), _p(rf), _p(cs), _p(h2), _p(c2),
                               _p(rf2), _p(cs2), _p(q), _p(k), _p(v), _p(alpha), per_key, _p(beta),
                               _p(out), _p(X), nthreads or default_threads())
    assert rc == 0
    return (out, (h2, c2, rf2, cs2), X) if return_x else (out, (h2, c2, rf2, cs2))


def stq_fit_rows(bits, X, cs):
    """The fit's second half for given column scales: ``(h, c, rf)`` of states ``X[n, D, D]``
    with column scales ``cs[n, D]`` (binary16 bits)."""
    X = _c(X, np.float32)
    n, D, _ = X.shape
    bits = _c(np.broadcast_to(bits, (n, D)), np.uint8)
    cs = _c(np.broadcast_to(cs, (n, D)), np.uint16)
    h = np.empty((n, D, D), np.uint16)
    c = np.empty((n, D, D), np.int8)
    rf = np.empty((n, D), np.uint16)
    rc = lib().oracle_stq_fit_rows(D, n, _p(bits), _p(X), _p(cs), _p(h), _p(c), _p(rf))
    assert rc == 0
    return h, c, rf
