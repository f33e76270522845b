"""Seeded synthetic inputs for the decode-step workloads.

This module only draws random numbers and shapes them into the step's inputs (gates, unit-norm
keys and queries, value columns with heavy-tailed magnitudes, pivot-row choices, slot
indices). It holds none of the step's own arithmetic (no reconstruction, update, readout,
quantization or row scoring): the tests feed its arrays to both the CPU oracle and the GPU
library, and the benchmark feeds them to the GPU library.

The workloads stand in for the decode states of GDN / KDA models served in SGLang that the
DAMP and STEPQuant pages measure; no model, weight or dataset is used. Structure follows the
pages: 128 x 128 states per head (STEPQuant page, Table C1 and Figure B2), a handful of key
rows and value columns far above the median magnitude (Figure B2: seven or eight rows and
columns above 5x the axis-median RMS), and one state per concurrent request in a slot pool.

Every workload draws from ``numpy.random.SeedSequence(seed).spawn(...)`` streams so that each
part (initial state, warm-up inputs, step inputs, ...) can be regenerated on its own.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

GDN = 0  # scalar gate per (slot, head)
KDA = 1  # per-key-channel gate vector per (slot, head)


# ------------------------------------------------------------------------------------------
# bfloat16 handling (input casting only): round to nearest even from binary32, and widen back
# (exact). numpy has no bfloat16 type, so the 16-bit patterns travel as uint16.
# ------------------------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_widen(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class StepInputs:
    """Inputs of one decode step for ``n`` = B*H units, shapes [B, H, D] / [B, H] / [B, H, D].

    ``q, k, v`` are the exact binary32 values both sides consume; when ``dtype == "bf16"`` the
    ``*_bits`` arrays hold the bfloat16 patterns the GPU receives (``q == bf16_widen(q_bits)``).
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray  # [B, H] (GDN) or [B, H, D] (KDA), float32 in (0, 1)
    beta: np.ndarray   # [B, H], float32 in (0, 1)
    dtype: str
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None


def _unit_norm(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _sigmoid_f32(g: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-g.astype(np.float64)))).astype(np.float32)


def step_inputs(rng: np.random.Generator, B: int, H: int, D: int, decay: int = GDN,
                dtype: str = "bf16", col_mult: np.ndarray | None = None,
                gate_mean: float = 0.0) -> StepInputs:
    """q, k ~ N(0, 1) then L2-normalised in fp32; v ~ N(0, 1) (times the per-head column
    multipliers ``col_mult[H, D]`` if given); alpha = exp(-softplus(g)) = sigmoid(-g) with
    g ~ N(gate_mean, 1), one per (slot, head) for GDN or per key channel for KDA;
    beta = sigmoid(N(0,1)). Draw order: q, k, v, g, beta."""
    q = _unit_norm(rng.standard_normal((B, H, D), dtype=np.float32))
    k = _unit_norm(rng.standard_normal((B, H, D), dtype=np.float32))
    v = rng.standard_normal((B, H, D), dtype=np.float32)
    if col_mult is not None:
        v = (v * col_mult[None, :, :]).astype(np.float32)
    g = rng.standard_normal((B, H, D) if decay == KDA else (B, H))
    if gate_mean:
        g = g + gate_mean
    alpha = _sigmoid_f32(-g)
    beta = _sigmoid_f32(rng.standard_normal((B, H)))
    if dtype == "fp32":
        return StepInputs(q, k, v, alpha, beta, "fp32")
    if dtype != "bf16":
        raise ValueError(dtype)
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    return StepInputs(bf16_widen(qb), bf16_widen(kb), bf16_widen(vb), alpha, beta, "bf16",
                      qb, kb, vb)


def random_rows(rng: np.random.Generator, H: int, D: int, r: int) -> np.ndarray:
    """r distinct key rows per head drawn without replacement, ascending: int32 [H, r]."""
    return np.stack([np.sort(rng.choice(D, r, replace=False)) for _ in range(H)]).astype(np.int32)


def rows_to_mask(rows: np.ndarray, D: int) -> np.ndarray:
    """[H, r] row lists -> uint8 [H, D] mask (1 = FP16 row)."""
    H = rows.shape[0]
    m = np.zeros((H, D), np.uint8)
    for h in range(H):
        m[h, rows[h]] = 1
    return m


def normal_states(rng: np.random.Generator, shape, std: float = 0.1) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


# ------------------------------------------------------------------------------------------
# Workloads. Each returns plain arrays; the caller runs warm-up, selection and quantization
# with whichever implementation it is testing or timing.
# ------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    pool_slots: int   # slots in the state pool
    batch: int        # active slots per step
    heads: int
    d: int
    fp16_rows: int
    decay: int
    dtype: str        # q/k/v dtype of the measured step
    steps: int        # decode steps of the measured part


TINY = Workload("tiny", 1000, 1, 1, 2, 16, 2, GDN, "fp32", 8)
GDN64 = Workload("gdn64", 1001, 64, 64, 32, 128, 24, GDN, "bf16", 1)
KDA256 = Workload("kda256", 1002, 256, 256, 32, 128, 24, KDA, "bf16", 1)
POOL4096 = Workload("pool4096", 1003, 4096, 1024, 32, 128, 24, GDN, "bf16", 1)
DRIFT = Workload("drift", 1004, 64, 64, 32, 128, 24, GDN, "bf16", 2048)
WORKLOADS = {w.name: w for w in (TINY, GDN64, KDA256, POOL4096, DRIFT)}

GDN64_WARMUP_STEPS = 256
KDA256_OUTLIER_ROWS = 4      # 3% of 128 key rows, rounded
KDA256_OUTLIER_GAIN = 20.0


def _streams(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def tiny():
    """1 slot, 2 GDN heads, D = 16, 2 FP16 rows per head drawn by seed, S0 ~ N(0, 0.1),
    8 steps of fp32 inputs. Returns (rows [H, r], S0 [1, H, D, D], [StepInputs] * 8)."""
    w = TINY
    r0, r1, r2 = _streams(w.seed, 3)
    rows = random_rows(r0, w.heads, w.d, w.fp16_rows)
    S0 = normal_states(r1, (w.pool_slots, w.heads, w.d, w.d))
    steps = [step_inputs(r2, w.batch, w.heads, w.d, GDN, "fp32") for _ in range(w.steps)]
    return rows, S0, steps


def gdn64_warmup(step: int | None = None):
    """The 256 fp32 warm-up steps of the 64-slot GDN workload, starting from S = 0.
    Yields StepInputs for slots 0..63 in order (or returns one step if ``step`` is given)."""
    w = GDN64
    if step is not None:
        return step_inputs(np.random.default_rng([w.seed, 1, step]), w.batch, w.heads, w.d,
                           GDN, "fp32")
    return (gdn64_warmup(t) for t in range(GDN64_WARMUP_STEPS))


def gdn64_step() -> StepInputs:
    """The measured bf16 step of the 64-slot GDN workload."""
    w = GDN64
    return step_inputs(np.random.default_rng([w.seed, 2]), w.batch, w.heads, w.d, GDN, "bf16")


def drift_step(t: int, gate_mean: float = 0.0) -> StepInputs:
    """Step t (0..2047) of the drift run, continuing from the warmed 64-slot GDN state.
    ``gate_mean`` < 0 gives the slow-decay variant (alpha near 1: errors are retained longer)."""
    w = DRIFT
    return step_inputs(np.random.default_rng([w.seed, 1, t]), w.batch, w.heads, w.d, GDN, "bf16",
                       gate_mean=gate_mean)


def kda256(slots: int | None = None):
    """256 slots x 32 KDA heads. S0 ~ N(0, 0.1); value-column multipliers m[h, j] ~
    lognormal(0, 1) scale S0's columns and v (column outliers that persist); per-key gates.
    Returns (S0 [n, H, D, D], col_mult [H, D], StepInputs for the n slots). ``slots`` limits n
    for small runs: slot i's state has its own stream, so the first n slots are the same
    arrays as in the full workload."""
    w = KDA256
    n = w.batch if slots is None else slots
    col_mult = np.random.default_rng([w.seed, 0]).lognormal(0.0, 1.0, (w.heads, w.d))
    col_mult = col_mult.astype(np.float32)
    S0 = np.empty((n, w.heads, w.d, w.d), np.float32)
    for i in range(n):
        S0[i] = normal_states(np.random.default_rng([w.seed, 1, i]), (w.heads, w.d, w.d))
        S0[i] *= col_mult[:, None, :]
    inp = step_inputs(np.random.default_rng([w.seed, 2]), w.batch, w.heads, w.d, KDA, "bf16",
                      col_mult)
    if n != w.batch:
        inp = StepInputs(inp.q[:n], inp.k[:n], inp.v[:n], inp.alpha[:n], inp.beta[:n],
                         inp.dtype, inp.q_bits[:n], inp.k_bits[:n], inp.v_bits[:n])
    return S0, col_mult, inp


def kda256_step() -> StepInputs:
    """The step inputs of the KDA workload alone (the same draws kda256() returns)."""
    w = KDA256
    col_mult = np.random.default_rng([w.seed, 0]).lognormal(0.0, 1.0, (w.heads, w.d))
    return step_inputs(np.random.default_rng([w.seed, 2]), w.batch, w.heads, w.d, KDA, "bf16",
                       col_mult.astype(np.float32))


def kda256_outlier_rows(int8_rows: np.ndarray) -> np.ndarray:
    """Given, per head, the key rows that are stored in INT8 (int [H, D - r]), draw 4 of them
    per head as outlier rows (scaled x20 by the caller, so that INT8 scales see outliers).
    Returns int32 [H, 4] ascending."""
    rng = np.random.default_rng([KDA256.seed, 3])
    return np.stack([np.sort(rng.choice(row, KDA256_OUTLIER_ROWS, replace=False))
                     for row in int8_rows]).astype(np.int32)


def pool4096_slots() -> np.ndarray:
    """1024 distinct active slots of the 4096-slot pool, int32, in draw order."""
    w = POOL4096
    return np.random.default_rng([w.seed, 0]).choice(w.pool_slots, w.batch,
                                                     replace=False).astype(np.int32)


def pool4096_rows() -> np.ndarray:
    """24 FP16 key rows per head drawn by seed (the states are i.i.d., so a score would not
    single out any row). int32 [32, 24]."""
    w = POOL4096
    return random_rows(np.random.default_rng([w.seed, 1]), w.heads, w.d, w.fp16_rows)


def pool4096_states(first: int, count: int) -> np.ndarray:
    """States of active slots ``first .. first+count-1`` (in slot-array order), N(0, 0.1):
    float32 [count, H, D, D]. Slot ``i``'s state is drawn from its own stream so that any
    subset can be regenerated."""
    w = POOL4096
    out = np.empty((count, w.heads, w.d, w.d), np.float32)
    for i in range(count):
        out[i] = normal_states(np.random.default_rng([w.seed, 2, first + i]),
                               (w.heads, w.d, w.d))
    return out


def pool4096_step(which: int = 0) -> StepInputs:
    """Input set ``which`` (0..3) of the pool workload; the benchmark cycles through 4 sets."""
    w = POOL4096
    return step_inputs(np.random.default_rng([w.seed, 3, which]), w.batch, w.heads, w.d,
                       GDN, "bf16")


# ---- budgeted selection: calibration data standing in for fp32 warm-up traces ----------------
BUDGET_SEED = 1005
BUDGET_CAL_STATES = 64


def budget_calibration(H: int = 32, D: int = 128, n: int = BUDGET_CAL_STATES, seed: int = BUDGET_SEED,
                       per_key: bool = False):
    """Calibration states and mean gates with the structure the DAMP pages report: a few key
    rows with large magnitude per head (the quantization-error energy concentrates there) and
    decay rates that differ between heads (GDN) or key channels (KDA) but not between states.
    States: N(0, 0.1), 4 random key rows per head times 10**U(0, 1.3). Mean gates:
    sigmoid(-c) with c ~ N(0, 1) per head (GDN, repeated over the head's rows) or per key
    channel (KDA). Returns (S float32 [n, H, D, D], abar float32 [H, D])."""
    rng = np.random.default_rng(seed)
    S = normal_states(rng, (n, H, D, D), 0.1)
    for h in range(H):
        rows = rng.choice(D, 4, replace=False)
        S[:, h, rows, :] *= (10.0 ** rng.uniform(0.0, 1.3, (4, 1))).astype(np.float32)
    c = rng.standard_normal((H, D) if per_key else (H, 1))
    abar = np.broadcast_to(_sigmoid_f32(-c), (H, D)).astype(np.float32)
    return S, np.ascontiguousarray(abar)


def raw_step_inputs(rng: np.random.Generator, B: int, H: int, D: int, decay: int = GDN,
                    dtype: str = "bf16") -> StepInputs:
    """Inputs of the fused pre-step, as a layer's projections give them: q, k ~ N(0, 1) times a
    per-(slot, head) magnitude 10**U(-1, 1) (not normalised), v ~ N(0, 1); ``alpha`` holds gate
    logits g ~ N(0, 1) (per (slot, head) or per key channel) and ``beta`` logits b ~ N(0, 1).
    Draw order: q, k, magnitudes, v, g, b."""
    q = rng.standard_normal((B, H, D), dtype=np.float32)
    k = rng.standard_normal((B, H, D), dtype=np.float32)
    mag = (10.0 ** rng.uniform(-1.0, 1.0, (2, B, H, 1))).astype(np.float32)
    q = (q * mag[0]).astype(np.float32)
    k = (k * mag[1]).astype(np.float32)
    v = rng.standard_normal((B, H, D), dtype=np.float32)
    g = rng.standard_normal((B, H, D) if decay == KDA else (B, H)).astype(np.float32)
    b = rng.standard_normal((B, H)).astype(np.float32)
    if dtype == "fp32":
        return StepInputs(q, k, v, g, b, "fp32")
    if dtype != "bf16":
        raise ValueError(dtype)
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    return StepInputs(bf16_widen(qb), bf16_widen(kb), bf16_widen(vb), g, b, "bf16", qb, kb, vb)


# ---- STEPQuant-style precision maps ----------------------------------------------------------
STQ_SEED = 1006


def stq_map(rng: np.random.Generator, H: int, D: int, pivots: int = 2):
    """A frozen precision map at a nominal 6-bit budget with row-impact scores: impact
    lognormal(0, 1) per key row; per head the `pivots` rows of largest impact are FP16 pivots,
    then the next quarter of the rows by impact 8-bit, the next half 6-bit and the rest 4-bit
    (integer widths from {4, 6, 8}, mean 6 bits). Returns (row_bits uint8 [H, D], impact float32
    [H, D])."""
    impact = np.exp(rng.standard_normal((H, D))).astype(np.float32)
    bits = np.empty((H, D), np.uint8)
    for h in range(H):
        order = np.argsort(-impact[h], kind="stable")
        rest = D - pivots
        n8, n6 = rest // 4, rest // 2
        bits[h, order[:pivots]] = 16
        bits[h, order[pivots:pivots + n8]] = 8
        bits[h, order[pivots + n8:pivots + n8 + n6]] = 6
        bits[h, order[pivots + n8 + n6:]] = 4
    return bits, impact
