"""Shared helpers of the GPU parity tests: upload oracle-made inputs, run the library's entry
points through the Python binding (which calls the C ABI), download, and compare with the
tolerances the tests state.

Tolerances (GPU vs oracle, from identical input states):
  readout                elementwise |got - ref| <= 1e-5 + 1e-3 |ref|
  INT8 codes             >= 99.9% equal, |delta| <= 1 everywhere
  FP16 rows              <= 1 ulp of binary16; infinities bit for bit
  INT8 scales            |got - ref| <= 1e-6 |ref| (exact when ref == 0)
  fp32 state             |got - ref| <= the worst-case binary32 error bound of the step's
                         arithmetic (fp32_state_bound below), computed per element
"""
from __future__ import annotations

import numpy as np
import torch

import layout_ref
from quantized_delta_rule_gdn_amd import lib

SENTINEL = 0xA5


def to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return to_dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def step_tensors(inp):
    """StepInputs -> (q, k, v, alpha, beta) device tensors in the step's dtype."""
    if inp.dtype == "bf16":
        q, k, v = bf16_dev(inp.q_bits), bf16_dev(inp.k_bits), bf16_dev(inp.v_bits)
    else:
        q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    return q, k, v, to_dev(inp.alpha.astype(np.float32)), to_dev(inp.beta.astype(np.float32))


def ref_vectors(inp, B, H, D):
    """Flattened fp32 vectors in the oracle's [n = B*H] unit order."""
    n = B * H
    alpha = inp.alpha.reshape(n, D) if inp.alpha.ndim == 3 else inp.alpha.reshape(n)
    return (inp.q.reshape(n, D), inp.k.reshape(n, D), inp.v.reshape(n, D), alpha,
            inp.beta.reshape(n))


# ------------------------------------------------------------------------------------------
# running the three formats on the GPU from logical (oracle) states
# ------------------------------------------------------------------------------------------
class DampPool:
    """A DAMP pool on the device holding the given logical states at ``slots``; every other
    block is filled with a sentinel byte."""

    def __init__(self, rows, h, c, s, slots, num_slots):
        n, H, D, _ = c.shape
        self.rows, self.D, self.H = rows, D, H
        self.state = lib.DampState(num_slots, H, D, rows)
        self.state.pool.fill_(SENTINEL)
        self.slots = np.asarray(slots, np.int32)
        blocks = to_dev(layout_ref.pack(rows, h, c, s))
        self.state.blocks()[torch.from_numpy(self.slots).long().cuda()] = blocks
        self.slot_dev = to_dev(self.slots)

    def step(self, inp, slot_order=None):
        B = len(self.slots)
        q, k, v, a, b = step_tensors(inp)
        out = torch.empty((B, self.H, self.D), dtype=torch.float32, device="cuda")
        self.state.decode_step(self.slot_dev, q, k, v, a, b, out)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def logical(self):
        blocks = self.state.blocks()[torch.from_numpy(self.slots).long().cuda()].cpu().numpy()
        return layout_ref.unpack(self.rows, blocks, self.D)


def gpu_fp32_step(S, inp, slots, num_slots):
    """S [B, H, D, D] at ``slots`` of an fp32 pool; returns (out, new S)."""
    B, H, D, _ = S.shape
    pool = torch.full((num_slots, H, D, D), float("nan"), dtype=torch.float32, device="cuda")
    sl = torch.from_numpy(np.asarray(slots, np.int64)).cuda()
    pool[sl] = to_dev(S)
    q, k, v, a, b = step_tensors(inp)
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    lib.fp32_decode_step(pool, to_dev(np.asarray(slots, np.int32)), q, k, v, a, b, out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), pool[sl].cpu().numpy()


def gpu_int8_step(c, s, inp, slots, num_slots):
    B, H, D, _ = c.shape
    codes = torch.zeros((num_slots, H, D, D), dtype=torch.int8, device="cuda")
    scales = torch.zeros((num_slots, H, D), dtype=torch.float32, device="cuda")
    sl = torch.from_numpy(np.asarray(slots, np.int64)).cuda()
    codes[sl] = to_dev(c)
    scales[sl] = to_dev(s)
    q, k, v, a, b = step_tensors(inp)
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    lib.uniform_int8_decode_step(codes, scales, to_dev(np.asarray(slots, np.int32)), q, k, v, a,
                                 b, out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), codes[sl].cpu().numpy(), scales[sl].cpu().numpy()


# ------------------------------------------------------------------------------------------
# comparisons
# ------------------------------------------------------------------------------------------
def check_readout(got, ref):
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    err = np.abs(got - ref)
    bad = err > 1e-5 + 1e-3 * np.abs(ref)
    assert not bad.any(), f"readout: {bad.sum()} of {bad.size} outside rtol 1e-3 / atol 1e-5, " \
                          f"max err {err.max():.3g}"
    return float((err / (np.abs(ref) + 1e-30)).max())


def _f16_ord(bits):
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def check_quant(mask, got, ref, scale_abs=0.0, min_code_eq=0.999):
    """mask broadcastable to [n, H, D] (1 = FP16 row); got/ref = (h, c, s) logical arrays.
    scale_abs: an absolute allowance added to the scales' relative bound, for rows whose
    arithmetic runs in the binary32 subnormal range (where rounding errors are absolute).
    min_code_eq: the equal-code fraction; a caller whose INT8 rows share one code pattern (a
    rank-one state) lowers it and checks instead that every differing code sits at a tie."""
    hg, cg, sg = got
    hr, cr, sr = ref
    m = np.broadcast_to(mask, sr.shape).astype(bool)
    stats = {}
    if m.any():
        ulp = np.abs(_f16_ord(hg[m]) - _f16_ord(hr[m]))
        stats["fp16_max_ulp"] = int(ulp.max())
        assert ulp.max() <= 1, f"FP16 rows: max {ulp.max()} ulp"
        # an infinity is one step from the largest finite value in that order: where either side
        # is not finite, the bits must agree
        nf = ((hg[m] & 0x7C00) == 0x7C00) | ((hr[m] & 0x7C00) == 0x7C00)
        stats["fp16_nonfinite"] = int(nf.sum())
        assert np.array_equal(hg[m][nf], hr[m][nf]), "FP16 rows: a non-finite value differs"
    if (~m).any():
        d = np.abs(cg[~m].astype(np.int32) - cr[~m].astype(np.int32))
        eq = float((d == 0).mean())
        stats["code_eq_frac"] = eq
        stats["code_max_abs"] = int(d.max())
        assert d.max() <= 1, f"INT8 codes differ by {d.max()}"
        assert eq >= min_code_eq, f"INT8 codes equal on {eq:.6f} < {min_code_eq}"
        sgv, srv = sg[~m].astype(np.float64), sr[~m].astype(np.float64)
        zero = srv == 0
        assert np.array_equal(sgv[zero], srv[zero]), "scale of an all-zero row is not 0"
        rel = np.abs(sgv[~zero] - srv[~zero]) / srv[~zero] if (~zero).any() else np.zeros(1)
        stats["scale_max_rel"] = float(rel.max())
        if scale_abs:
            over = np.abs(sgv[~zero] - srv[~zero]) - (1e-6 * srv[~zero] + scale_abs)
            assert (over <= 0).all(), f"INT8 scales: {int((over > 0).sum())} beyond 1e-6 rel + {scale_abs:.3g}"
        else:
            assert rel.max() <= 1e-6, f"INT8 scales: max rel {rel.max():.3g}"
    return stats


EPS32 = 2.0 ** -24


def fp32_state_bound(S_hat, alpha, k, v, beta, X_ref):
    """Per-element worst-case bound of |X_gpu - X_exact| for the fp32-state step, from the
    binary32 error model fl(a op b) = (a op b)(1 + e), |e| <= 2^-24, for any summation order:
      S' = fl(a S_hat)                              error <= eps |S'|
      u_j = sum_i k_i S'_ij (D terms, any order)    error <= gamma_{D+1} sum_i |k_i| |S'_ij|
                                                             + sum_i |k_i| eps |S'_ij|
      delta_j = fl(beta fl(v_j - u_j))              error <= |beta| (|du_j| + 2 eps (|v_j| + |u_j|))
      X_ij = fl(S'_ij + k_i delta_j)                error <= eps |S'_ij| + |k_i| |d delta_j| + eps |X_ij|
    plus the reference's own rounding to binary32 (eps |X_ij|). Shapes: S_hat [n, D, D],
    alpha [n] or [n, D], k, v [n, D], beta [n]."""
    n, D, _ = S_hat.shape
    a = alpha.reshape(n, -1, 1) if alpha.ndim == 2 else alpha.reshape(n, 1, 1)
    Sp = np.abs(a.astype(np.float64) * S_hat.astype(np.float64))
    kk = np.abs(k.astype(np.float64))
    g = (D + 1) * EPS32 / (1 - (D + 1) * EPS32)
    sum_abs = np.einsum("ni,nij->nj", kk, Sp)
    du = (g + EPS32) * sum_abs
    dd = np.abs(beta.reshape(n, 1)) * (du + 2 * EPS32 * (np.abs(v) + sum_abs))
    return 2 * EPS32 * Sp + kk[:, :, None] * dd[:, None, :] + 2 * EPS32 * np.abs(X_ref)


def check_fp32_state(got, ref, bound):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    bad = err > bound
    assert not bad.any(), f"fp32 state: {bad.sum()} elements above the error bound"
    return float(err.max())
