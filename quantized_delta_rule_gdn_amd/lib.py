"""ctypes binding of libdamp.so (include/damp.h). Argument marshalling only.

Torch tensors provide device memory and the stream; every computation runs in the library's
HIP kernels. There is no fallback: if ``libdamp.so`` is missing or cannot be loaded, every call
raises. Shapes, dtypes, devices and contiguity are checked here so that the kernels never see
an array smaller than the sizes passed to them.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdamp.so")

DAMP_OK = 0
DAMP_ERR_INVALID_ARGUMENT = -1
DAMP_ERR_UNSUPPORTED = -2
DAMP_ERR_OUT_OF_MEMORY = -3
DAMP_ERR_SLOT_INDEX = -4
DAMP_ERR_HIP = -5

DAMP_DECAY_SCALAR = 0
DAMP_DECAY_PER_KEY = 1
DAMP_F32 = 0
DAMP_BF16 = 1
SORTED_MAX_B = 65536  # DAMP_SORTED_MAX_B: the library-held order buffer of damp_decode_step_sorted

EXPORTS = (
    "damp_block_bytes", "damp_block_data_bytes", "damp_state_bytes", "damp_state_alloc",
    "damp_state_free", "damp_state_layout", "damp_state_quantize", "damp_state_dequantize",
    "damp_decode_step", "fp32_decode_step", "uniform_int8_decode_step", "uniform_int8_quantize",
    "damp_last_error", "damp_abi_version", "damp_state_bytes_per_head",
    "damp_state_alloc_per_head", "damp_state_head_info", "damp_risk_scores", "damp_budget_rows",
    "damp_allocate_rows", "damp_decode_step_fused", "damp_window_bytes", "damp_window_step",
    "damp_window_flush", "stq_state_bytes", "stq_state_alloc", "stq_state_free",
    "stq_state_head_info", "stq_state_quantize", "stq_state_dequantize", "stq_decode_step",
    "damp_batch_order", "damp_decode_step_ordered", "damp_decode_step_fused_ordered",
    "damp_window_step_ordered", "damp_decode_step_sorted",
)


class DampError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"damp status {status}: {message}")
        self.status = status


class Layout(ctypes.Structure):
    _fields_ = [("num_slots", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("num_fp16_rows", ctypes.c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libdamp.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m quantized_delta_rule_gdn_amd.build`"
                          " or __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    LP = ctypes.POINTER(Layout)
    sig = {
        "damp_block_bytes": ([LP], SZ),
        "damp_block_data_bytes": ([LP], SZ),
        "damp_state_bytes": ([LP], SZ),
        "damp_state_alloc": ([LP, P, P, SZ, ctypes.POINTER(P)], ctypes.c_int),
        "damp_state_free": ([P], ctypes.c_int),
        "damp_state_layout": ([P, LP], ctypes.c_int),
        "damp_state_quantize": ([P, P, P, I32, P], ctypes.c_int),
        "damp_state_dequantize": ([P, P, P, I32, P], ctypes.c_int),
        "damp_decode_step": ([P, P, I32, P, P, P, ctypes.c_int, P, ctypes.c_int, P, P, P],
                             ctypes.c_int),
        "fp32_decode_step": ([P, I32, I32, I32, I32, P, I32, P, P, P, ctypes.c_int, P,
                              ctypes.c_int, P, P, P], ctypes.c_int),
        "uniform_int8_decode_step": ([P, P, I32, I32, I32, I32, P, I32, P, P, P, ctypes.c_int, P,
                                      ctypes.c_int, P, P, P], ctypes.c_int),
        "uniform_int8_quantize": ([P, P, I32, I32, I32, I32, P, P, I32, P], ctypes.c_int),
        "damp_last_error": ([], ctypes.c_char_p),
        "damp_abi_version": ([], I32),
        "damp_state_bytes_per_head": ([LP, P], SZ),
        "damp_state_alloc_per_head": ([LP, P, P, P, SZ, ctypes.POINTER(P)], ctypes.c_int),
        "damp_state_head_info": ([P, P, P, P], ctypes.c_int),
        "damp_risk_scores": ([P, I32, I32, I32, P, P, P, P], ctypes.c_int),
        "damp_budget_rows": ([I32, I32, ctypes.c_double, I32, I32], ctypes.c_int64),
        "damp_allocate_rows": ([P, I32, I32, ctypes.c_int64, I32, I32, P, P, P], ctypes.c_int),
        "damp_decode_step_fused": ([P, P, I32, P, P, P, ctypes.c_int, P, ctypes.c_int, P, P, P],
                                   ctypes.c_int),
        "damp_window_bytes": ([LP, I32], SZ),
        "damp_window_step": ([P, P, I32, P, I32, P, P, P, ctypes.c_int, P, ctypes.c_int, P, P, P],
                             ctypes.c_int),
        "damp_window_flush": ([P, P, I32, P, I32, P], ctypes.c_int),
        "stq_state_bytes": ([I32, I32, I32, P], SZ),
        "stq_state_alloc": ([I32, I32, I32, P, P, P, SZ, ctypes.POINTER(P)], ctypes.c_int),
        "stq_state_free": ([P], ctypes.c_int),
        "stq_state_head_info": ([P, P, P], ctypes.c_int),
        "stq_state_quantize": ([P, P, P, I32, P], ctypes.c_int),
        "stq_state_dequantize": ([P, P, P, I32, P], ctypes.c_int),
        "stq_decode_step": ([P, P, P, I32, P, P, P, ctypes.c_int, P, ctypes.c_int, P, P, P],
                            ctypes.c_int),
        "damp_batch_order": ([P, I32, I32, P, P], ctypes.c_int),
        "damp_decode_step_ordered": ([P, P, P, I32, P, P, P, ctypes.c_int, P, ctypes.c_int, P, P,
                                      P], ctypes.c_int),
        "damp_decode_step_fused_ordered": ([P, P, P, I32, P, P, P, ctypes.c_int, P, ctypes.c_int,
                                            P, P, P], ctypes.c_int),
        "damp_window_step_ordered": ([P, P, I32, P, P, I32, P, P, P, ctypes.c_int, P,
                                      ctypes.c_int, P, P, P], ctypes.c_int),
        "damp_decode_step_sorted": ([P, P, I32, P, P, P, ctypes.c_int, P, ctypes.c_int, P, P, P],
                                    ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def last_error() -> str:
    return load().damp_last_error().decode()


def _check(status: int) -> None:
    if status != DAMP_OK:
        raise DampError(status, last_error())


def layout(num_slots: int, num_heads: int, d: int, num_fp16_rows: int) -> Layout:
    return Layout(num_slots, num_heads, d, d, num_fp16_rows)


def block_bytes(num_slots: int, num_heads: int, d: int, num_fp16_rows: int) -> int:
    return load().damp_block_bytes(ctypes.byref(layout(num_slots, num_heads, d, num_fp16_rows)))


def block_data_bytes(num_slots: int, num_heads: int, d: int, num_fp16_rows: int) -> int:
    return load().damp_block_data_bytes(ctypes.byref(layout(num_slots, num_heads, d,
                                                            num_fp16_rows)))


def state_bytes(num_slots: int, num_heads: int, d: int, num_fp16_rows: int) -> int:
    return load().damp_state_bytes(ctypes.byref(layout(num_slots, num_heads, d, num_fp16_rows)))


# ------------------------------------------------------------------------------------------
# torch marshalling
# ------------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t) -> int:
    return t.data_ptr()


def _need(t, name, dtype, shape, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _step_vectors(slot_idx, q, k, v, alpha, beta, out, H, d):
    torch = _torch()
    if slot_idx.dim() != 1:
        raise ValueError("slot_idx must be 1-D")
    B = slot_idx.shape[0]
    dev = slot_idx.device
    _need(slot_idx, "slot_idx", torch.int32, (B,), dev)
    if q.dtype == torch.bfloat16:
        dt = DAMP_BF16
    elif q.dtype == torch.float32:
        dt = DAMP_F32
    else:
        raise TypeError(f"q/k/v dtype {q.dtype} is not float32 or bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype, (B, H, d), dev)
    if alpha.dim() == 3:
        decay = DAMP_DECAY_PER_KEY
        _need(alpha, "alpha", torch.float32, (B, H, d), dev)
    else:
        decay = DAMP_DECAY_SCALAR
        _need(alpha, "alpha", torch.float32, (B, H), dev)
    _need(beta, "beta", torch.float32, (B, H), dev)
    _need(out, "out", torch.float32, (B, H, d), dev)
    return B, dt, decay


class DampState:
    """A DAMP state pool bound to its frozen per-head FP16 row map.

    ``pool`` (uint8 device tensor of ``nbytes`` bytes) is allocated here unless given.
    Uniform layout: ``fp16_rows`` is an int array [num_heads, r] of ascending key rows per head.
    Per-head layout (``r_per_head`` given): ``fp16_rows`` is the int row map [num_heads, d] of
    ``allocate_rows`` (each head's r_h FP16 rows ascending, then its other rows ascending)."""

    def __init__(self, num_slots: int, num_heads: int, d: int, fp16_rows, pool=None,
                 device=None, r_per_head=None):
        torch = _torch()
        self.num_slots, self.num_heads, self.d = num_slots, num_heads, d
        self.per_head = r_per_head is not None
        if self.per_head:
            rh = np.ascontiguousarray(np.asarray(r_per_head, dtype=np.int32).reshape(num_heads))
            rows = np.ascontiguousarray(np.asarray(fp16_rows, dtype=np.int32).reshape(num_heads, d))
            self.r = None
            self.r_per_head = rh
            self._layout = layout(num_slots, num_heads, d, 0)
            nbytes = load().damp_state_bytes_per_head(ctypes.byref(self._layout),
                                                      rh.ctypes.data_as(ctypes.c_void_p))
        else:
            rows = np.ascontiguousarray(np.asarray(fp16_rows, dtype=np.int32).reshape(num_heads, -1))
            r = rows.shape[1]
            self.r = r
            self.r_per_head = np.full(num_heads, r, np.int32)
            self._layout = layout(num_slots, num_heads, d, r)
            nbytes = load().damp_state_bytes(ctypes.byref(self._layout))
        self.fp16_rows = rows
        if nbytes == 0:
            raise DampError(DAMP_ERR_INVALID_ARGUMENT, "invalid or unsupported layout")
        self.nbytes = nbytes
        if not self.per_head:
            self.block_bytes = load().damp_block_bytes(ctypes.byref(self._layout))
            self.block_data_bytes = load().damp_block_data_bytes(ctypes.byref(self._layout))
        if pool is None:
            pool = torch.empty(nbytes, dtype=torch.uint8,
                               device=device if device is not None else "cuda")
        _need(pool, "pool", torch.uint8, (pool.numel(),))
        if pool.numel() < nbytes:
            raise ValueError(f"pool has {pool.numel()} bytes, {nbytes} needed")
        self.pool = pool
        h = ctypes.c_void_p()
        with torch.cuda.device(pool.device):
            if self.per_head:
                _check(load().damp_state_alloc_per_head(
                    ctypes.byref(self._layout), rh.ctypes.data_as(ctypes.c_void_p),
                    rows.ctypes.data_as(ctypes.c_void_p), _ptr(pool), pool.numel(), ctypes.byref(h)))
            else:
                _check(load().damp_state_alloc(ctypes.byref(self._layout),
                                               rows.ctypes.data_as(ctypes.c_void_p) if r else None,
                                               _ptr(pool), pool.numel(), ctypes.byref(h)))
        self._h = h
        r_out = np.empty(num_heads, np.int32)
        off = np.empty(num_heads, np.int64)
        sb = ctypes.c_int64()
        _check(load().damp_state_head_info(h, r_out.ctypes.data_as(ctypes.c_void_p),
                                           off.ctypes.data_as(ctypes.c_void_p), ctypes.byref(sb)))
        self.head_offsets = off
        self.slot_bytes = sb.value

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            _check(load().damp_state_free(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def blocks(self):
        """The pool as uint8 [num_slots, num_heads, block_bytes] (a view; uniform layout)."""
        if self.per_head:
            raise ValueError("a per-head layout has no uniform block; use slots()")
        return self.pool[: self.nbytes].view(self.num_slots, self.num_heads, self.block_bytes)

    def slots(self):
        """The pool as uint8 [num_slots, slot_bytes] (a view); head h's block of a slot starts
        at head_offsets[h]."""
        return self.pool[: self.nbytes].view(self.num_slots, self.slot_bytes)

    def quantize(self, S, slot_idx, stream=None) -> None:
        torch = _torch()
        n = slot_idx.shape[0]
        _need(slot_idx, "slot_idx", torch.int32, (n,), self.pool.device)
        _need(S, "S", torch.float32, (n, self.num_heads, self.d, self.d), self.pool.device)
        _check(load().damp_state_quantize(self._h, _ptr(S), _ptr(slot_idx), n, _stream(stream)))

    def dequantize(self, slot_idx, S=None, stream=None):
        torch = _torch()
        n = slot_idx.shape[0]
        _need(slot_idx, "slot_idx", torch.int32, (n,), self.pool.device)
        if S is None:
            S = torch.empty((n, self.num_heads, self.d, self.d), dtype=torch.float32,
                            device=self.pool.device)
        _need(S, "S", torch.float32, (n, self.num_heads, self.d, self.d), self.pool.device)
        _check(load().damp_state_dequantize(self._h, _ptr(S), _ptr(slot_idx), n, _stream(stream)))
        return S

    def decode_step(self, slot_idx, q, k, v, alpha, beta, out, stream=None, order=None) -> None:
        """One decode step; with ``order`` (int32 [B], a permutation of the batch positions, as
        ``batch_order`` makes) the units are processed in that order."""
        B, dt, decay = _step_vectors(slot_idx, q, k, v, alpha, beta, out, self.num_heads, self.d)
        if slot_idx.device != self.pool.device:
            raise ValueError("slot_idx and the pool are on different devices")
        if order is None:
            _check(load().damp_decode_step(self._h, _ptr(slot_idx), B, _ptr(q), _ptr(k), _ptr(v),
                                           dt, _ptr(alpha), decay, _ptr(beta), _ptr(out),
                                           _stream(stream)))
            return
        _need(order, "order", _torch().int32, (B,), self.pool.device)
        _check(load().damp_decode_step_ordered(self._h, _ptr(slot_idx), _ptr(order), B, _ptr(q),
                                               _ptr(k), _ptr(v), dt, _ptr(alpha), decay,
                                               _ptr(beta), _ptr(out), _stream(stream)))

    def decode_step_sorted(self, slot_idx, q, k, v, alpha, beta, out, stream=None) -> None:
        """One decode step with the batch listed by slot in the library-held order buffer
        (damp_decode_step_sorted: no allocation, no workspace; calls on one device must not
        overlap). At most SORTED_MAX_B requests."""
        B, dt, decay = _step_vectors(slot_idx, q, k, v, alpha, beta, out, self.num_heads, self.d)
        if slot_idx.device != self.pool.device:
            raise ValueError("slot_idx and the pool are on different devices")
        _check(load().damp_decode_step_sorted(self._h, _ptr(slot_idx), B, _ptr(q), _ptr(k), _ptr(v),
                                              dt, _ptr(alpha), decay, _ptr(beta), _ptr(out),
                                              _stream(stream)))

    def batch_order(self, slot_idx, out=None, stream=None):
        """The batch positions by ascending slot of this pool (damp_batch_order)."""
        return batch_order(slot_idx, self.num_slots, out=out, stream=stream)


    def decode_step_fused(self, slot_idx, q, k, v, gate_logit, beta_logit, out, stream=None,
                          order=None) -> None:
        """The step with the pre-step fused: q, k unnormalised, gate and beta as logits; with
        ``order`` the units are processed in that order."""
        B, dt, decay = _step_vectors(slot_idx, q, k, v, gate_logit, beta_logit, out,
                                     self.num_heads, self.d)
        if slot_idx.device != self.pool.device:
            raise ValueError("slot_idx and the pool are on different devices")
        if order is None:
            _check(load().damp_decode_step_fused(self._h, _ptr(slot_idx), B, _ptr(q), _ptr(k),
                                                 _ptr(v), dt, _ptr(gate_logit), decay,
                                                 _ptr(beta_logit), _ptr(out), _stream(stream)))
            return
        _need(order, "order", _torch().int32, (B,), self.pool.device)
        _check(load().damp_decode_step_fused_ordered(self._h, _ptr(slot_idx), _ptr(order), B,
                                                     _ptr(q), _ptr(k), _ptr(v), dt,
                                                     _ptr(gate_logit), decay, _ptr(beta_logit),
                                                     _ptr(out), _stream(stream)))


    # ---- per-window requantization ----
    def window_buffer(self, window: int):
        """A zero-filled window buffer of the pool for windows of ``window`` tokens."""
        torch = _torch()
        lay = layout(self.num_slots, self.num_heads, self.d, 0)
        n = load().damp_window_bytes(ctypes.byref(lay), window)
        if n == 0:
            raise DampError(DAMP_ERR_INVALID_ARGUMENT, f"invalid window length {window}")
        return torch.zeros(n, dtype=torch.uint8, device=self.pool.device)

    def window_step(self, wbuf, window: int, slot_idx, q, k, v, alpha, beta, out, stream=None,
                    order=None) -> None:
        """One token of a window; with ``order`` the units are processed in that order."""
        B, dt, decay = _step_vectors(slot_idx, q, k, v, alpha, beta, out, self.num_heads, self.d)
        self._check_wbuf(wbuf, window)
        if order is None:
            _check(load().damp_window_step(self._h, _ptr(wbuf), window, _ptr(slot_idx), B, _ptr(q),
                                           _ptr(k), _ptr(v), dt, _ptr(alpha), decay, _ptr(beta),
                                           _ptr(out), _stream(stream)))
            return
        _need(order, "order", _torch().int32, (B,), self.pool.device)
        _check(load().damp_window_step_ordered(self._h, _ptr(wbuf), window, _ptr(slot_idx), _ptr(order),
                                               B, _ptr(q), _ptr(k), _ptr(v), dt, _ptr(alpha), decay,
                                               _ptr(beta), _ptr(out), _stream(stream)))

    def window_flush(self, wbuf, window: int, slot_idx, stream=None) -> None:
        torch = _torch()
        n = slot_idx.shape[0]
        _need(slot_idx, "slot_idx", torch.int32, (n,), self.pool.device)
        self._check_wbuf(wbuf, window)
        _check(load().damp_window_flush(self._h, _ptr(wbuf), window, _ptr(slot_idx), n, _stream(stream)))

    def _check_wbuf(self, wbuf, window):
        torch = _torch()
        lay = layout(self.num_slots, self.num_heads, self.d, 0)
        need = load().damp_window_bytes(ctypes.byref(lay), window)
        _need(wbuf, "window buffer", torch.uint8, (wbuf.numel(),), self.pool.device)
        if wbuf.numel() < need:
            raise ValueError(f"window buffer has {wbuf.numel()} bytes, {need} needed")


def batch_order(slot_idx, num_slots: int, out=None, stream=None):
    """int32 [B] permutation of the batch positions by ascending slot bucket of a pool of
    ``num_slots`` slots (damp_batch_order), written into ``out`` if given."""
    torch = _torch()
    B = slot_idx.shape[0]
    _need(slot_idx, "slot_idx", torch.int32, (B,))
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=slot_idx.device)
    _need(out, "order", torch.int32, (B,), slot_idx.device)
    _check(load().damp_batch_order(_ptr(slot_idx), B, num_slots, _ptr(out), _stream(stream)))
    return out


def fp32_decode_step(pool, slot_idx, q, k, v, alpha, beta, out, stream=None) -> None:
    """Decode step on an fp32 state pool [num_slots, H, d, d]."""
    torch = _torch()
    if pool.dim() != 4:
        raise ValueError("pool must be [num_slots, H, d, d]")
    S_, H, d, d2 = pool.shape
    _need(pool, "pool", torch.float32, (S_, H, d, d2), slot_idx.device)
    B, dt, decay = _step_vectors(slot_idx, q, k, v, alpha, beta, out, H, d)
    _check(load().fp32_decode_step(_ptr(pool), S_, H, d, d2, _ptr(slot_idx), B, _ptr(q),
                                   _ptr(k), _ptr(v), dt, _ptr(alpha), decay, _ptr(beta),
                                   _ptr(out), _stream(stream)))


def uniform_int8_decode_step(codes, scales, slot_idx, q, k, v, alpha, beta, out,
                             stream=None) -> None:
    """Decode step on a uniform-INT8 state: codes int8 [num_slots, H, d, d], scales fp32
    [num_slots, H, d]."""
    torch = _torch()
    if codes.dim() != 4:
        raise ValueError("codes must be [num_slots, H, d, d]")
    S_, H, d, d2 = codes.shape
    _need(codes, "codes", torch.int8, (S_, H, d, d2), slot_idx.device)
    _need(scales, "scales", torch.float32, (S_, H, d), slot_idx.device)
    B, dt, decay = _step_vectors(slot_idx, q, k, v, alpha, beta, out, H, d)
    _check(load().uniform_int8_decode_step(_ptr(codes), _ptr(scales), S_, H, d, d2,
                                           _ptr(slot_idx), B, _ptr(q), _ptr(k), _ptr(v), dt,
                                           _ptr(alpha), decay, _ptr(beta), _ptr(out),
                                           _stream(stream)))


def uniform_int8_quantize(codes, scales, S, slot_idx, stream=None) -> None:
    torch = _torch()
    S_, H, d, d2 = codes.shape
    n = slot_idx.shape[0]
    _need(codes, "codes", torch.int8, (S_, H, d, d2), slot_idx.device)
    _need(scales, "scales", torch.float32, (S_, H, d), slot_idx.device)
    _need(slot_idx, "slot_idx", torch.int32, (n,), codes.device)
    _need(S, "S", torch.float32, (n, H, d, d2), codes.device)
    _check(load().uniform_int8_quantize(_ptr(codes), _ptr(scales), S_, H, d, d2, _ptr(S),
                                        _ptr(slot_idx), n, _stream(stream)))


# ------------------------------------------------------------------------------------------
# offline calibration
# ------------------------------------------------------------------------------------------
def risk_scores(S, abar, row_error=None, score=None, stream=None):
    """Per (head, key row) risk scores of calibration states ``S`` fp32 [n, H, d, d] with mean
    gates ``abar`` fp32 [H, d]. Returns ``(score fp64 [H, d], row_error fp64 [n, H, d])``."""
    torch = _torch()
    if S.dim() != 4:
        raise ValueError("S must be [n, H, d, d]")
    n, H, d, d2 = S.shape
    dev = S.device
    _need(S, "S", torch.float32, (n, H, d, d2), dev)
    _need(abar, "abar", torch.float32, (H, d), dev)
    if row_error is None:
        row_error = torch.empty((n, H, d), dtype=torch.float64, device=dev)
    if score is None:
        score = torch.empty((H, d), dtype=torch.float64, device=dev)
    _need(row_error, "row_error", torch.float64, (n, H, d), dev)
    _need(score, "score", torch.float64, (H, d), dev)
    if d != d2:
        raise ValueError("S must be square per head")
    _check(load().damp_risk_scores(_ptr(S), n, H, d, _ptr(abar), _ptr(row_error), _ptr(score),
                                   _stream(stream)))
    return score, row_error


def budget_rows(d: int, num_heads: int, bits_per_value: float, g: int = 1, r_max: int | None = None) -> int:
    """FP16 rows per slot (all heads) that fit ``bits_per_value`` data bits per state value."""
    return int(load().damp_budget_rows(d, num_heads, float(bits_per_value), g,
                                       d if r_max is None else r_max))


def allocate_rows(score, R: int, g: int = 1, r_max: int | None = None, stream=None):
    """Allocation of ``R`` FP16 rows over the heads of ``score`` fp64 [H, d] in groups of ``g``.
    Returns device tensors ``(r int32 [H], row_map int32 [H, d])``."""
    torch = _torch()
    H, d = score.shape
    _need(score, "score", torch.float64, (H, d), score.device)
    r = torch.empty(H, dtype=torch.int32, device=score.device)
    m = torch.empty((H, d), dtype=torch.int32, device=score.device)
    _check(load().damp_allocate_rows(_ptr(score), H, d, R, g, d if r_max is None else r_max,
                                     _ptr(r), _ptr(m), _stream(stream)))
    return r, m


# ------------------------------------------------------------------------------------------
# STEPQuant-style state
# ------------------------------------------------------------------------------------------
class StqState:
    """A pool in the STEPQuant-style layout bound to its frozen precision map ``row_bits``
    (uint8 [num_heads, d]: 16 = FP16 pivot, or 8, 6, 4) and row-impact scores ``impact`` (fp32
    [num_heads, d])."""

    def __init__(self, num_slots: int, num_heads: int, d: int, row_bits, impact, pool=None,
                 device=None):
        torch = _torch()
        self.num_slots, self.num_heads, self.d = num_slots, num_heads, d
        self.row_bits = np.ascontiguousarray(np.asarray(row_bits, np.uint8).reshape(num_heads, d))
        self.impact = np.ascontiguousarray(np.asarray(impact, np.float32).reshape(num_heads, d))
        nbytes = load().stq_state_bytes(num_slots, num_heads, d,
                                        self.row_bits.ctypes.data_as(ctypes.c_void_p))
        if nbytes == 0:
            raise DampError(DAMP_ERR_INVALID_ARGUMENT, "invalid or unsupported layout")
        self.nbytes = nbytes
        if pool is None:
            pool = torch.zeros(nbytes, dtype=torch.uint8, device=device if device is not None else "cuda")
        _need(pool, "pool", torch.uint8, (pool.numel(),))
        if pool.numel() < nbytes:
            raise ValueError(f"pool has {pool.numel()} bytes, {nbytes} needed")
        self.pool = pool
        h = ctypes.c_void_p()
        with torch.cuda.device(pool.device):
            _check(load().stq_state_alloc(num_slots, num_heads, d,
                                          self.row_bits.ctypes.data_as(ctypes.c_void_p),
                                          self.impact.ctypes.data_as(ctypes.c_void_p), _ptr(pool),
                                          pool.numel(), ctypes.byref(h)))
        self._h = h
        off = np.empty(num_heads, np.int64)
        sb = ctypes.c_int64()
        _check(load().stq_state_head_info(h, off.ctypes.data_as(ctypes.c_void_p), ctypes.byref(sb)))
        self.head_offsets, self.slot_bytes = off, sb.value

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            _check(load().stq_state_free(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def slots(self, pool=None):
        """A pool as uint8 [num_slots, slot_bytes] (a view)."""
        p = self.pool if pool is None else pool
        return p[: self.nbytes].view(self.num_slots, self.slot_bytes)

    def quantize(self, S, slot_idx, stream=None) -> None:
        torch = _torch()
        n = slot_idx.shape[0]
        _need(slot_idx, "slot_idx", torch.int32, (n,), self.pool.device)
        _need(S, "S", torch.float32, (n, self.num_heads, self.d, self.d), self.pool.device)
        _check(load().stq_state_quantize(self._h, _ptr(S), _ptr(slot_idx), n, _stream(stream)))

    def dequantize(self, slot_idx, S=None, stream=None):
        torch = _torch()
        n = slot_idx.shape[0]
        _need(slot_idx, "slot_idx", torch.int32, (n,), self.pool.device)
        if S is None:
            S = torch.empty((n, self.num_heads, self.d, self.d), dtype=torch.float32, device=self.pool.device)
        _need(S, "S", torch.float32, (n, self.num_heads, self.d, self.d), self.pool.device)
        _check(load().stq_state_dequantize(self._h, _ptr(S), _ptr(slot_idx), n, _stream(stream)))
        return S

    def decode_step(self, slot_idx, q, k, v, alpha, beta, out, dst=None, stream=None) -> None:
        """One step; ``dst`` (a pool of the same size) receives the new state, else in place."""
        torch = _torch()
        B, dt, decay = _step_vectors(slot_idx, q, k, v, alpha, beta, out, self.num_heads, self.d)
        if dst is not None:
            _need(dst, "dst", torch.uint8, (dst.numel(),), self.pool.device)
            if dst.numel() < self.nbytes:
                raise ValueError(f"dst has {dst.numel()} bytes, {self.nbytes} needed")
        _check(load().stq_decode_step(self._h, _ptr(dst) if dst is not None else None, _ptr(slot_idx),
                                      B, _ptr(q), _ptr(k), _ptr(v), dt, _ptr(alpha), decay,
                                      _ptr(beta), _ptr(out), _stream(stream)))
