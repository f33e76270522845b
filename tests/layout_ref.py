"""Test-side conversion between the oracle's logical quantized state and the byte layout that
include/damp.h documents for the DAMP pool (written from that documentation, in numpy; shares
no code with the library or the oracle).

Logical form (oracle): mask [H, D] (1 = FP16 row), h uint16 [n, H, D, D], c int8 [n, H, D, D],
s float32 [n, H, D], all in original key-row order.
Block of one (slot, head), rows in storage order (FP16 rows ascending, then INT8 rows ascending):
    r*D binary16 | (D-r)*D int8 | (D-r) fp32 scales | zero padding to the block stride.
"""
from __future__ import annotations

import numpy as np


def storage_order(rows: np.ndarray, D: int) -> np.ndarray:
    """[H, r] FP16 rows -> [H, D] storage-row -> key-row map."""
    H, r = rows.shape
    perm = np.empty((H, D), np.int64)
    for h in range(H):
        rest = np.setdiff1d(np.arange(D), rows[h])
        perm[h] = np.concatenate([rows[h], rest])
    return perm


def block_data_bytes(D: int, r: int) -> int:
    return 2 * r * D + (D - r) * D + 4 * (D - r)


def block_stride(D: int, r: int) -> int:
    return (block_data_bytes(D, r) + 255) // 256 * 256


def pack(rows: np.ndarray, h: np.ndarray, c: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Logical (n, H, ...) -> uint8 blocks [n, H, stride]."""
    n, H, D, _ = c.shape
    r = rows.shape[1]
    stride = block_stride(D, r)
    out = np.zeros((n, H, stride), np.uint8)
    perm = storage_order(rows, D)
    o1, o2 = 2 * r * D, 2 * r * D + (D - r) * D
    for hh in range(H):
        p16, p8 = perm[hh, :r], perm[hh, r:]
        out[:, hh, :o1] = np.ascontiguousarray(h[:, hh][:, p16, :]).view(np.uint8).reshape(n, -1)
        out[:, hh, o1:o2] = np.ascontiguousarray(c[:, hh][:, p8, :]).view(np.uint8).reshape(n, -1)
        out[:, hh, o2:o2 + 4 * (D - r)] = np.ascontiguousarray(s[:, hh][:, p8]).view(np.uint8).reshape(n, -1)
    return out


def unpack(rows: np.ndarray, blocks: np.ndarray, D: int):
    """uint8 blocks [n, H, stride] -> logical (h, c, s); entries of the other row kind are 0."""
    n, H, _ = blocks.shape
    r = rows.shape[1]
    perm = storage_order(rows, D)
    o1, o2 = 2 * r * D, 2 * r * D + (D - r) * D
    h = np.zeros((n, H, D, D), np.uint16)
    c = np.zeros((n, H, D, D), np.int8)
    s = np.zeros((n, H, D), np.float32)
    for hh in range(H):
        p16, p8 = perm[hh, :r], perm[hh, r:]
        b = np.ascontiguousarray(blocks[:, hh])
        h[:, hh][:, p16, :] = b[:, :o1].copy().view(np.uint16).reshape(n, r, D)
        c[:, hh][:, p8, :] = b[:, o1:o2].copy().view(np.int8).reshape(n, D - r, D)
        s[:, hh][:, p8] = b[:, o2:o2 + 4 * (D - r)].copy().view(np.float32).reshape(n, D - r)
    return h, c, s


# ---- per-head layout: head h has its own r_h; its block sits at offset off_h in the slot -------
def head_offsets(D: int, r_per_head) -> tuple[np.ndarray, int]:
    """Byte offset of each head's block inside a slot, and the slot's bytes."""
    off, o = [], 0
    for r in r_per_head:
        off.append(o)
        o += block_stride(D, int(r))
    return np.array(off, np.int64), o


def pack_per_head(r_per_head, row_map, h, c, s) -> np.ndarray:
    """Logical (n, H, ...) -> uint8 slots [n, slot_bytes]; row_map [H, D] lists each head's
    FP16 rows then its INT8 rows (storage order)."""
    n, H, D, _ = c.shape
    off, slot = head_offsets(D, r_per_head)
    out = np.zeros((n, slot), np.uint8)
    for hh in range(H):
        r = int(r_per_head[hh])
        p16, p8 = row_map[hh, :r], row_map[hh, r:]
        o1, o2 = 2 * r * D, 2 * r * D + (D - r) * D
        b = off[hh]
        out[:, b:b + o1] = np.ascontiguousarray(h[:, hh][:, p16, :]).view(np.uint8).reshape(n, -1)
        out[:, b + o1:b + o2] = np.ascontiguousarray(c[:, hh][:, p8, :]).view(np.uint8).reshape(n, -1)
        out[:, b + o2:b + o2 + 4 * (D - r)] = np.ascontiguousarray(s[:, hh][:, p8]).view(np.uint8).reshape(n, -1)
    return out


def unpack_per_head(r_per_head, row_map, slots: np.ndarray, D: int):
    """uint8 slots [n, slot_bytes] -> logical (h, c, s); entries of the other row kind are 0."""
    n = slots.shape[0]
    H = len(r_per_head)
    off, _ = head_offsets(D, r_per_head)
    h = np.zeros((n, H, D, D), np.uint16)
    c = np.zeros((n, H, D, D), np.int8)
    s = np.zeros((n, H, D), np.float32)
    for hh in range(H):
        r = int(r_per_head[hh])
        p16, p8 = row_map[hh, :r], row_map[hh, r:]
        o1, o2 = 2 * r * D, 2 * r * D + (D - r) * D
        b = np.ascontiguousarray(slots[:, off[hh]:off[hh] + o2 + 4 * (D - r)])
        h[:, hh][:, p16, :] = b[:, :o1].copy().view(np.uint16).reshape(n, r, D)
        c[:, hh][:, p8, :] = b[:, o1:o2].copy().view(np.int8).reshape(n, D - r, D)
        s[:, hh][:, p8] = b[:, o2:o2 + 4 * (D - r)].copy().view(np.float32).reshape(n, D - r)
    return h, c, s


def mask_per_head(r_per_head, row_map, D: int) -> np.ndarray:
    """[H, D] uint8: 1 on each head's FP16 rows."""
    H = len(r_per_head)
    m = np.zeros((H, D), np.uint8)
    for hh in range(H):
        m[hh, row_map[hh, :int(r_per_head[hh])]] = 1
    return m
