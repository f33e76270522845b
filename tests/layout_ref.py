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


# ---- STEPQuant-style layout (written from include/damp.h) ------------------------------------
STQ_WIDTHS = (16, 8, 6, 4)


def stq_storage(row_bits_h: np.ndarray) -> np.ndarray:
    """One head's storage order: pivots, 8-bit, 6-bit, 4-bit rows, each ascending."""
    return np.concatenate([np.flatnonzero(row_bits_h == b) for b in STQ_WIDTHS])


def _up128(x: int) -> int:
    return (x + 127) // 128 * 128


def stq_regions(D: int, row_bits_h: np.ndarray) -> dict:
    """Byte offsets of a block's regions: each after the pivots starts on a 128-byte line."""
    n = {b: int((row_bits_h == b).sum()) for b in STQ_WIDTHS}
    b2, b3 = n[16] + n[8], n[16] + n[8] + n[6]
    o = {16: 0}
    # the 6- and 4-bit regions begin at the 4-row group of their first storage row: "lead" rows
    # of padding come before the first row
    o["lead6"] = b2 % 4 if n[6] else 0
    o["lead4"] = b3 % 4 if n[4] else 0
    o[8] = _up128(2 * D * n[16])
    o[6] = _up128(o[8] + D * n[8])
    o[4] = _up128(o[6] + 3 * D // 4 * (n[6] + o["lead6"]))
    o["rf"] = _up128(o[4] + D // 2 * (n[4] + o["lead4"]))
    o["cs"] = _up128(o["rf"] + 2 * (D - n[16]))
    o["end"] = o["cs"] + 2 * D
    return o


def stq_block_bytes(D: int, row_bits_h: np.ndarray) -> int:
    return (stq_regions(D, row_bits_h)["end"] + 255) // 256 * 256


def _nibbles(codes: np.ndarray) -> np.ndarray:
    """[rows, D] signed codes -> [rows, D/2] bytes of their low nibbles (column c at bits 4(c%2))."""
    u = codes.astype(np.int64) & 0xF
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def _tops(codes: np.ndarray) -> np.ndarray:
    u = (codes.astype(np.int64) >> 4) & 0x3
    return (u[:, 0::4] | (u[:, 1::4] << 2) | (u[:, 2::4] << 4) | (u[:, 3::4] << 6)).astype(np.uint8)


def stq_pack(row_bits, h, c, rf, cs) -> np.ndarray:
    """Logical (n, H, ...) -> uint8 slots [n, slot_bytes]."""
    n, H, D, _ = c.shape
    sizes = [stq_block_bytes(D, row_bits[hh]) for hh in range(H)]
    out = np.zeros((n, sum(sizes)), np.uint8)
    off = 0
    for hh in range(H):
        rb = row_bits[hh]
        order = stq_storage(rb)
        reg = stq_regions(D, rb)
        for u in range(n):
            blk = out[u, off:off + sizes[hh]]
            for b in STQ_WIDTHS:
                rows = order[rb[order] == b]
                if b == 16:
                    seg = np.ascontiguousarray(h[u, hh][rows]).view(np.uint8).ravel()
                elif b == 8:
                    seg = c[u, hh][rows].view(np.uint8).ravel()
                elif b == 6:
                    cc = c[u, hh][rows]
                    seg = np.concatenate([_nibbles(cc), _tops(cc)], axis=1).ravel()
                else:
                    seg = _nibbles(c[u, hh][rows]).ravel()
                at = reg[b] + (reg["lead6"] * 3 * D // 4 if b == 6 else (reg["lead4"] * D // 2 if b == 4 else 0))
                blk[at:at + seg.size] = seg
            ints = order[rb[order] != 16]
            seg = np.ascontiguousarray(rf[u, hh][ints]).view(np.uint8).ravel()
            blk[reg["rf"]:reg["rf"] + seg.size] = seg
            seg = np.ascontiguousarray(cs[u, hh]).view(np.uint8).ravel()
            blk[reg["cs"]:reg["cs"] + seg.size] = seg
        off += sizes[hh]
    return out


def _from_nibbles(b: np.ndarray) -> np.ndarray:
    lo = (b & 0xF).astype(np.int64)
    hi = (b >> 4).astype(np.int64)
    out = np.empty((b.shape[0], 2 * b.shape[1]), np.int64)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return out


def _from_tops(b: np.ndarray) -> np.ndarray:
    out = np.empty((b.shape[0], 4 * b.shape[1]), np.int64)
    for k in range(4):
        out[:, k::4] = (b >> (2 * k)) & 0x3
    return out


def stq_unpack(row_bits, slots: np.ndarray, D: int):
    """uint8 slots [n, slot_bytes] -> logical (h, c, rf, cs) in key order."""
    n = slots.shape[0]
    H = row_bits.shape[0]
    h = np.zeros((n, H, D, D), np.uint16)
    c = np.zeros((n, H, D, D), np.int8)
    rf = np.zeros((n, H, D), np.uint16)
    cs = np.zeros((n, H, D), np.uint16)
    off = 0
    for hh in range(H):
        rb = row_bits[hh]
        order = stq_storage(rb)
        reg = stq_regions(D, rb)
        for b in STQ_WIDTHS:
            o = off + reg[b] + (reg["lead6"] * 3 * D // 4 if b == 6 else (reg["lead4"] * D // 2 if b == 4 else 0))
            rows = order[rb[order] == b]
            m = len(rows)
            if b == 16:
                nb = 2 * D * m
                h[:, hh][:, rows, :] = slots[:, o:o + nb].copy().view(np.uint16).reshape(n, m, D)
            elif b == 8:
                nb = D * m
                c[:, hh][:, rows, :] = slots[:, o:o + nb].copy().view(np.int8).reshape(n, m, D)
            elif b == 6:
                nb = 3 * D // 4 * m
                blk = slots[:, o:o + nb].reshape(n * m, 3 * D // 4)
                v = _from_nibbles(blk[:, :D // 2]) | (_from_tops(blk[:, D // 2:]) << 4)
                v = np.where(v >= 32, v - 64, v)
                c[:, hh][:, rows, :] = v.reshape(n, m, D).astype(np.int8)
            else:
                nb = D // 2 * m
                v = _from_nibbles(slots[:, o:o + nb].reshape(n * m, D // 2))
                v = np.where(v >= 8, v - 16, v)
                c[:, hh][:, rows, :] = v.reshape(n, m, D).astype(np.int8)
        ints = order[rb[order] != 16]
        o = off + reg["rf"]
        rf[:, hh][:, ints] = slots[:, o:o + 2 * len(ints)].copy().view(np.uint16).reshape(n, len(ints))
        o = off + reg["cs"]
        cs[:, hh] = slots[:, o:o + 2 * D].copy().view(np.uint16).reshape(n, D)
        off += stq_block_bytes(D, rb)
    return h, c, rf, cs
