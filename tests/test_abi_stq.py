"""CPU-only checks of the STEPQuant-style entry points of the C-ABI library: storage accounting of
the block layout documented in damp.h, and rejection of bad arguments on the host (before any HIP
call) with the documented status codes."""
import ctypes

import numpy as np

import layout_ref
from quantized_delta_rule_gdn_amd import lib, synth


def _bytes(num_slots, H, d, bits):
    b = None if bits is None else np.ascontiguousarray(np.asarray(bits, np.uint8))
    ptr = None if b is None else b.ctypes.data_as(ctypes.c_void_p)
    return lib.load().stq_state_bytes(num_slots, H, d, ptr)


def test_block_accounting_of_the_nominal_map():
    bits, _ = synth.stq_map(np.random.default_rng(synth.STQ_SEED), 32, 128)
    counts = [(int((bits[h] == 16).sum()), int((bits[h] == 8).sum()), int((bits[h] == 6).sum()),
               int((bits[h] == 4).sum())) for h in range(32)]
    assert all(c == (2, 31, 63, 32) for c in counts)
    # FP16 pivots 2 x 256 | 31 x 128 | 63 x 96 | 32 x 64 | 126 row factors x 2 | 128 column scales x 2
    data = 512 + 3968 + 6048 + 2048 + 252 + 256
    assert data == 13084
    # each region on a 128-byte line, the 6-bit region from the row group of its first row (row
    # 33: one lead row of 96 bytes): 8-bit rows at 512, 6-bit at 4480 (first row at 4576), 4-bit
    # at 10624 (row 96 starts a group: no lead), row factors at 12672, column scales at 12924 ->
    # 12928, end 13184 (13312 with the 256-byte rounding, the same stride as without padding)
    reg = layout_ref.stq_regions(128, bits[0])
    assert (reg[8], reg[6], reg[4], reg["rf"], reg["cs"], reg["end"]) == (512, 4480, 10624, 12672, 12928, 13184)
    assert (reg["lead6"], reg["lead4"]) == (1, 0)
    assert layout_ref.stq_block_bytes(128, bits[0]) == 13312
    assert abs(8 * data / (128 * 128) - 6.389) < 5e-4
    assert _bytes(1, 32, 128, bits) == 32 * 13312         # each block rounded up to 256 bytes
    assert _bytes(7, 32, 128, bits) == 7 * 32 * 13312


def test_block_accounting_of_edge_maps():
    d = 64
    all16 = np.full((1, d), 16, np.uint8)
    all4 = np.full((1, d), 4, np.uint8)
    all8 = np.full((1, d), 8, np.uint8)
    # all pivots: no row factors; all 4-bit: d / 2 bytes a row, 2 d row-factor bytes
    assert _bytes(1, 1, d, all16) == -(-(2 * d * d + 2 * d) // 256) * 256
    assert _bytes(1, 1, d, all4) == -(-(d * d // 2 + 2 * d + 2 * d) // 256) * 256
    assert _bytes(1, 1, d, all8) == -(-(d * d + 2 * d + 2 * d) // 256) * 256
    mixed = np.array([[16, 6, 4, 8] * (d // 4)], np.uint8)   # any row order: rows are stored by kind
    # 16 rows of each kind at d = 64 (every region starts a row group): pivots 2048 @0, 8-bit 1024
    # @2048, 6-bit 768 @3072, 4-bit 512 @3840, 48 row factors 96 @4352, column scales 128 @4480
    # (4448 rounded to a line): end 4608
    assert _bytes(3, 1, d, mixed) == 3 * 4608
    odd = np.array([[16] * 3 + [8] * 5 + [6] * 7 + [4] * (d - 15)], np.uint8)
    # pivots 384 @0, 8-bit 320 @384; 6-bit from row 8 (no lead) 7 x 48 = 336 @768 (704 rounded);
    # 4-bit from row 15: lead 3 rows, (3 + 49) x 32 = 1664 @1152 (1104 rounded); 61 row factors
    # 122 @2816; column scales 128 @2944 (2938 rounded): end 3072
    reg = layout_ref.stq_regions(d, odd[0])
    assert (reg[6], reg[4], reg["rf"], reg["cs"], reg["end"], reg["lead6"], reg["lead4"]) == (768, 1152, 2816, 2944, 3072, 0, 3)
    assert _bytes(2, 1, d, odd) == 2 * 3072


def test_invalid_layouts_report_zero_bytes():
    good = np.full((2, 128), 8, np.uint8)
    bad = good.copy()
    bad[1, 5] = 5
    assert _bytes(4, 2, 128, good) > 0
    assert _bytes(4, 2, 128, bad) == 0             # a width outside {16, 8, 6, 4}
    assert _bytes(4, 2, 128, None) == 0            # NULL map
    assert _bytes(0, 2, 128, good) == 0            # no slots
    assert _bytes(4, 0, 128, good) == 0            # no heads
    assert _bytes(4, 2, 96, np.full((2, 96), 8, np.uint8)) == 0     # d outside {64, 128}


def _alloc(num_slots, H, d, bits, impact, pool, pool_bytes, out=True):
    L = lib.load()
    b = None if bits is None else np.ascontiguousarray(np.asarray(bits, np.uint8))
    w = None if impact is None else np.ascontiguousarray(np.asarray(impact, np.float32))
    h = ctypes.c_void_p()
    st = L.stq_state_alloc(num_slots, H, d, None if b is None else b.ctypes.data_as(ctypes.c_void_p),
                           None if w is None else w.ctypes.data_as(ctypes.c_void_p),
                           None if pool is None else ctypes.c_void_p(pool), pool_bytes,
                           ctypes.byref(h) if out else None)
    return st, h


def test_alloc_rejects_bad_arguments_on_host():
    H, d = 2, 64
    bits = np.full((H, d), 6, np.uint8)
    bits[:, :3] = 16
    w = np.ones((H, d), np.float32)
    need = _bytes(4, H, d, bits)
    fake = 0x100000  # never dereferenced: every case fails validation first
    neg, nan, inf = w.copy(), w.copy(), w.copy()
    neg[1, 7] = -1.0
    nan[0, 0] = np.nan
    inf[0, 3] = np.inf
    bad_bits = bits.copy()
    bad_bits[0, 9] = 7
    cases = [
        ((4, H, d, bits, w, fake, need), {"out": False}, lib.DAMP_ERR_INVALID_ARGUMENT, "out is NULL"),
        ((0, H, d, bits, w, fake, need), {}, lib.DAMP_ERR_INVALID_ARGUMENT, "positive"),
        ((4, H, 96, np.full((H, 96), 8, np.uint8), np.ones((H, 96), np.float32), fake, 1 << 30), {},
         lib.DAMP_ERR_UNSUPPORTED, "d in {64, 128}"),
        ((4, H, d, None, w, fake, need), {}, lib.DAMP_ERR_INVALID_ARGUMENT, "row_bits is NULL"),
        ((4, H, d, bad_bits, w, fake, need), {}, lib.DAMP_ERR_INVALID_ARGUMENT, "is not 16, 8, 6 or 4"),
        ((4, H, d, bits, None, fake, need), {}, lib.DAMP_ERR_INVALID_ARGUMENT, "impact is NULL"),
        ((4, H, d, bits, neg, fake, need), {}, lib.DAMP_ERR_INVALID_ARGUMENT, "finite and >= 0"),
        ((4, H, d, bits, nan, fake, need), {}, lib.DAMP_ERR_INVALID_ARGUMENT, "finite and >= 0"),
        ((4, H, d, bits, inf, fake, need), {}, lib.DAMP_ERR_INVALID_ARGUMENT, "finite and >= 0"),
        ((4, H, d, bits, w, None, need), {}, lib.DAMP_ERR_INVALID_ARGUMENT, "pool is NULL"),
        ((4, H, d, bits, w, fake + 64, need), {}, lib.DAMP_ERR_INVALID_ARGUMENT, "aligned"),
        ((4, H, d, bits, w, fake, need - 1), {}, lib.DAMP_ERR_INVALID_ARGUMENT, "needed"),
    ]
    for args, kw, want, msg in cases:
        st, h = _alloc(*args, **kw)
        assert st == want, (st, want, lib.last_error())
        assert msg in lib.last_error(), lib.last_error()
        assert not h.value


def test_entry_points_reject_a_null_handle():
    L = lib.load()
    p = ctypes.c_void_p(0x200000)
    assert L.stq_state_free(None) == lib.DAMP_OK
    assert L.stq_state_head_info(None, None, None) == lib.DAMP_ERR_INVALID_ARGUMENT
    assert L.stq_state_quantize(None, p, p, 1, None) == lib.DAMP_ERR_INVALID_ARGUMENT
    assert L.stq_state_dequantize(None, p, p, 1, None) == lib.DAMP_ERR_INVALID_ARGUMENT
    st = L.stq_decode_step(None, None, p, 1, p, p, p, lib.DAMP_BF16, p, 0, p, p, None)
    assert st == lib.DAMP_ERR_INVALID_ARGUMENT
    assert "state is NULL" in lib.last_error()


def test_block_bytes_of_random_maps_match_the_layout_reference():
    """The library's block size (stq_state_bytes) equals the layout written from the header's
    description (every region on a 128-byte line, the 6- and 4-bit rows from the 4-row group of
    their first row, the block rounded to 256 bytes) for random precision maps."""
    rng = np.random.default_rng(2718)
    for _ in range(60):
        d = int(rng.choice([64, 128]))
        H = int(rng.integers(1, 4))
        bits = rng.choice(np.array([16, 8, 6, 4], np.uint8), size=(H, d), p=rng.dirichlet(np.ones(4)))
        want = sum(layout_ref.stq_block_bytes(d, bits[h]) for h in range(H))
        assert _bytes(3, H, d, bits) == 3 * want
