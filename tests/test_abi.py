"""CPU-only checks of the C-ABI library: it loads without a GPU, exports every entry point the
header declares, reports the documented storage accounting, and rejects bad arguments on the
host (before any HIP call) with the documented status codes."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

from quantized_delta_rule_gdn_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "damp.h")
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_0-9]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_library_loads_and_exports_every_declared_symbol():
    L = lib.load()
    declared = _header_functions()
    assert len(declared) >= 14
    assert set(declared) == set(lib.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    assert L.damp_abi_version() == (1 << 16) | 3


def test_block_accounting_d128():
    assert lib.block_data_bytes(1, 1, 128, 24) == 6144 + 13312 + 416 == 19872
    assert lib.block_bytes(1, 1, 128, 24) == 19968
    assert lib.block_data_bytes(1, 1, 128, 0) == 16384 + 512       # uniform INT8 + row scales
    assert lib.block_data_bytes(1, 1, 128, 128) == 32768            # all FP16 = 16 bits/value
    assert lib.state_bytes(4096, 32, 128, 24) == 4096 * 32 * 19968
    bits = 8 * lib.block_data_bytes(1, 1, 128, 24) / 128 ** 2
    assert abs(bits - 9.703125) < 1e-12
    assert abs((1 - bits / 32) - 0.6967773) < 1e-6


def test_bits_accounting_matches_page_identities():
    """bits/value -> compression and storage reduction, as printed on the pages."""
    g = json.load(open(os.path.join(GOLD, "page_identities.json")))
    for case in g["cases"]:
        if "reduction_pct" in case:
            assert round(100 * (1 - case["bits"] / 32), 1) == case["reduction_pct"]
        if "compression" in case:
            # both numbers are printed rounded (bits to 3 decimals, compression to 2): the
            # identity compression = 32 / bits must hold for some value in both intervals
            b, c = case["bits"], case["compression"]
            lo, hi = 32 / (c + 0.005), 32 / (c - 0.005)
            assert max(lo, b - 0.0005) <= min(hi, b + 0.0005)
            assert abs(32 / b - c) < 0.006
    # with fp32 row scales, r FP16 rows per 128x128 head give 9.9 bits/value at r ~ 27
    r_for_9_9 = min(range(129), key=lambda r: abs(8 * lib.block_data_bytes(1, 1, 128, r) / 128 ** 2 - 9.9))
    assert r_for_9_9 == 27


@pytest.mark.parametrize("d,r", [(0, 0), (128, 129), (128, -1), (100, 4), (256, 8), (48, 0)])
def test_invalid_layouts_report_zero_bytes(d, r):
    assert lib.state_bytes(4, 2, d, r) == 0


def _alloc(layout, rows, pool, nbytes):
    L = lib.load()
    h = ctypes.c_void_p()
    rows_p = rows.ctypes.data_as(ctypes.c_void_p) if rows is not None else None
    st = L.damp_state_alloc(ctypes.byref(layout) if layout is not None else None, rows_p, pool,
                            nbytes, ctypes.byref(h))
    return st, h


def test_alloc_rejects_bad_arguments_on_host():
    L = lib.load()
    good_rows = np.array([[0, 5], [1, 7]], np.int32)
    lay = lib.layout(4, 2, 16, 2)
    need = lib.state_bytes(4, 2, 16, 2)
    fake_pool = 0x100000  # never dereferenced: every case fails validation first
    cases = [
        (None, good_rows, fake_pool, need, lib.DAMP_ERR_INVALID_ARGUMENT, "layout is NULL"),
        (lib.layout(4, 2, 100, 2), good_rows, fake_pool, 1 << 30, lib.DAMP_ERR_UNSUPPORTED, "supported"),
        (lib.layout(4, 2, 16, 17), good_rows, fake_pool, need, lib.DAMP_ERR_INVALID_ARGUMENT, "num_fp16_rows"),
        (lay, None, fake_pool, need, lib.DAMP_ERR_INVALID_ARGUMENT, "fp16_rows is NULL"),
        (lay, good_rows, None, need, lib.DAMP_ERR_INVALID_ARGUMENT, "pool is NULL"),
        (lay, good_rows, fake_pool + 16, need, lib.DAMP_ERR_INVALID_ARGUMENT, "aligned"),
        (lay, good_rows, fake_pool, need - 1, lib.DAMP_ERR_INVALID_ARGUMENT, "needed"),
        (lay, np.array([[5, 0], [1, 7]], np.int32), fake_pool, need, lib.DAMP_ERR_INVALID_ARGUMENT, "ascending"),
        (lay, np.array([[0, 16], [1, 7]], np.int32), fake_pool, need, lib.DAMP_ERR_INVALID_ARGUMENT, "outside"),
        (lay, np.array([[3, 3], [1, 7]], np.int32), fake_pool, need, lib.DAMP_ERR_INVALID_ARGUMENT, "ascending"),
    ]
    for layout, rows, pool, nbytes, want, msg in cases:
        st, h = _alloc(layout, rows, pool, nbytes)
        assert st == want, (st, want, lib.last_error())
        assert msg in lib.last_error()
        assert not h.value


def test_step_entry_points_reject_bad_arguments_on_host():
    L = lib.load()
    fp = ctypes.c_void_p(0x100000)
    ok = ctypes.c_void_p(0x200000)
    # unsupported size
    st = L.fp32_decode_step(fp, 4, 2, 48, 48, ok, 1, ok, ok, ok, lib.DAMP_F32, ok, 0, ok, ok, None)
    assert st == lib.DAMP_ERR_UNSUPPORTED
    st = L.uniform_int8_decode_step(fp, fp, 4, 2, 128, 64, ok, 1, ok, ok, ok, lib.DAMP_F32, ok, 0,
                                    ok, ok, None)
    assert st == lib.DAMP_ERR_UNSUPPORTED
    # negative batch, bad enums, null pointers, misaligned output
    assert L.fp32_decode_step(fp, 4, 2, 16, 16, ok, -1, ok, ok, ok, 0, ok, 0, ok, ok, None) == \
        lib.DAMP_ERR_INVALID_ARGUMENT
    assert L.fp32_decode_step(fp, 4, 2, 16, 16, ok, 1, ok, ok, ok, 7, ok, 0, ok, ok, None) == \
        lib.DAMP_ERR_INVALID_ARGUMENT
    assert L.fp32_decode_step(fp, 4, 2, 16, 16, ok, 1, ok, ok, ok, 0, ok, 3, ok, ok, None) == \
        lib.DAMP_ERR_INVALID_ARGUMENT
    assert L.fp32_decode_step(fp, 4, 2, 16, 16, ok, 1, None, ok, ok, 0, ok, 0, ok, ok, None) == \
        lib.DAMP_ERR_INVALID_ARGUMENT
    assert L.fp32_decode_step(fp, 4, 2, 16, 16, ok, 1, ok, ok, ok, 0, ok, 0, ok,
                              ctypes.c_void_p(0x200004), None) == lib.DAMP_ERR_INVALID_ARGUMENT
    assert "16-byte" in lib.last_error()
    assert L.fp32_decode_step(None, 4, 2, 16, 16, ok, 1, ok, ok, ok, 0, ok, 0, ok, ok, None) == \
        lib.DAMP_ERR_INVALID_ARGUMENT
    assert L.fp32_decode_step(fp, 0, 2, 16, 16, ok, 1, ok, ok, ok, 0, ok, 0, ok, ok, None) == \
        lib.DAMP_ERR_INVALID_ARGUMENT
    # B == 0 is a no-op that needs no GPU
    assert L.fp32_decode_step(fp, 4, 2, 16, 16, None, 0, None, None, None, 0, None, 0, None, None,
                              None) == lib.DAMP_OK
    assert L.uniform_int8_decode_step(None, None, 4, 2, 16, 16, None, 0, None, None, None, 0, None,
                                      0, None, None, None) == lib.DAMP_OK
    # NULL handles
    assert L.damp_decode_step(None, ok, 1, ok, ok, ok, 0, ok, 0, ok, ok, None) == \
        lib.DAMP_ERR_INVALID_ARGUMENT
    assert L.damp_state_quantize(None, ok, ok, 1, None) == lib.DAMP_ERR_INVALID_ARGUMENT
    assert L.damp_state_dequantize(None, ok, ok, 1, None) == lib.DAMP_ERR_INVALID_ARGUMENT
    assert L.damp_state_free(None) == lib.DAMP_OK
    assert L.uniform_int8_quantize(fp, fp, 4, 2, 16, 16, ok, ok, -2, None) == \
        lib.DAMP_ERR_INVALID_ARGUMENT


# ---- per-head layout and calibration entry points (host logic only) -------------------------
def _vp(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def test_per_head_bytes():
    L = lib.load()
    lay = lib.layout(5, 32, 128, 0)
    # every head at r = 24 is the uniform layout
    r = np.full(32, 24, np.int32)
    assert L.damp_state_bytes_per_head(ctypes.byref(lay), _vp(r)) == lib.state_bytes(5, 32, 128, 24)
    # mixed r: each head's block rounds up to 256 bytes on its own
    r = np.array([0, 8, 24, 32, 128] + [16] * 27, np.int32)
    blk = lambda x: (2 * x * 128 + (128 - x) * 128 + 4 * (128 - x) + 255) // 256 * 256
    assert L.damp_state_bytes_per_head(ctypes.byref(lay), _vp(r)) == 5 * sum(blk(int(x)) for x in r)
    # invalid r
    r[3] = 129
    assert L.damp_state_bytes_per_head(ctypes.byref(lay), _vp(r)) == 0
    assert L.damp_state_bytes_per_head(ctypes.byref(lay), None) == 0


def test_alloc_per_head_rejects_bad_arguments_on_host():
    L = lib.load()
    H, d = 2, 16
    lay = lib.layout(4, H, d, 0)
    r = np.array([2, 0], np.int32)
    good = np.array([[3, 9] + [i for i in range(d) if i not in (3, 9)], list(range(d))], np.int32)
    need = L.damp_state_bytes_per_head(ctypes.byref(lay), _vp(r))
    fake_pool = 0x100000

    def alloc(lay_, r_, m_, pool, nbytes):
        h = ctypes.c_void_p()
        st = L.damp_state_alloc_per_head(ctypes.byref(lay_) if lay_ is not None else None, _vp(r_),
                                         _vp(m_), pool, nbytes, ctypes.byref(h))
        return st, h

    bad_order = good.copy()
    bad_order[0, :2] = [9, 3]
    dup = good.copy()
    dup[1, 5] = 4
    out_of_range = good.copy()
    out_of_range[1, 0] = 16
    cases = [
        (lay, np.array([2, 17], np.int32), good, fake_pool, need, "r_per_head[1]"),
        (lay, None, good, fake_pool, need, "r_per_head is NULL"),
        (lay, r, None, fake_pool, need, "row_map is NULL"),
        (lay, r, good, None, need, "pool is NULL"),
        (lay, r, good, fake_pool + 64, need, "aligned"),
        (lay, r, good, fake_pool, need - 1, "needed"),
        (lay, r, bad_order, fake_pool, need, "ascending"),
        (lay, r, dup, fake_pool, need, "repeats"),
        (lay, r, out_of_range, fake_pool, need, "outside"),
    ]
    for lay_, r_, m_, pool, nbytes, msg in cases:
        st, h = alloc(lay_, r_, m_, pool, nbytes)
        assert st == lib.DAMP_ERR_INVALID_ARGUMENT, (msg, st, lib.last_error())
        assert msg in lib.last_error(), (msg, lib.last_error())
        assert not h.value
    st, _ = alloc(lib.layout(4, H, 48, 0), np.zeros(H, np.int32), good, fake_pool, need)
    assert st == lib.DAMP_ERR_UNSUPPORTED


def test_budget_rows_matches_the_oracle():
    import oracle
    for d in (16, 32, 64, 128):
        for H in (1, 3, 32):
            for bits in (8.0, 8.25, 8.3, 9.0, 9.703125, 9.9, 10.5, 12.0, 16.0, 17.0):
                for g in (1, 4, 8):
                    for r_max in (0, d // 4, d):
                        assert lib.budget_rows(d, H, bits, g, r_max) == oracle.budget_rows(d, H, bits, g, r_max)
    assert lib.budget_rows(128, 32, 9.9) == 872
    assert lib.budget_rows(4, 32, 9.9) == -1       # d <= 4
    assert lib.budget_rows(128, 32, 9.9, g=0) == -1


def test_calibration_entry_points_reject_bad_arguments_on_host():
    L = lib.load()
    p = ctypes.c_void_p(0x100000)
    E = lib.DAMP_ERR_INVALID_ARGUMENT
    assert L.damp_risk_scores(p, 0, 2, 16, p, p, p, None) == E
    assert L.damp_risk_scores(p, 2, 2, 48, p, p, p, None) == lib.DAMP_ERR_UNSUPPORTED
    assert L.damp_risk_scores(None, 2, 2, 16, p, p, p, None) == E
    assert L.damp_risk_scores(ctypes.c_void_p(0x100004), 2, 2, 16, p, p, p, None) == E
    assert L.damp_allocate_rows(p, 2, 16, 6, 4, 16, p, p, None) == E        # R % g
    assert "multiple" in lib.last_error()
    assert L.damp_allocate_rows(p, 2, 16, 8, 0, 16, p, p, None) == E        # g
    assert L.damp_allocate_rows(p, 2, 16, 8, 1, 17, p, p, None) == E        # r_max
    assert L.damp_allocate_rows(p, 2, 256, 8, 1, 16, p, p, None) == lib.DAMP_ERR_UNSUPPORTED
    assert L.damp_allocate_rows(p, 128, 128, 8, 1, 128, p, p, None) == lib.DAMP_ERR_UNSUPPORTED
    assert L.damp_allocate_rows(p, 64, 128, 8, 1, 128, p, p, None) == lib.DAMP_ERR_UNSUPPORTED
    assert "groups" in lib.last_error()
    assert L.damp_allocate_rows(None, 2, 16, 8, 1, 16, p, p, None) == E


def test_order_entry_points_reject_bad_arguments_on_host():
    L = lib.load()
    a, o = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    bad = lib.DAMP_ERR_INVALID_ARGUMENT
    assert L.damp_batch_order(a, -1, 16, o, None) == bad
    assert L.damp_batch_order(a, 4, 0, o, None) == bad and "num_slots" in lib.last_error()
    assert L.damp_batch_order(None, 4, 16, o, None) == bad
    assert L.damp_batch_order(a, 4, 16, None, None) == bad
    assert L.damp_batch_order(a, 4, 16, ctypes.c_void_p(0x200002), None) == bad
    assert "aligned" in lib.last_error()
    # order overlapping slot_idx (both ways), and adjacent buffers that do not overlap
    assert L.damp_batch_order(a, 4, 16, ctypes.c_void_p(0x10000c), None) == bad
    assert "overlaps" in lib.last_error()
    assert L.damp_batch_order(ctypes.c_void_p(0x10000c), 4, 16, a, None) == bad
    # B == 0 is a no-op that needs no GPU
    assert L.damp_batch_order(None, 0, 16, None, None) == lib.DAMP_OK
    assert L.damp_decode_step_ordered(None, a, o, 1, a, a, a, 0, a, 0, a, a, None) == bad
    assert "state is NULL" in lib.last_error()
    assert L.damp_decode_step_fused_ordered(None, a, o, 1, a, a, a, 0, a, 0, a, a, None) == bad
    assert L.damp_window_step_ordered(None, a, 4, a, o, 1, a, a, a, 0, a, 0, a, a, None) == bad


def test_sorted_step_rejects_bad_arguments_on_host():
    """damp_decode_step_sorted checks the batch against its library-held buffer before anything
    else, then the arguments as damp_decode_step does; none of it needs a GPU."""
    L = lib.load()
    a = ctypes.c_void_p(0x100000)
    assert L.damp_decode_step_sorted(None, a, lib.SORTED_MAX_B + 1, a, a, a, 0, a, 0, a, a,
                                     None) == lib.DAMP_ERR_UNSUPPORTED
    assert "order buffer" in lib.last_error()
    assert L.damp_decode_step_sorted(None, a, lib.SORTED_MAX_B, a, a, a, 0, a, 0, a, a,
                                     None) == lib.DAMP_ERR_INVALID_ARGUMENT
    assert "state is NULL" in lib.last_error()


def test_header_is_plain_c99_and_the_library_links_from_c(tmp_path):
    """tests/c/abi_from_c.c, built with gcc -std=c99 -pedantic -Werror against include/damp.h and
    linked with libdamp.so, prints the host-side results of a few calls; each must equal the
    same call made through the Python binding (no GPU involved)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not on PATH")
    libdir = os.path.dirname(lib.LIB_PATH)
    exe = os.path.join(os.path.dirname(__file__), "c", "abi_from_c")   # built with the library
    if not os.path.exists(exe):
        exe = str(tmp_path / "abi_from_c")
        src = os.path.join(os.path.dirname(__file__), "c", "abi_from_c.c")
        subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I",
                        os.path.join(ROOT, "include"), src, "-L", libdir, "-ldamp",
                        f"-Wl,-rpath,{libdir}", "-o", exe], check=True, capture_output=True, text=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.splitlines()
    got = {ln.split(" ", 1)[0]: ln.split(" ", 1)[1] for ln in out}

    L = lib.load()
    big, small, bad = lib.layout(4096, 32, 128, 24), lib.layout(64, 2, 16, 2), lib.layout(0, 32, 128, 24)
    r_per_head = np.array([2, 5], np.int32)
    bits = np.array([16 if i % 16 < 2 else (8 if i % 16 < 6 else (6 if i % 16 < 11 else 4))
                     for i in range(32)], np.uint8)
    st = ctypes.c_void_p()
    rc_alloc = L.damp_state_alloc(ctypes.byref(bad), None, None, 0, ctypes.byref(st))
    err_alloc = L.damp_last_error().decode()
    rc_step = L.damp_decode_step(None, None, 1, None, None, None, 1, None, 0, None, None, None)
    err_step = L.damp_last_error().decode()
    want = {
        "block_bytes": str(L.damp_block_bytes(ctypes.byref(big))),
        "block_data_bytes": str(L.damp_block_data_bytes(ctypes.byref(big))),
        "state_bytes": str(L.damp_state_bytes(ctypes.byref(big))),
        "window_bytes_8": str(L.damp_window_bytes(ctypes.byref(big), 8)),
        "window_bytes_9": str(L.damp_window_bytes(ctypes.byref(big), 9)),
        "state_bytes_per_head": str(L.damp_state_bytes_per_head(
            ctypes.byref(small), r_per_head.ctypes.data_as(ctypes.c_void_p))),
        "stq_state_bytes": str(L.stq_state_bytes(64, 2, 16, bits.ctypes.data_as(ctypes.c_void_p))),
        "alloc_bad": f"{rc_alloc} {err_alloc}",
        "step_null": f"{rc_step} {err_step}",
    }
    assert got == want
    assert want["window_bytes_9"] == "0" and rc_alloc == lib.DAMP_ERR_INVALID_ARGUMENT
