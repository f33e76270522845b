"""CPU checks of bench.py's host logic: the algorithmic bytes it divides by, the window average,
the traffic file's source hash, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_per_update():
    # block 2 x 19,872 + q, k, v bf16 (768) + alpha (4) + beta (4) + readout (512) + slot index (4)
    assert bench.alg_bytes_per_update("damp", 128, 24, False) == 2 * 19872 + 1292 == 41036
    assert bench.alg_bytes_per_update("damp", 128, 24, True) == 41036 + 508 == 41544   # KDA gate
    assert bench.alg_bytes_per_update("int8", 128) == 2 * 16896 + 1292 == 35084
    assert bench.alg_bytes_per_update("fp32", 128) == 2 * 65536 + 1292 == 132364
    assert bench.alg_bytes_per_update("damp", 128, 24, False, qkv_bytes=4) == 41036 + 768


def test_window_bytes_reduce_to_the_per_token_step():
    # a window of one token reads and writes the block once per token, plus the empty header
    assert abs(bench.alg_bytes_window(1) - (41036 + 4)) < 1e-9
    assert abs(bench.alg_bytes_window(1, per_key=True) - (41544 + 4)) < 1e-9
    for pk in (False, True):
        w4, w8 = bench.alg_bytes_window(4, per_key=pk), bench.alg_bytes_window(8, per_key=pk)
        assert w4 < 41036 and w8 < 41036      # the block is written once per window
    # per-row gates: every buffered key is rewritten decayed each token, so the bytes grow with W
    assert bench.alg_bytes_window(8, per_key=True) > bench.alg_bytes_window(4, per_key=True)
    # one gate per unit, W = 2, bf16 inputs, by hand: token 0 reads the block and the count
    # (19,872 + 4) and writes the header words, c[0], its key as bf16 and its delta
    # (16 + 4 + 256 + 512); token 1 reads the block, the count, a, the key-format word, c[0], one
    # bf16 key and one delta (19,872 + 4 + 4 + 4 + 4 + 256 + 512) and writes the block; each token
    # also moves its 1,292 vector bytes
    t0 = 19872 + 4 + 16 + 4 + 256 + 512 + 1292
    t1 = 19872 + 4 + 4 + 4 + 4 + 256 + 512 + 19872 + 1292
    assert abs(bench.alg_bytes_window(2) - (t0 + t1) / 2) < 1e-9
    # fp32 inputs keep fp32 keys (512 bytes each) and fp32 q, k, v (1,536 bytes)
    f0 = 19872 + 4 + 16 + 4 + 512 + 512 + 2060
    f1 = 19872 + 4 + 4 + 4 + 4 + 512 + 512 + 19872 + 2060
    assert abs(bench.alg_bytes_window(2, qkv_bytes=4) - (f0 + f1) / 2) < 1e-9


def test_traffic_is_reported_only_for_the_profiled_source():
    t = bench.measured_traffic()
    if t is None:
        pytest.skip("the step's source changed since its HBM counters were taken (traffic: null)")
    # counter bytes of one pool4096 launch (32,768 updates) within 1% of the algorithmic bytes
    assert abs(t / (32768 * 41036) - 1) < 0.01


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_order_policy():
    # auto: the 32,768-unit pool4096 batch is ordered, the 8,192-unit kda256 and 2,048-unit gdn64
    # batches are not; the per-window step stays in batch order; on / off force it; never for
    # the STEPQuant-style step
    assert bench.order_enabled("auto", 1024 * 32)
    assert not bench.order_enabled("auto", 256 * 32)
    assert not bench.order_enabled("auto", 64 * 32)
    assert not bench.order_enabled("auto", 1024 * 32, window=4)
    assert bench.order_enabled("on", 64 * 32) and bench.order_enabled("on", 1024 * 32, window=4)
    assert not bench.order_enabled("off", 1024 * 32)
    assert not bench.order_enabled("on", 1024 * 32, stq=True)
