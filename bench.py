#!/usr/bin/env python3
"""Throughput of the DAMP decode step on one MI355X.

Workload (default, --workload pool4096): the serving pool -- 4,096 request slots x 32 GDN heads
of 128 x 128 states in the DAMP layout (24 FP16 key rows per head, INT8 + fp32 row scale for the
other 104), of which 1,024 random slots are active; each step updates 1,024 x 32 = 32,768
(slot, head) states with bf16 q, k, v and fp32 alpha, beta, cycling through 4 pre-made input
sets. The touched state (654 MB read + written per step) is larger than the 256 MB Infinity
Cache. Other workloads (--workload gdn64 | kda256 | drift) have 64 or 256 contiguous slots whose
state fits in that cache: gdn64 and kda256 rotate over enough copies of the pool that each launch
finds its state in HBM (cold), drift reruns the same 64 slots (warm, labelled so).

A step = one pass of the decode step over the batch (reconstruct, decay, delta update, readout,
requantize). On pool4096 a step is two launches: damp_batch_order lists the batch by ascending
slot, then damp_decode_step_ordered takes the units in that order (the results are those of
damp_decode_step bit for bit; nearby blocks stream faster together). Smaller batches run
damp_decode_step alone (--order). Timing: HIP events recorded on the stream the kernels are
launched on, around exactly --steps steps after --warmup untimed ones, with device
synchronisation on both sides.

Prints ONE JSON line. value = (slot, head) state updates per second over whole steps (both
launches on pool4096). roofline describes the dominant kernel, the step kernel: the algorithmic
bytes of one update (state block read + written, q/k/v, alpha, beta, readout, slot index) times
the updates per launch, divided by the kernel's average launch duration -- on pool4096 timed in
a run of its own (--steps launches of the ordered step with the orders computed beforehand), so
that it is the figure a kernel trace gives for that kernel; kernel_us is that duration.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD published peak
# Batches of at least this many (slot, head) units run the step in ascending slot order under
# --order auto. The step holds at most 2,048 units at once (8 per CU); a batch that spans many
# such waves gains from streaming nearby blocks together more than the ordering launch costs
# (about 2-5 us), a batch that is resident at once does not.
ORDER_MIN_UNITS = 16384
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "damp_step_pool4096_hbm_traffic.txt")
# the DAMP step's kernel source: its building blocks and its kernels
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_delta_rule_gdn_amd", "csrc", f)
                  for f in ("step_common.h", "step_kernels.hip")]


def measured_traffic():
    """HBM bytes per launch of the DAMP step from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, each calibrated on a copy of known size), or None when the kernel
    source has changed since the counters were taken."""
    import hashlib
    try:
        kv = {}
        for line in open(TRAFFIC_FILE):
            line = line.strip()
            if line and not line.startswith("#") and "=" in line:
                key, val = (x.strip() for x in line.split("=", 1))
                kv[key] = val
        sha = hashlib.sha256(b"".join(open(f, "rb").read() for f in KERNEL_SOURCES)).hexdigest()
    except OSError:
        return None
    if kv.get("kernel_source_sha256") != sha:
        return None
    return int(kv["traffic_bytes_per_launch"])


def order_enabled(order: str, units: int, window: int = 0, stq: bool = False) -> bool:
    """Whether the timed DAMP steps list their batch by slot first (damp_batch_order, then the
    ordered step). "on" / "off" force it; "auto" orders batches of at least ORDER_MIN_UNITS units
    and leaves the per-window step in batch order: measured on pool4096, the order gains nothing
    there (W = 4: 188.5 us ordered against 187.4 us; W = 8: 206.9 against 205.7 us). The
    STEPQuant-style step has no ordered entry point."""
    if stq:
        return False
    if order == "on":
        return True
    return order == "auto" and units >= ORDER_MIN_UNITS and not window


def alg_bytes_window(W: int, d: int = 128, r: int = 24, per_key: bool = False, qkv_bytes: int = 2) -> float:
    """Bytes per (slot, head) update of the windowed step, averaged over the W tokens of a
    window: every token reads the stored block and its buffered terms (a key and a delta each);
    a token that does not end the window appends its key and delta, the last one writes the
    block instead. Deltas are fp32 (4 d bytes). The decay: with a gate per key row (KDA) the row
    gains (4 d bytes) and every buffered key (fp32) are read and written back decayed; with one
    gate per unit (GDN) the decay is one number for the window and one per buffered key, in the
    buffer's header words, and the keys stay as given: 2 d bytes each from bf16 inputs."""
    block = 2 * r * d + (d - r) * d + 4 * (d - r)
    vecs = 3 * qkv_bytes * d + (4 * d if per_key else 4) + 4 + 4 * d + 4
    key = 4 * d if per_key or qkv_bytes != 2 else 2 * d
    total = 0
    for t in range(W):
        last = t == W - 1
        if per_key:
            rd = block + 4 + (4 * d if t else 0) + t * 2 * 4 * d
            wr = block if last else 12 + 4 * d + t * 4 * d + 2 * 4 * d
        else:
            rd = block + 4 + (8 + 4 * t if t else 0) + t * (key + 4 * d)
            wr = block if last else 16 + 4 * (t + 1) + key + 4 * d
        total += rd + wr + vecs
    return total / W


def alg_bytes_per_update(fmt: str, d: int = 128, r: int = 24, per_key: bool = False,
                         qkv_bytes: int = 2) -> int:
    """Bytes one (slot, head) update must move: the state block in and out, q/k/v, the gate
    (scalar or per key), beta, the fp32 readout and the 4-byte slot index (shared by the
    heads of a slot: counted per unit as 4/H, rounded into the total below)."""
    if fmt == "damp":
        state = 2 * r * d + (d - r) * d + 4 * (d - r)
    elif fmt == "int8":
        state = d * d + 4 * d
    else:
        state = 4 * d * d
    vecs = 3 * qkv_bytes * d + (4 * d if per_key else 4) + 4 + 4 * d + 4
    return 2 * state + vecs


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-baselines", action="store_true",
                   help="skip the in-library fp32 / uniform-INT8 comparison runs")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--only", choices=["damp", "fp32", "int8"], default=None,
                   help="time only this format (for profiling)")
    p.add_argument("--workload", choices=["pool4096", "gdn64", "kda256", "drift"],
                   default="pool4096")
    p.add_argument("--budget-bits", type=float, default=None, metavar="BITS",
                   help="DAMP with per-head FP16 rows: calibrate on the device (risk scores and "
                        "allocation) and spend BITS data bits per state value (the pages: 9.9)")
    p.add_argument("--budget-group", type=int, default=8,
                   help="FP16 rows are handed out per head in groups of this many")
    p.add_argument("--budget-rmax", type=int, default=32, help="at most this many FP16 rows per head")
    p.add_argument("--fused-prestep", action="store_true",
                   help="DAMP step with the pre-step fused (raw q/k projections, gate and beta "
                        "logits); also times the same pre-step as separate torch kernels + step")
    p.add_argument("--window", type=int, default=0, metavar="W",
                   help="DAMP with per-window requantization: windows of W tokens (1..8); the "
                        "timed launches run whole windows, so the figures average over a window")
    p.add_argument("--stq", action="store_true",
                   help="the STEPQuant-style state instead of DAMP (FP16 pivots, 8/6/4-bit rows at "
                        "a nominal 6-bit map, FP16 row factors and column scales refitted each step)")
    p.add_argument("--order", choices=["auto", "on", "off"], default="auto",
                   help="DAMP steps (plain, per-head layout, fused pre-step, per-window) with the "
                        "batch taken in ascending slot order: damp_batch_order runs inside every "
                        "timed step, then the ordered entry point; auto = on for batches of at "
                        f"least {ORDER_MIN_UNITS} units, except the per-window step")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="instead of the step, run a plain device copy of MIB MiB --steps times "
                        "(the reference kernel of known size for HBM byte counters)")
    return p.parse_args()


def copy_calibration(mib: int, steps: int) -> None:
    import torch
    dev = torch.device("cuda", 0)
    src = torch.ones(mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.zeros_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": mib << 20, "bytes_written": mib << 20,
                      "launches": steps}), flush=True)


def fill_states(torch, fn, slots_dev, H, d, dev, chunk=128, seed=1003):
    """Active slots get S ~ N(0, 0.1) from a seeded device generator, written by ``fn``
    (S_chunk [c, H, d, d], slot_idx_chunk) in chunks."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    for i in range(0, slots_dev.numel(), chunk):
        sl = slots_dev[i:i + chunk]
        S = torch.randn((sl.numel(), H, d, d), generator=g, device=dev, dtype=torch.float32)
        S.mul_(0.1)
        fn(S, sl)
    torch.cuda.synchronize()


def time_launches(torch, launch, steps, warmup):
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        launch(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per launch


def host_threads():
    """Threads for the oracle's timed run: OMP_NUM_THREADS when the host environment sets it
    (the share of the host's cores this process is given), else every CPU this process may run
    on (its affinity mask). Returns (threads, where the figure came from)."""
    n = os.environ.get("OMP_NUM_THREADS", "")
    if n.isdigit() and int(n) > 0:
        return int(n), "OMP_NUM_THREADS"
    return len(os.sched_getaffinity(0)), "sched_getaffinity"


def cpu_baseline(seconds: float, mode: dict):
    """The oracle timed on this host's cores on a bounded sample of the workload being measured:
    its first 64 active slots (x heads units per call), in the format and mode the GPU runs.
    ``mode``: workload (synth.Workload), inputs (its first StepInputs), rows (FP16 rows [H, r]),
    and at most one of stq=(bits, impact), window=W, raw=(raw StepInputs for the fused pre-step),
    budget=(r_per_head, row_map)."""
    import oracle
    from quantized_delta_rule_gdn_amd import synth
    w, inp = mode["workload"], mode["inputs"]
    n_slots = min(64, w.batch)
    H, D = w.heads, w.d
    n = n_slots * H
    per_key = w.decay == synth.KDA
    S = synth.normal_states(np.random.default_rng([w.seed, 99]), (n, D, D), 0.1)
    vec = (inp.q[:n_slots].reshape(n, D), inp.k[:n_slots].reshape(n, D), inp.v[:n_slots].reshape(n, D),
           inp.alpha[:n_slots].reshape(n, D) if per_key else inp.alpha[:n_slots].reshape(n),
           inp.beta[:n_slots].reshape(n))
    if mode.get("budget") is not None:
        r_h, row_map = mode["budget"]
        mh = np.zeros((H, D), np.uint8)
        for hh in range(H):
            mh[hh, row_map[hh][:r_h[hh]]] = 1
    else:
        mh = synth.rows_to_mask(mode["rows"], D)
    mask = np.ascontiguousarray(np.broadcast_to(mh, (n_slots, H, D)).reshape(n, D))
    what = "DAMP"
    if mode.get("stq") is not None:
        bits, impact = mode["stq"]
        bb = np.ascontiguousarray(np.broadcast_to(bits, (n_slots, H, D)).reshape(n, D))
        ww = np.ascontiguousarray(np.broadcast_to(impact, (n_slots, H, D)).reshape(n, D))
        st = oracle.stq_quantize(bb, ww, S)
        call = lambda nt: oracle.stq_step(bb, ww, *st, *vec, nthreads=nt)
        what = "STEPQuant-style"
    elif mode.get("window"):
        h, c, s = oracle.quantize(mask, S)
        win = oracle.Window(mask, h, c, s, mode["window"])
        call = lambda nt: win.step(*vec, nthreads=nt)
        what = f"per-window (W = {mode['window']}) DAMP"
    elif mode.get("raw") is not None:
        raw = mode["raw"]
        h, c, s = oracle.quantize(mask, S)
        rv = (raw.q[:n_slots].reshape(n, D), raw.k[:n_slots].reshape(n, D),
              raw.alpha[:n_slots].reshape(n, D) if per_key else raw.alpha[:n_slots].reshape(n),
              raw.beta[:n_slots].reshape(n))

        def call(nt):
            qh, kh, a, bt = oracle.prestep(*rv)
            oracle.step_quant(mask, h, c, s, qh, kh, vec[2], a, bt, nthreads=nt)
        what = "pre-step + DAMP"
    else:
        h, c, s = oracle.quantize(mask, S)
        call = lambda nt: oracle.step_quant(mask, h, c, s, *vec, nthreads=nt)

    def timed(nthreads, budget):
        calls = 0
        t0 = time.perf_counter()
        while True:
            call(nthreads)
            calls += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return calls, el

    threads, source = host_threads()
    calls, el = timed(threads, seconds)
    calls1, el1 = timed(1, max(1.0, seconds / 4))
    model = ""
    try:
        model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": calls * n / el, "unit": "state-updates/s", "cores": threads,
            "threads_from": source, "host_logical_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{calls} oracle calls of {n:,} (slot, head) {what} updates (the first {n_slots} "
                      f"active slots of the workload) in {el:.1f} s",
            "gbs": calls * n * mode["alg_bytes"] / el / 1e9,
            "one_core": {"value": calls1 * n / el1, "sample": f"{calls1} calls in {el1:.1f} s"},
            "cpu_model": model}


def calibrate_budget(torch, lib, synth, dev, H, d, per_key, args):
    """Per-head FP16 rows for the budget: risk scores of the synthetic calibration states and
    the allocation, both on the device (each timed over 5 launches after one untimed)."""
    S_cal, abar = synth.budget_calibration(H, d, per_key=per_key)
    S_dev = torch.from_numpy(S_cal).to(dev)
    a_dev = torch.from_numpy(abar).to(dev)
    score, row_err = lib.risk_scores(S_dev, a_dev)
    t_score = time_launches(torch, lambda i: lib.risk_scores(S_dev, a_dev, row_err, score), 5, 1)
    g, r_max = args.budget_group, args.budget_rmax
    R = lib.budget_rows(d, H, args.budget_bits, g, r_max)
    if R < 0:
        raise SystemExit(f"--budget-bits {args.budget_bits}: below the all-INT8 layout")
    t_alloc = time_launches(torch, lambda i: lib.allocate_rows(score, R, g, r_max), 5, 1)
    r_dev, m_dev = lib.allocate_rows(score, R, g, r_max)
    r_h = r_dev.cpu().numpy()
    data = sum(2 * int(x) * d + (d - int(x)) * d + 4 * (d - int(x)) for x in r_h)
    return {"kind": "per-head FP16 rows under a storage budget", "bits_per_value": args.budget_bits,
            "data_bits_per_value": 8.0 * data / (H * d * d), "fp16_rows_total": R, "group": g,
            "r_max": r_max, "r_per_head": r_h.tolist(), "row_map": m_dev.cpu().numpy(),
            "calibration_states": int(S_cal.shape[0]), "risk_scores_ms": t_score,
            "allocate_ms": t_alloc}


WORKLOADS = ("pool4096", "gdn64", "kda256", "drift")
COLD_BYTES = 1 << 30  # rotate copies until this much state lies between two uses of one copy


def workload_setup(name, synth, torch, dev):
    """Slot sets (one per pool copy), FP16 rows, input sets and a description."""
    if name == "pool4096":
        w = synth.POOL4096
        active = synth.pool4096_slots()
        rows = synth.pool4096_rows()
        sets = [synth.pool4096_step(i) for i in range(4)]
        return w, [active], w.pool_slots, rows, sets, True, (
            "pool4096: GDN decode step, 4096-slot DAMP pool x 32 heads x 128x128, 1024 active "
            "random slots, 24 FP16 rows/head, bf16 qkv")
    w = {"gdn64": synth.GDN64, "kda256": synth.KDA256, "drift": synth.DRIFT}[name]
    rng = np.random.default_rng([w.seed, 7])
    rows = synth.random_rows(rng, w.heads, w.d, w.fp16_rows)
    sets = [synth.step_inputs(rng, w.batch, w.heads, w.d, w.decay, "bf16") for _ in range(4)]
    blk = 2 * w.fp16_rows * w.d + (w.d - w.fp16_rows) * w.d + 4 * (w.d - w.fp16_rows)
    copies = 1 if name == "drift" else -(-COLD_BYTES // (w.batch * w.heads * blk))
    slot_sets = [np.arange(c * w.batch, (c + 1) * w.batch, dtype=np.int32) for c in range(copies)]
    desc = {"gdn64": "gdn64: GDN decode step, 64 slots x 32 heads x 128x128, 24 FP16 rows/head, bf16 qkv",
            "kda256": "kda256: KDA decode step (per-key gate), 256 slots x 32 heads x 128x128, 24 FP16 rows/head, bf16 qkv",
            "drift": "drift: GDN decode step repeated on the same 64 slots x 32 heads x 128x128, 24 FP16 rows/head, bf16 qkv"}[name]
    return w, slot_sets, copies * w.batch, rows, sets, copies > 1, desc


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (every unit is "
              "independent; a multi-GPU run would shard slots or heads with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    import torch
    from quantized_delta_rule_gdn_amd import lib, synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w, slot_sets_np, pool_slots, rows, inputs, cold, desc = workload_setup(args.workload, synth, torch, dev)
    H, d, r = w.heads, w.d, w.fp16_rows
    per_key = w.decay == synth.KDA
    slot_sets = [torch.from_numpy(x).to(dev) for x in slot_sets_np]
    all_slots = torch.cat(slot_sets)
    B = slot_sets[0].numel()
    units = B * H
    bf = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev).view(torch.bfloat16)
    sets = [(bf(i.q_bits), bf(i.k_bits), bf(i.v_bits), torch.from_numpy(i.alpha).to(dev),
             torch.from_numpy(i.beta).to(dev)) for i in inputs]
    out = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    R = len(slot_sets)
    results = {}
    budget = None
    prestep_info = {}
    raw_sets = None
    stq_bits = stq_impact = None
    stq_data = 0
    if args.stq:
        stq_bits, stq_impact = synth.stq_map(np.random.default_rng(synth.STQ_SEED), H, d)
        for hh in range(H):
            n = {b: int((stq_bits[hh] == b).sum()) for b in (16, 8, 6, 4)}
            stq_data += (2 * d * n[16] + d * n[8] + 3 * d // 4 * n[6] + d // 2 * n[4]
                         + 2 * (d - n[16]) + 2 * d)
        stq_data /= H
        desc = desc.replace(f"{r} FP16 rows/head", "STEPQuant-style state, 2 FP16 pivots/head, "
                            f"8/6/4-bit rows at a nominal 6-bit map ({8 * stq_data / (d * d):.3f} bits/value)")
    if args.window:
        if not 1 <= args.window <= 8:
            raise SystemExit("--window must be in 1..8")
        # whole windows per timed run, and every pool copy at the same window position
        args.steps = -(-args.steps // (args.window * R)) * args.window * R
        args.warmup = -(-args.warmup // (args.window * R)) * args.window * R
        desc += f"; per-window requantization, windows of {args.window} tokens"
    if args.fused_prestep:
        rng = np.random.default_rng([w.seed, 11])
        raw = [synth.raw_step_inputs(rng, B, H, d, w.decay, "bf16") for _ in range(4)]
        raw_sets = [(bf(i.q_bits), bf(i.k_bits), bf(i.v_bits), torch.from_numpy(i.alpha).to(dev),
                     torch.from_numpy(i.beta).to(dev)) for i in raw]
        desc += "; pre-step fused (raw q/k, gate and beta logits)"
    if args.budget_bits is not None:
        budget = calibrate_budget(torch, lib, synth, dev, H, d, per_key, args)
        desc = desc.replace(f"{r} FP16 rows/head", f"per-head FP16 rows at {args.budget_bits} bits/value")
        print(f"# budget {args.budget_bits} bits: R = {budget['fp16_rows_total']}, r per head "
              f"{budget['r_per_head']}; risk scores {budget['risk_scores_ms']:.3f} ms, allocation "
              f"{budget['allocate_ms']:.3f} ms", file=sys.stderr, flush=True)

    use_order = order_enabled(args.order, units, args.window, args.stq)
    order_bufs = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(R)]

    def with_order(fmt, st, step):
        """The timed launch: step(i, order). With the order on, the DAMP steps ("damp", and the
        per-token step a window run compares with) list their batch by slot first, in every step,
        then run in that order; "damp_batch_order" is the same step in batch order."""
        if use_order and fmt in ("damp", "damp_token"):
            launch = lambda i: step(i, st.batch_order(slot_sets[i % R], out=order_bufs[i % R]))
            launch.ordered = (st, step)
            return launch
        return lambda i: step(i, None)

    def time_step(launch):
        """(ms per step, ms per launch of the step kernel alone). A step in slot order is its
        ordering launch and the ordered step; the step kernel alone is then timed again, in a run
        of its own with the orders computed beforehand."""
        ms = time_launches(torch, launch, args.steps, args.warmup)
        ordered = getattr(launch, "ordered", None)
        if ordered is None:
            return ms, ms
        st, step = ordered
        pre = [st.batch_order(x) for x in slot_sets]
        return ms, time_launches(torch, lambda i: step(i, pre[i % R]), args.steps, args.warmup)

    shared = {}

    def damp_pool():
        """The DAMP pool of the plain step (uniform r, or the budget's per-head layout), made and
        filled once: the step in batch order and the step in slot order run on the same pool,
        one after the other."""
        if "damp" not in shared:
            if budget is not None:
                st = lib.DampState(pool_slots, H, d, budget["row_map"], device=dev,
                                   r_per_head=budget["r_per_head"])
            else:
                st = lib.DampState(pool_slots, H, d, rows, device=dev)
            st.pool.zero_()
            fill_states(torch, st.quantize, all_slots, H, d, dev)
            shared["damp"] = st
        return shared["damp"]

    def run(fmt):
        if fmt == "damp" and args.stq:
            st = lib.StqState(pool_slots, H, d, stq_bits, stq_impact, device=dev)
            fill_states(torch, st.quantize, all_slots, H, d, dev)
            launch = lambda i: st.decode_step(slot_sets[i % R], *sets[i % 4], out)
            keep = st
        elif fmt == "damp" and args.window:
            st = lib.DampState(pool_slots, H, d, rows, device=dev)
            st.pool.zero_()
            fill_states(torch, st.quantize, all_slots, H, d, dev)
            wbuf = st.window_buffer(args.window)
            launch = with_order(fmt, st, lambda i, o: st.window_step(wbuf, args.window, slot_sets[i % R],
                                                                      *sets[i % 4], out, order=o))
            keep = (st, wbuf)
        elif fmt == "damp" and args.fused_prestep:
            st = lib.DampState(pool_slots, H, d, rows, device=dev)
            st.pool.zero_()
            fill_states(torch, st.quantize, all_slots, H, d, dev)
            launch = with_order(fmt, st, lambda i, o: st.decode_step_fused(slot_sets[i % R], *raw_sets[i % 4],
                                                                            out, order=o))
            keep = st
            F = torch.nn.functional

            def unfused(i, o):
                q, k, v, g, b = raw_sets[i % 4]
                qn = F.normalize(q.float(), dim=-1)
                kn = F.normalize(k.float(), dim=-1)
                st.decode_step(slot_sets[i % R], qn, kn, v.float(), torch.sigmoid(-g), torch.sigmoid(b), out,
                               order=o)
            prestep_info["unfused_ms"] = time_step(with_order(fmt, st, unfused))[0]
        elif fmt in ("damp", "damp_token", "damp_batch_order"):
            st = damp_pool()
            launch = with_order(fmt, st, lambda i, o: st.decode_step(slot_sets[i % R], *sets[i % 4], out, order=o))
            keep = None
        elif fmt == "fp32":
            pool = torch.zeros((pool_slots, H, d, d), dtype=torch.float32, device=dev)
            fill_states(torch, lambda S, sl: pool.index_copy_(0, sl.long(), S), all_slots, H, d, dev)
            launch = lambda i: lib.fp32_decode_step(pool, slot_sets[i % R], *sets[i % 4], out)
            keep = pool
        else:
            codes = torch.zeros((pool_slots, H, d, d), dtype=torch.int8, device=dev)
            scales = torch.zeros((pool_slots, H, d), dtype=torch.float32, device=dev)
            fill_states(torch, lambda S, sl: lib.uniform_int8_quantize(codes, scales, S, sl),
                        all_slots, H, d, dev)
            launch = lambda i: lib.uniform_int8_decode_step(codes, scales, slot_sets[i % R],
                                                            *sets[i % 4], out)
            keep = (codes, scales)
        ms, kernel_ms = time_step(launch)
        del keep
        torch.cuda.empty_cache()
        if fmt == "damp" and args.stq:
            ab = (2 * stq_data + alg_bytes_per_update("damp", d, r, per_key) - 2 * (2 * r * d + (d - r) * d + 4 * (d - r))) * units
        elif fmt == "damp" and args.window:
            ab = alg_bytes_window(args.window, d, r, per_key) * units
        elif fmt in ("damp", "damp_batch_order") and budget is not None:
            ab = sum(alg_bytes_per_update("damp", d, int(rh), per_key) for rh in budget["r_per_head"]) * B
        elif fmt in ("damp_token", "damp_batch_order"):
            ab = alg_bytes_per_update("damp", d, r, per_key) * units
        else:
            ab = alg_bytes_per_update(fmt, d, r, per_key) * units
        return {"ms_per_step": ms, "updates_per_s": units / (ms * 1e-3),
                "alg_bytes_per_launch": ab, "gbs": ab / (ms * 1e-3) / 1e9,
                "kernel_ms": kernel_ms, "kernel_gbs": ab / (kernel_ms * 1e-3) / 1e9}

    # The headline format runs last, right after the comparison runs: a long memory-bound run
    # settles the GPU's clocks, and a few launches after idle time run at other clocks than the
    # steady state (seen in kernel traces: the first tens of steps after a pause vary by up to
    # 10% before they settle).
    fmts = [args.only] if args.only else (["damp"] if args.no_baselines else ["fp32", "int8", "damp"])
    if args.window and not args.only:
        fmts.insert(len(fmts) - 1, "damp_token")   # the per-token step on the same pool, for comparison
    if use_order and "fp32" in fmts:
        fmts.insert(len(fmts) - 1, "damp_batch_order")   # like for like with the baselines (batch order)
    for f in fmts:
        results[f] = run(f)
        label = "stq" if (f == "damp" and args.stq) else f
        print(f"# {args.workload} {label}: {results[f]['ms_per_step'] * 1e3:.1f} us/step, "
              f"{results[f]['gbs']:.0f} GB/s; step kernel alone {results[f]['kernel_ms'] * 1e3:.1f} us",
              file=sys.stderr, flush=True)

    main_fmt = args.only or "damp"
    m = results[main_fmt]
    line = {
        "metric": "state-updates/s (slot·head·token) + achieved HBM GB/s vs peak, 1 MI355X",
        "value": m["updates_per_s"],
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32+fp16+int8" if main_fmt == "damp" else ("f32" if main_fmt == "fp32" else "f32+int8"),
        "data": "synthetic: seeded N(0, 0.1) states, unit-norm bf16 q/k, N(0,1) bf16 v, "
                "sigmoid gates; no model weights",
        "config": {"workload": desc, "format": "stq" if args.stq else main_fmt, "slots_active": B, "heads": H, "d": d,
                   "fp16_rows": r if budget is None else "per head", "global_batch": B, "seq_len": 1,
                   "state_cache": "cold (HBM)" if (cold or args.workload == "pool4096") else "warm (Infinity Cache)",
                   "pool_copies": R,
                   "unit_order": "ascending slot (damp_batch_order, then the ordered step, both timed "
                                 "in every step)" if use_order else "batch order"},
        "roofline": {"bound": "hbm", "achieved": m["kernel_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": m["kernel_gbs"] / PEAK_HBM_GBS, "kernel_us": m["kernel_ms"] * 1e3,
                     "traffic": measured_traffic() if (main_fmt == "damp" and args.workload == "pool4096"
                                                       and budget is None and not args.window
                                                       and not args.fused_prestep and not args.stq) else None},
    }
    if budget is not None:
        line["config"]["layout"] = {k: v for k, v in budget.items() if k != "row_map"}
    if prestep_info:
        prestep_info["fused_ms"] = results["damp"]["ms_per_step"]
        prestep_info["unfused"] = ("torch normalize(q), normalize(k), sigmoid(-g), sigmoid(b) in fp32, "
                                   "then damp_decode_step" + (" in slot order" if use_order else ""))
        line["prestep"] = prestep_info
    if "fp32" in results and "damp" in results:
        line["baselines"] = {f: {"ms_per_step": v["ms_per_step"], "updates_per_s": v["updates_per_s"],
                                 "gbs": v["gbs"], "frac": v["gbs"] / PEAK_HBM_GBS}
                             for f, v in results.items() if f != "damp"}
        same = results.get("damp_batch_order", results["damp"])   # the baselines run in batch order
        line["speedup_vs_fp32"] = results["fp32"]["ms_per_step"] / same["ms_per_step"]
    if not args.no_cpu_baseline:
        mode = {"workload": w, "inputs": inputs[0], "rows": rows,
                "alg_bytes": results[main_fmt]["alg_bytes_per_launch"] / units,
                "stq": (stq_bits, stq_impact) if args.stq else None,
                "window": args.window,
                "raw": raw[0] if args.fused_prestep else None,
                "budget": (budget["r_per_head"], budget["row_map"]) if budget is not None else None}
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds, mode)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
