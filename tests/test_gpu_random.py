"""Randomized parity sweep: seeded random shapes (d, r, batch, heads), gate forms, input types,
state outliers and unit orders for the DAMP step, and random shapes, pivot counts, edge precision
maps and in-place / second-pool writes for the STEPQuant-style step, each against the oracle
from identical input states with the tolerances of gpu_common / test_gpu_stq. DAMP_SWEEP_SCALE=n
runs n times as many cases of each sweep (the first ones are the same); at n = 60 (18,000 DAMP
steps, 9,000 STEPQuant-style steps, 2,400 window runs, 6,000 fused steps) every case passes."""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle  # noqa: E402
from gpu_common import DampPool, check_quant, check_readout, ref_vectors, step_tensors  # noqa: E402
from quantized_delta_rule_gdn_amd import synth  # noqa: E402
from test_gpu_parity import _random_case  # noqa: E402
from test_gpu_stq import _edge_map, _step_case  # noqa: E402

SCALE = int(os.environ.get("DAMP_SWEEP_SCALE", "1"))


def _random_per_head(master, H, D):
    """A random per-head layout: each head's r (all multiples of the row step up to 32, half the
    time at d = 128, else any r) and a row map listing its FP16 rows, then its other rows, each
    ascending."""
    if D == 128 and master.random() < 0.5:
        r_per_head = (8 * master.integers(0, 5, H)).astype(np.int32)
    else:
        r_per_head = master.integers(0, D + 1, H).astype(np.int32)
    row_map = np.empty((H, D), np.int32)
    for h in range(H):
        p = master.permutation(D)
        row_map[h] = np.concatenate([np.sort(p[:r_per_head[h]]), np.sort(p[r_per_head[h]:])])
    return r_per_head, row_map


class _PerHeadPool:
    """The per-head counterpart of gpu_common.DampPool: logical states packed at ``slots``."""

    def __init__(self, r_per_head, row_map, logical, slots, num_slots):
        import layout_ref
        from gpu_common import SENTINEL, to_dev
        from quantized_delta_rule_gdn_amd import lib
        H, D = row_map.shape
        self.r_per_head, self.row_map, self.D, self.H = r_per_head, row_map, D, H
        self.state = lib.DampState(num_slots, H, D, row_map, r_per_head=r_per_head)
        self.state.pool.fill_(SENTINEL)
        self.slot_dev = to_dev(np.asarray(slots, np.int32))
        self.state.slots()[self.slot_dev.long()] = to_dev(layout_ref.pack_per_head(r_per_head, row_map, *logical))

    def logical(self):
        import layout_ref
        return layout_ref.unpack_per_head(self.r_per_head, self.row_map,
                                          self.state.slots()[self.slot_dev.long()].cpu().numpy(), self.D)


def test_random_damp_steps():
    master = np.random.default_rng(20261203)
    worst = 1.0
    for i in range(300 * SCALE):
        D = int(master.choice([16, 32, 64, 128, 128, 128]))
        if master.random() < 0.3:
            r = int(master.integers(0, D + 1))
        else:
            r = min(int(master.choice([0, 8, 16, 24, 32, 27])), D)
        B, H = int(master.integers(1, 40)), int(master.integers(1, 6))
        decay, dtype = int(master.integers(0, 2)), ("bf16" if master.random() < 0.7 else "fp32")
        seed, ordered = int(master.integers(0, 2**31)), bool(master.random() < 0.5)
        outliers = bool(master.random() < 0.7)
        case = f"case {i}: D={D} r={r} B={B} H={H} decay={decay} {dtype} seed={seed} ordered={ordered}"
        rows, S, inp = _random_case(seed, B, H, D, r, decay, dtype, outliers=outliers)
        num_slots = 2 * B + 3
        slots = np.random.default_rng(seed + 1).choice(num_slots, B, replace=False)
        mask = synth.rows_to_mask(rows, D)
        maskn = np.broadcast_to(mask, (B, H, D)).reshape(B * H, D)
        h, c, s = oracle.quantize(maskn, S.reshape(B * H, D, D))
        pool = DampPool(rows, h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D), slots,
                        num_slots)
        q, k, v, a, b = step_tensors(inp)
        out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
        order = pool.state.batch_order(pool.slot_dev) if ordered else None
        pool.state.decode_step(pool.slot_dev, q, k, v, a, b, out, order=order)
        torch.cuda.synchronize()
        ref_out = oracle.step_quant(maskn, h, c, s, *ref_vectors(inp, B, H, D))
        try:
            check_readout(out.cpu().numpy(), ref_out.reshape(B, H, D))
            st = check_quant(mask, pool.logical(), (h.reshape(B, H, D, D), c.reshape(B, H, D, D),
                                                    s.reshape(B, H, D)))
        except AssertionError as e:
            raise AssertionError(f"{case}: {e}") from None
        worst = min(worst, st.get("code_eq_frac", 1.0))
    print(f"{300 * SCALE} random DAMP steps, worst code agreement {worst:.6f}", flush=True)


def test_random_stq_steps():
    master = np.random.default_rng(7070)
    for i in range(150 * SCALE):
        D = int(master.choice([64, 128, 128]))
        H, B = int(master.integers(1, 5)), int(master.integers(1, 12))
        decay, dtype = int(master.integers(0, 2)), ("bf16" if master.random() < 0.7 else "fp32")
        pivots, seed = int(master.integers(0, 5)), int(master.integers(0, 2**31))
        inplace = bool(master.random() < 0.6)
        bits = impact = None
        name = "nominal"
        if master.random() < 0.3:
            name = str(master.choice(["one_of_each", "all4", "ragged", "all16"]))
            bits, impact = _edge_map(name, H, D, np.random.default_rng(seed))
        try:
            _step_case(D, H, B, decay, dtype, pivots, seed, inplace, bits=bits, impact=impact)
        except AssertionError as e:
            raise AssertionError(f"case {i}: D={D} H={H} B={B} decay={decay} {dtype} pivots={pivots} "
                                 f"seed={seed} inplace={inplace} map={name}: {e}") from None


def test_random_window_runs():
    """Random window lengths, token counts (ending mid-window, then a flush), shapes, gate forms,
    unit orders and (a third of the runs) per-head layouts, against the oracle's windowed step
    token by token."""
    from test_gpu_window import _resync, _setup
    master = np.random.default_rng(4242)
    for i in range(40 * SCALE):
        D = int(master.choice([16, 64, 128, 128]))
        r = min(int(master.choice([0, 8, 24, 27])), D)
        B, H = int(master.integers(1, 12)), int(master.integers(1, 4))
        W, tokens = int(master.integers(1, 9)), int(master.integers(1, 12))
        decay, dtype = int(master.integers(0, 2)), ("bf16" if master.random() < 0.7 else "fp32")
        seed, ordered = int(master.integers(0, 2**31)), bool(master.random() < 0.5)
        per_head = D >= 64 and master.random() < 0.34
        case = (f"case {i}: D={D} r={r} B={B} H={H} W={W} tokens={tokens} decay={decay} {dtype} "
                f"ordered={ordered} per_head={per_head}")
        slots = np.random.default_rng(seed + 1).choice(2 * B, B, replace=False)
        if per_head:
            import layout_ref
            r_per_head, row_map = _random_per_head(master, H, D)
            rng = np.random.default_rng(seed)
            S = synth.normal_states(rng, (B, H, D, D), 0.1)
            mask = layout_ref.mask_per_head(r_per_head, row_map, D)
            maskn = np.broadcast_to(mask, (B, H, D)).reshape(B * H, D)
            h, c, s = oracle.quantize(maskn, S.reshape(B * H, D, D))
            pool = _PerHeadPool(r_per_head, row_map, (h.reshape(B, H, D, D), c.reshape(B, H, D, D),
                                                      s.reshape(B, H, D)), slots, 2 * B)
            case += f" r_per_head={r_per_head.tolist()}"
        else:
            rng, rows, mask, maskn, h, c, s = _setup(seed, B, H, D, r, decay)
            pool = DampPool(rows, h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D), slots, 2 * B)
        win = oracle.Window(maskn, h.copy(), c.copy(), s.copy(), W)
        wbuf = pool.state.window_buffer(W)
        order = pool.state.batch_order(pool.slot_dev) if ordered else None
        want = lambda: (win.h.reshape(B, H, D, D), win.c.reshape(B, H, D, D), win.s.reshape(B, H, D))
        try:
            for tok in range(tokens):
                inp = synth.step_inputs(rng, B, H, D, decay, dtype)
                q, k, v, a, b = step_tensors(inp)
                out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
                pool.state.window_step(wbuf, W, pool.slot_dev, q, k, v, a, b, out, order=order)
                torch.cuda.synchronize()
                check_readout(out.cpu().numpy(), win.step(*ref_vectors(inp, B, H, D)).reshape(B, H, D))
                if (tok + 1) % W == 0:
                    got = pool.logical()
                    check_quant(mask, got, want())
                    _resync(win, got)
            pool.state.window_flush(wbuf, W, pool.slot_dev)
            win.flush()
            torch.cuda.synchronize()
            check_quant(mask, pool.logical(), want())
        except AssertionError as e:
            raise AssertionError(f"{case}: {e}") from None


def test_random_fused_steps():
    """Random shapes, gate forms and unit orders of the step with the pre-step fused (raw q, k
    with magnitudes over two decades, gate and beta logits), against the oracle's pre-step and
    step."""
    from test_gpu_prestep import _case, _oracle_fused
    master = np.random.default_rng(5151)
    for i in range(100 * SCALE):
        D = int(master.choice([16, 64, 128, 128]))
        r = min(int(master.choice([0, 8, 12, 24, 27])), D)
        B, H = int(master.integers(1, 30)), int(master.integers(1, 5))
        decay, dtype = int(master.integers(0, 2)), ("bf16" if master.random() < 0.7 else "fp32")
        seed, ordered = int(master.integers(0, 2**31)), bool(master.random() < 0.5)
        case = f"case {i}: D={D} r={r} B={B} H={H} decay={decay} {dtype} seed={seed} ordered={ordered}"
        rows, S, inp = _case(seed, B, H, D, r, decay, dtype)
        mask = synth.rows_to_mask(rows, D)
        maskn = np.broadcast_to(mask, (B, H, D)).reshape(B * H, D)
        h, c, s = oracle.quantize(maskn, S.reshape(B * H, D, D))
        slots = np.random.default_rng(seed + 1).choice(2 * B, B, replace=False)
        pool = DampPool(rows, h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D), slots, 2 * B)
        q, k, v, g, b = step_tensors(inp)
        out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
        order = pool.state.batch_order(pool.slot_dev) if ordered else None
        pool.state.decode_step_fused(pool.slot_dev, q, k, v, g, b, out, order=order)
        torch.cuda.synchronize()
        try:
            check_readout(out.cpu().numpy(), _oracle_fused(maskn, h, c, s, inp, B, H, D).reshape(B, H, D))
            check_quant(mask, pool.logical(), (h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D)))
        except AssertionError as e:
            raise AssertionError(f"{case}: {e}") from None


def test_random_per_head_layouts():
    """Random per-head layouts (each head its own r and FP16 rows; all r multiples of the row
    step up to 32, which takes the compile-time row-kind instance, or any r), random gate forms
    and unit orders, the step (a third of the cases with the pre-step fused) against the oracle."""
    import layout_ref
    from gpu_common import SENTINEL, to_dev
    from quantized_delta_rule_gdn_amd import lib
    from test_gpu_prestep import _oracle_fused
    master = np.random.default_rng(6161)
    for i in range(30 * SCALE):
        D = int(master.choice([64, 128, 128]))
        H, B = int(master.integers(1, 6)), int(master.integers(1, 20))
        r_per_head, row_map = _random_per_head(master, H, D)
        decay, dtype = int(master.integers(0, 2)), ("bf16" if master.random() < 0.7 else "fp32")
        seed, ordered = int(master.integers(0, 2**31)), bool(master.random() < 0.5)
        fused = bool(master.random() < 0.34)
        case = (f"case {i}: D={D} H={H} B={B} r={r_per_head.tolist()} decay={decay} {dtype} "
                f"ordered={ordered} fused={fused}")
        rng = np.random.default_rng(seed)
        S = synth.normal_states(rng, (B, H, D, D), 0.1)
        mask = layout_ref.mask_per_head(r_per_head, row_map, D)
        maskn = np.broadcast_to(mask, (B, H, D)).reshape(B * H, D)
        h_, c_, s_ = oracle.quantize(maskn, S.reshape(B * H, D, D))
        logical = (h_.reshape(B, H, D, D), c_.reshape(B, H, D, D), s_.reshape(B, H, D))
        num = 2 * B + 1
        st = lib.DampState(num, H, D, row_map, r_per_head=r_per_head)
        st.pool.fill_(SENTINEL)
        slots = np.random.default_rng(seed + 1).choice(num, B, replace=False).astype(np.int32)
        sl = to_dev(slots)
        st.slots()[sl.long()] = to_dev(layout_ref.pack_per_head(r_per_head, row_map, *logical))
        out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
        order = st.batch_order(sl) if ordered else None
        if fused:
            inp = synth.raw_step_inputs(rng, B, H, D, decay, dtype)
            st.decode_step_fused(sl, *step_tensors(inp), out, order=order)
            ref = _oracle_fused(maskn, h_, c_, s_, inp, B, H, D)
        else:
            inp = synth.step_inputs(rng, B, H, D, decay, dtype)
            st.decode_step(sl, *step_tensors(inp), out, order=order)
            ref = oracle.step_quant(maskn, h_, c_, s_, *ref_vectors(inp, B, H, D))
        torch.cuda.synchronize()
        got = layout_ref.unpack_per_head(r_per_head, row_map, st.slots()[sl.long()].cpu().numpy(), D)
        try:
            check_readout(out.cpu().numpy(), ref.reshape(B, H, D))
            check_quant(mask, got, logical)
        except AssertionError as e:
            raise AssertionError(f"{case}: {e}") from None
