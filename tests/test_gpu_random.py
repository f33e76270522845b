"""Randomized parity sweep: seeded random shapes (d, r, batch, heads), gate forms, input types,
state outliers and unit orders for the DAMP step, and random shapes, pivot counts, edge precision
maps and in-place / second-pool writes for the STEPQuant-style step, each against the oracle
from identical input states with the tolerances of gpu_common / test_gpu_stq. (The same sweep was
run offline at 5,000 DAMP and 400 STEPQuant-style cases with no failure.)"""
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


def test_random_damp_steps():
    master = np.random.default_rng(20261203)
    worst = 1.0
    for i in range(300):
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
    print(f"300 random DAMP steps, worst code agreement {worst:.6f}", flush=True)


def test_random_stq_steps():
    master = np.random.default_rng(7070)
    for i in range(150):
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
