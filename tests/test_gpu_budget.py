"""GPU parity of the budgeted selection and the per-head DAMP layout (through the C ABI).

- Risk scores: the device computes them in binary64 in the order the oracle defines, so scores
  and per-row errors must be bit-identical to the oracle's.
- Allocation: an integer result decided by comparing scores; from identical scores the device's
  per-head counts and row maps must equal the oracle's exactly (ties included).
- Per-head layout: the decode step, pack and unpack on a layout whose heads keep different
  numbers of FP16 rows, against the oracle step on the same mask, with the tolerances of
  gpu_common. Both step kernels are covered: every r a multiple of the row step (compile-time
  row kinds, selected per head) and arbitrary r (the general kernel).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle  # noqa: E402
import layout_ref  # noqa: E402
from gpu_common import check_quant, check_readout, ref_vectors, step_tensors, to_dev  # noqa: E402
from quantized_delta_rule_gdn_amd import lib, synth  # noqa: E402


def _log(msg):
    print(msg, flush=True)


def _calib_states(seed, n, H, D):
    """Calibration states with structure: heavy rows and columns, a zero row, tiny and large
    heads, and rows of exact code multiples (zero error)."""
    rng = np.random.default_rng(seed)
    S = synth.normal_states(rng, (n, H, D, D), 0.1)
    for h in range(H):
        S[:, h, rng.choice(D, max(1, D // 16), replace=False), :] *= 10
        S[:, h, :, rng.choice(D, max(1, D // 32), replace=False)] *= 4
    S[:, 0, 1, :] = 0.0
    if H > 2:
        S[:, 1] *= np.float32(1e-20)
        S[:, 2] *= np.float32(300.0)
    S[0, 0, 2, :] = np.float32(2.0 ** -7) * rng.integers(-127, 128, D).astype(np.float32)
    S[0, 0, 2, 0] = np.float32(127 * 2.0 ** -7)
    abar = rng.uniform(0.0, 0.97, (H, D)).astype(np.float32)
    abar[0, :5] = 0.5
    return S, abar


@pytest.mark.parametrize("D,n,H", [(16, 5, 3), (64, 3, 4), (128, 8, 4)])
def test_risk_scores_bit_exact(D, n, H):
    S, abar = _calib_states(D + n, n, H, D)
    score, row_err = lib.risk_scores(to_dev(S), to_dev(abar))
    torch.cuda.synchronize()
    ref = oracle.risk_scores(S, abar)
    ref_err = np.array([[[oracle.int8_row_error(S[s, h, i]) for i in range(D)] for h in range(H)]
                        for s in range(n)])
    assert np.array_equal(row_err.cpu().numpy(), ref_err)
    assert np.array_equal(score.cpu().numpy(), ref)


def _scores(seed, H, D, ties):
    rng = np.random.default_rng(seed)
    sc = rng.exponential(1.0, (H, D)) * rng.uniform(0.1, 10.0, (H, 1))
    if ties:
        sc = np.round(sc, 1)
        sc[0] = 1.0
    return sc


@pytest.mark.parametrize("H,D,g,r_max,R", [
    (3, 16, 1, 16, 7), (3, 16, 2, 8, 10), (4, 32, 4, 16, 24), (2, 16, 3, 16, 9),
    (5, 16, 8, 4, 8),                                   # r_max < g: no group can be taken
    (32, 128, 8, 32, 872), (32, 128, 1, 128, 872),      # 9.9 bits at D = 128: 4,096 groups
    (32, 128, 8, 32, 32 * 32), (64, 128, 2, 128, 0),
])
@pytest.mark.parametrize("ties", [False, True])
def test_allocation_bit_exact(H, D, g, r_max, R, ties):
    sc = _scores(H * 1000 + D + g + R, H, D, ties)
    r, m = lib.allocate_rows(to_dev(sc), R, g, r_max)
    torch.cuda.synchronize()
    rr, mr = oracle.allocate_rows(sc, R, g, r_max)
    assert np.array_equal(r.cpu().numpy(), rr)
    assert np.array_equal(m.cpu().numpy(), mr)


def _per_head_case(seed, B, H, D, r_per_head, row_map, decay, dtype):
    rng = np.random.default_rng(seed)
    S = synth.normal_states(rng, (B, H, D, D), 0.1)
    for h in range(H):
        S[:, h, rng.choice(D, max(1, D // 32), replace=False), :] *= 8
    inp = synth.step_inputs(rng, B, H, D, decay, dtype)
    mask = layout_ref.mask_per_head(r_per_head, row_map, D)
    maskn = np.broadcast_to(mask, (B, H, D)).reshape(B * H, D)
    h, c, s = oracle.quantize(maskn, S.reshape(B * H, D, D))
    return S, inp, mask, maskn, h, c, s


def _run_per_head(r_per_head, row_map, S, inp, mask, maskn, h, c, s, num_slots, slots):
    B, H, D, _ = S.shape
    st = lib.DampState(num_slots, H, D, row_map, r_per_head=r_per_head)
    assert st.slot_bytes == layout_ref.head_offsets(D, r_per_head)[1]
    st.pool.fill_(0xA5)
    sl = torch.from_numpy(np.asarray(slots, np.int64)).cuda()
    st.slots()[sl] = to_dev(layout_ref.pack_per_head(r_per_head, row_map, h.reshape(B, H, D, D),
                                                     c.reshape(B, H, D, D), s.reshape(B, H, D)))
    q, k, v, a, b = step_tensors(inp)
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    st.decode_step(to_dev(np.asarray(slots, np.int32)), q, k, v, a, b, out)
    torch.cuda.synchronize()
    got = layout_ref.unpack_per_head(r_per_head, row_map, st.slots()[sl].cpu().numpy(), D)
    ref_out = oracle.step_quant(maskn, h, c, s, *ref_vectors(inp, B, H, D))
    check_readout(out.cpu().numpy(), ref_out)
    stats = check_quant(mask, got, (h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D)))
    other = np.setdiff1d(np.arange(num_slots), slots)
    assert bool((st.slots()[torch.from_numpy(other).long().cuda()] == 0xA5).all())
    return st, stats


@pytest.mark.parametrize("D,H,B,g,r_max,bits,decay,dtype", [
    (128, 8, 9, 8, 32, 9.9, synth.GDN, "bf16"),   # r in {0, 8, .., 32}: compile-time row kinds
    (128, 6, 5, 1, 40, 9.9, synth.KDA, "bf16"),   # arbitrary r: the general kernel
    (64, 4, 7, 8, 16, 10.5, synth.KDA, "fp32"),
    (16, 3, 4, 1, 16, 11.0, synth.GDN, "fp32"),
])
def test_per_head_layout_step(D, H, B, g, r_max, bits, decay, dtype):
    # calibrate on the device, allocate the budget there, then step on that layout
    Sc, abar = _calib_states(D * 7 + H, 4, H, D)
    score, _ = lib.risk_scores(to_dev(Sc), to_dev(abar))
    R = lib.budget_rows(D, H, bits, g, r_max)
    r_dev, m_dev = lib.allocate_rows(score, R, g, r_max)
    r_per_head, row_map = r_dev.cpu().numpy(), m_dev.cpu().numpy()
    rr, mr = oracle.allocate_rows(oracle.risk_scores(Sc, abar), R, g, r_max)
    assert np.array_equal(r_per_head, rr) and np.array_equal(row_map, mr)
    _log(f"D={D} H={H} g={g} bits={bits}: R={R}, r per head {r_per_head.tolist()}")
    S, inp, mask, maskn, h, c, s = _per_head_case(D + B, B, H, D, r_per_head, row_map, decay, dtype)
    num_slots = 2 * B + 1
    slots = np.random.default_rng(B).choice(num_slots, B, replace=False)
    _, stats = _run_per_head(r_per_head, row_map, S, inp, mask, maskn, h, c, s, num_slots, slots)
    _log(str(stats))


@pytest.mark.parametrize("r_per_head", [[0, 8, 16, 24, 32, 8], [5, 0, 13, 40, 128, 1]])
def test_per_head_pack_unpack_bit_exact(r_per_head):
    D, H, n = 128, 6, 3
    rng = np.random.default_rng(len(r_per_head) + sum(r_per_head))
    r_per_head = np.array(r_per_head, np.int32)
    row_map = np.empty((H, D), np.int32)
    for hh in range(H):
        f = np.sort(rng.choice(D, r_per_head[hh], replace=False))
        row_map[hh] = np.concatenate([f, np.setdiff1d(np.arange(D), f)])
    S = synth.normal_states(rng, (n, H, D, D), 0.1)
    S[0, 1, 3, :] = 0.0
    mask = layout_ref.mask_per_head(r_per_head, row_map, D)
    maskn = np.broadcast_to(mask, (n, H, D)).reshape(n * H, D)
    h, c, s = oracle.quantize(maskn, S.reshape(n * H, D, D))
    st = lib.DampState(2 * n, H, D, row_map, r_per_head=r_per_head)
    st.pool.zero_()
    slots = torch.tensor([4, 1, 2], dtype=torch.int32, device="cuda")
    st.quantize(to_dev(S), slots)
    back = st.dequantize(slots)
    torch.cuda.synchronize()
    got = layout_ref.unpack_per_head(r_per_head, row_map, st.slots()[slots.long()].cpu().numpy(), D)
    assert np.array_equal(got[0], h.reshape(n, H, D, D))
    assert np.array_equal(got[1], c.reshape(n, H, D, D))
    assert np.array_equal(got[2], s.reshape(n, H, D))
    ref_back = oracle.dequantize(maskn, h, c, s).reshape(n, H, D, D)
    assert np.array_equal(back.cpu().numpy(), ref_back)


@pytest.mark.parametrize("per_key", [False, True])
def test_budget_workload_full_heads(per_key):
    """The benchmark's calibration data (32 heads x 128 rows, 64 states) at 9.9 bits, groups of
    8, at most 32 rows per head; then the step on 64 slots of that layout against the oracle."""
    H, D, B = 32, 128, 64
    Sc, abar = synth.budget_calibration(H, D, per_key=per_key)
    score, _ = lib.risk_scores(to_dev(Sc), to_dev(abar))
    R = lib.budget_rows(D, H, 9.9, 8, 32)
    assert R == 872 // 8 * 8
    r_dev, m_dev = lib.allocate_rows(score, R, 8, 32)
    r_per_head, row_map = r_dev.cpu().numpy(), m_dev.cpu().numpy()
    ref_score = oracle.risk_scores(Sc, abar)
    assert np.array_equal(score.cpu().numpy(), ref_score)
    rr, mr = oracle.allocate_rows(ref_score, R, 8, 32)
    assert np.array_equal(r_per_head, rr) and np.array_equal(row_map, mr)
    assert int(r_per_head.sum()) == R and len(set(r_per_head.tolist())) > 1
    _log(f"budget workload per_key={per_key}: r per head {r_per_head.tolist()}")
    decay = synth.KDA if per_key else synth.GDN
    S, inp, mask, maskn, h, c, s = _per_head_case(11 + per_key, B, H, D, r_per_head, row_map, decay, "bf16")
    _, stats = _run_per_head(r_per_head, row_map, S, inp, mask, maskn, h, c, s, B + 5,
                             np.random.default_rng(3).choice(B + 5, B, replace=False))
    _log(str(stats))
