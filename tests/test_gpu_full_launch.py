"""GPU parity of the other entry points at the benchmark's launch configuration: a 4,096-slot
pool, 1,024 random active slots x 32 heads x 128 x 128, bf16 inputs -- the STEPQuant-style step,
per-window requantization over a whole window, the step with the pre-step fused, and the step on
the per-head layout the 9.9-bit budget allocates. Every active slot is processed in the one
launch; 32 of them (every 32nd of the batch) hold states the oracle packed and are compared with
it unit by unit, the others hold device-packed random states and are checked for finite outputs;
inactive slots must keep their sentinel bytes. Tolerances as in gpu_common / test_gpu_stq."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle  # noqa: E402
import layout_ref  # noqa: E402
from gpu_common import SENTINEL, check_quant, check_readout, ref_vectors, step_tensors, to_dev  # noqa: E402
from quantized_delta_rule_gdn_amd import lib, synth  # noqa: E402
from test_gpu_stq import check_stq  # noqa: E402

W = synth.POOL4096
B, H, D = W.batch, W.heads, W.d
SAMPLE_B = np.arange(0, B, 32)          # batch positions compared with the oracle


def _log(msg):
    print(msg, flush=True)


def _fill_random(quantize, slots_dev, seed):
    """Device-packed N(0, 0.1) states for the given slots, in chunks."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for i in range(0, slots_dev.numel(), 128):
        sl = slots_dev[i:i + 128]
        quantize(torch.randn((sl.numel(), H, D, D), generator=g, device="cuda") * 0.1, sl)
    torch.cuda.synchronize()


def _sample(inp):
    """The sampled batch positions of a StepInputs, flattened for the oracle."""
    sub = synth.StepInputs(*(x[SAMPLE_B] for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta)), inp.dtype)
    return ref_vectors(sub, len(SAMPLE_B), H, D)


def _inactive_untouched(pool_rows, slots):
    inactive = torch.ones(pool_rows.shape[0], dtype=torch.bool, device="cuda")
    inactive[torch.from_numpy(slots).long().cuda()] = False
    assert bool((pool_rows[inactive] == SENTINEL).all()), "an inactive slot was written"


def test_stq_step_pool4096_launch():
    bits, impact = synth.stq_map(np.random.default_rng(synth.STQ_SEED), H, D)
    slots = synth.pool4096_slots()
    st = lib.StqState(W.pool_slots, H, D, bits, impact)
    st.pool.fill_(SENTINEL)
    _fill_random(st.quantize, to_dev(slots), 5)
    ns = len(SAMPLE_B)
    S = synth.normal_states(np.random.default_rng(51), (ns, H, D, D), 0.1)
    bb = np.broadcast_to(bits, (ns, H, D)).reshape(ns * H, D)
    ww = np.broadcast_to(impact, (ns, H, D)).reshape(ns * H, D)
    h, c, rf, cs = oracle.stq_quantize(bb, ww, S.reshape(ns * H, D, D))
    logical = tuple(x.reshape((ns, H) + x.shape[1:]) for x in (h, c, rf, cs))
    st.slots()[torch.from_numpy(slots[SAMPLE_B]).long().cuda()] = to_dev(layout_ref.stq_pack(bits, *logical))
    inp = synth.pool4096_step(0)
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    st.decode_step(to_dev(slots), *step_tensors(inp), out)
    torch.cuda.synchronize()
    _inactive_untouched(st.slots(), slots)
    out = out.cpu().numpy()
    assert np.isfinite(out).all()
    ref_out, ref_state, X_ref = oracle.stq_step(bb, ww, h, c, rf, cs, *_sample(inp), return_x=True)
    check_readout(out[SAMPLE_B], ref_out.reshape(ns, H, D))
    got = layout_ref.stq_unpack(bits, st.slots()[torch.from_numpy(slots[SAMPLE_B]).long().cuda()].cpu().numpy(), D)
    _log("stq pool4096: " + str(check_stq(bits, impact, got, tuple(x.reshape((ns, H) + x.shape[1:]) for x in ref_state),
                                          X_ref.reshape(ns, H, D, D))))


def _damp_pool(rows, slots, seed, r_per_head=None, row_map=None):
    if r_per_head is None:
        st = lib.DampState(W.pool_slots, H, D, rows)
    else:
        st = lib.DampState(W.pool_slots, H, D, row_map, r_per_head=r_per_head)
    st.pool.fill_(SENTINEL)
    _fill_random(st.quantize, to_dev(slots), seed)
    return st


def test_window_pool4096_launch():
    Wn = 4
    rows = synth.pool4096_rows()
    slots = synth.pool4096_slots()
    st = _damp_pool(rows, slots, 6)
    mask = synth.rows_to_mask(rows, D)
    ns = len(SAMPLE_B)
    maskn = np.broadcast_to(mask, (ns, H, D)).reshape(ns * H, D)
    S = synth.normal_states(np.random.default_rng(61), (ns * H, D, D), 0.1)
    h, c, s = oracle.quantize(maskn, S)
    st.blocks()[torch.from_numpy(slots[SAMPLE_B]).long().cuda()] = to_dev(
        layout_ref.pack(rows, h.reshape(ns, H, D, D), c.reshape(ns, H, D, D), s.reshape(ns, H, D)))
    win = oracle.Window(maskn, h, c, s, Wn)
    wbuf = st.window_buffer(Wn)
    slots_dev = to_dev(slots)
    for t in range(Wn):
        inp = synth.pool4096_step(t)
        out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
        st.window_step(wbuf, Wn, slots_dev, *step_tensors(inp), out)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        assert np.isfinite(out).all()
        check_readout(out[SAMPLE_B], win.step(*_sample(inp)).reshape(ns, H, D))
    _inactive_untouched(st.blocks(), slots)
    got = layout_ref.unpack(rows, st.blocks()[torch.from_numpy(slots[SAMPLE_B]).long().cuda()].cpu().numpy(), D)
    _log("window pool4096: " + str(check_quant(mask, got, (win.h.reshape(ns, H, D, D), win.c.reshape(ns, H, D, D),
                                                            win.s.reshape(ns, H, D)))))


def test_fused_prestep_pool4096_launch():
    rows = synth.pool4096_rows()
    slots = synth.pool4096_slots()
    st = _damp_pool(rows, slots, 7)
    mask = synth.rows_to_mask(rows, D)
    ns = len(SAMPLE_B)
    maskn = np.broadcast_to(mask, (ns, H, D)).reshape(ns * H, D)
    S = synth.normal_states(np.random.default_rng(71), (ns * H, D, D), 0.1)
    h, c, s = oracle.quantize(maskn, S)
    st.blocks()[torch.from_numpy(slots[SAMPLE_B]).long().cuda()] = to_dev(
        layout_ref.pack(rows, h.reshape(ns, H, D, D), c.reshape(ns, H, D, D), s.reshape(ns, H, D)))
    raw = synth.raw_step_inputs(np.random.default_rng(72), B, H, D, synth.GDN, "bf16")
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    st.decode_step_fused(to_dev(slots), *step_tensors(raw), out)
    torch.cuda.synchronize()
    _inactive_untouched(st.blocks(), slots)
    out = out.cpu().numpy()
    assert np.isfinite(out).all()
    q, k, v, g, b = _sample(raw)
    qh, kh, a, bt = oracle.prestep(q, k, g, b)
    ref = oracle.step_quant(maskn, h, c, s, qh, kh, v, a, bt)
    check_readout(out[SAMPLE_B], ref.reshape(ns, H, D))
    got = layout_ref.unpack(rows, st.blocks()[torch.from_numpy(slots[SAMPLE_B]).long().cuda()].cpu().numpy(), D)
    _log("fused pool4096: " + str(check_quant(mask, got, (h.reshape(ns, H, D, D), c.reshape(ns, H, D, D),
                                                           s.reshape(ns, H, D)))))


def test_budget_layout_pool4096_launch():
    Sc, abar = synth.budget_calibration(H, D, per_key=False)
    score, _ = lib.risk_scores(to_dev(Sc), to_dev(abar))
    R = lib.budget_rows(D, H, 9.9, 8, 32)
    r_dev, m_dev = lib.allocate_rows(score, R, 8, 32)
    r_per_head, row_map = r_dev.cpu().numpy(), m_dev.cpu().numpy()
    slots = synth.pool4096_slots()
    st = _damp_pool(None, slots, 8, r_per_head, row_map)
    mask = layout_ref.mask_per_head(r_per_head, row_map, D)
    ns = len(SAMPLE_B)
    maskn = np.broadcast_to(mask, (ns, H, D)).reshape(ns * H, D)
    S = synth.normal_states(np.random.default_rng(81), (ns * H, D, D), 0.1)
    h, c, s = oracle.quantize(maskn, S)
    st.slots()[torch.from_numpy(slots[SAMPLE_B]).long().cuda()] = to_dev(
        layout_ref.pack_per_head(r_per_head, row_map, h.reshape(ns, H, D, D), c.reshape(ns, H, D, D),
                                 s.reshape(ns, H, D)))
    inp = synth.pool4096_step(0)
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    st.decode_step(to_dev(slots), *step_tensors(inp), out)
    torch.cuda.synchronize()
    _inactive_untouched(st.slots(), slots)
    out = out.cpu().numpy()
    assert np.isfinite(out).all()
    ref = oracle.step_quant(maskn, h, c, s, *_sample(inp))
    check_readout(out[SAMPLE_B], ref.reshape(ns, H, D))
    got = layout_ref.unpack_per_head(r_per_head, row_map,
                                     st.slots()[torch.from_numpy(slots[SAMPLE_B]).long().cuda()].cpu().numpy(), D)
    _log(f"budget pool4096 (r per head {sorted(set(r_per_head.tolist()))}): " +
         str(check_quant(mask, got, (h.reshape(ns, H, D, D), c.reshape(ns, H, D, D), s.reshape(ns, H, D)))))


def test_ordered_step_pool4096_launch():
    """The benchmark's step at its launch configuration: batch_order, then the step in that
    order, against the step in batch order on a copy of the pool -- every byte of the pool and
    every readout equal (inactive slots included, which keep their sentinel)."""
    rows = synth.pool4096_rows()
    slots = synth.pool4096_slots()
    ref = _damp_pool(rows, slots, 9)
    got = lib.DampState(W.pool_slots, H, D, rows)
    got.pool.copy_(ref.pool)
    slots_dev = to_dev(slots)
    order = got.batch_order(slots_dev)
    assert np.array_equal(slots[order.cpu().numpy()], np.sort(slots))
    for t in range(2):
        x = step_tensors(synth.pool4096_step(t))
        o_ref = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
        o_got = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
        ref.decode_step(slots_dev, *x, o_ref)
        got.decode_step(slots_dev, *x, o_got, order=order)
        torch.cuda.synchronize()
        assert torch.equal(o_got, o_ref), f"readout, step {t}"
        assert torch.equal(got.pool, ref.pool), f"pool, step {t}"
    _inactive_untouched(got.blocks(), slots)
