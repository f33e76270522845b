"""Slot indices outside [0, num_slots), outside debug mode: every kernel that addresses a pool by
slot skips such a request (nothing of it is read or written; its readout rows and unpacked
states stay as they were), and the other requests give, bit for bit, what a call with only them
gives. Covers the DAMP step (plain, ordered, sorted), the fp32 and uniform-INT8 steps, pack and
unpack, the window step and flush, and the STEPQuant-style state."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from gpu_common import step_tensors, to_dev  # noqa: E402
from quantized_delta_rule_gdn_amd import lib, synth  # noqa: E402

NUM_SLOTS, H, D, R = 8, 3, 128, 24
SLOTS = np.array([2, 9, 5, -1, 7, 2 ** 31 - 1, 8, -2 ** 31], np.int32)
VALID = np.array([0, 2, 4])                       # the positions of slots 2, 5 and 7
BAD = np.setdiff1d(np.arange(len(SLOTS)), VALID)
MARK = 12345.0


def _sub(inp, idx):
    return synth.StepInputs(inp.q[idx], inp.k[idx], inp.v[idx], inp.alpha[idx], inp.beta[idx],
                            inp.dtype, inp.q_bits[idx], inp.k_bits[idx], inp.v_bits[idx])


def _states(seed):
    rng = np.random.default_rng(seed)
    return rng, synth.normal_states(rng, (NUM_SLOTS, H, D, D), 0.1), synth.random_rows(rng, H, D, R)


def _damp_pools(S, rows):
    pools = [lib.DampState(NUM_SLOTS, H, D, rows) for _ in range(2)]
    every = torch.arange(NUM_SLOTS, dtype=torch.int32, device="cuda")
    for p in pools:
        p.pool.zero_()
        p.quantize(to_dev(S), every)
    return pools


def _check_outputs(out, ref):
    assert torch.equal(out[torch.from_numpy(VALID).cuda()], ref), "a valid request differs"
    assert bool((out[torch.from_numpy(BAD).cuda()] == MARK).all()), "a skipped request wrote its readout"


@pytest.mark.parametrize("decay", [synth.GDN, synth.KDA])
@pytest.mark.parametrize("mode", ["plain", "ordered", "sorted"])
def test_damp_step_skips_out_of_range_slots(decay, mode):
    rng, S, rows = _states(11 + decay)
    a, b = _damp_pools(S, rows)
    inp = synth.step_inputs(rng, len(SLOTS), H, D, decay, "bf16")
    out = torch.full((len(SLOTS), H, D), MARK, device="cuda")
    sl = to_dev(SLOTS)
    print(f"bad slots: DAMP step, {mode}, decay {decay}", flush=True)
    if mode == "plain":
        a.decode_step(sl, *step_tensors(inp), out)
    elif mode == "ordered":
        a.decode_step(sl, *step_tensors(inp), out, order=a.batch_order(sl))
    else:
        a.decode_step_sorted(sl, *step_tensors(inp), out)
    ref = torch.empty((len(VALID), H, D), device="cuda")
    b.decode_step(to_dev(SLOTS[VALID]), *step_tensors(_sub(inp, VALID)), ref)
    torch.cuda.synchronize()
    _check_outputs(out, ref)
    assert torch.equal(a.pool, b.pool)


def test_baseline_steps_skip_out_of_range_slots():
    rng, S, _ = _states(21)
    inp = synth.step_inputs(rng, len(SLOTS), H, D, synth.GDN, "bf16")
    sl, sv = to_dev(SLOTS), to_dev(SLOTS[VALID])
    print("bad slots: fp32 and uniform-INT8 steps", flush=True)
    f = [to_dev(S) for _ in range(2)]
    out = torch.full((len(SLOTS), H, D), MARK, device="cuda")
    ref = torch.empty((len(VALID), H, D), device="cuda")
    lib.fp32_decode_step(f[0], sl, *step_tensors(inp), out)
    lib.fp32_decode_step(f[1], sv, *step_tensors(_sub(inp, VALID)), ref)
    torch.cuda.synchronize()
    _check_outputs(out, ref)
    assert torch.equal(f[0], f[1])
    every = torch.arange(NUM_SLOTS, dtype=torch.int32, device="cuda")
    cs = [(torch.zeros((NUM_SLOTS, H, D, D), dtype=torch.int8, device="cuda"),
           torch.zeros((NUM_SLOTS, H, D), device="cuda")) for _ in range(2)]
    for c, s in cs:
        lib.uniform_int8_quantize(c, s, to_dev(S), every)
    out.fill_(MARK)
    lib.uniform_int8_decode_step(*cs[0], sl, *step_tensors(inp), out)
    lib.uniform_int8_decode_step(*cs[1], sv, *step_tensors(_sub(inp, VALID)), ref)
    torch.cuda.synchronize()
    _check_outputs(out, ref)
    assert torch.equal(cs[0][0], cs[1][0]) and torch.equal(cs[0][1], cs[1][1])


def test_pack_and_unpack_skip_out_of_range_slots():
    rng, _, rows = _states(31)
    Sb = synth.normal_states(rng, (len(SLOTS), H, D, D), 0.1)   # one state per request
    print("bad slots: pack and unpack", flush=True)
    pools = [lib.DampState(NUM_SLOTS, H, D, rows) for _ in range(2)]
    for p in pools:
        p.pool.fill_(0xA5)
    pools[0].quantize(to_dev(Sb), to_dev(SLOTS))
    pools[1].quantize(to_dev(Sb[VALID]), to_dev(SLOTS[VALID]))
    back = torch.full((len(SLOTS), H, D, D), MARK, device="cuda")
    pools[0].dequantize(to_dev(SLOTS), back)
    ref = pools[1].dequantize(to_dev(SLOTS[VALID]))
    torch.cuda.synchronize()
    assert torch.equal(pools[0].pool, pools[1].pool)
    assert torch.equal(back[torch.from_numpy(VALID).cuda()], ref)
    assert bool((back[torch.from_numpy(BAD).cuda()] == MARK).all())


@pytest.mark.parametrize("decay", [synth.GDN, synth.KDA])
def test_window_skips_out_of_range_slots(decay):
    rng, S, rows = _states(41 + decay)
    pools = _damp_pools(S, rows)
    W = 4
    bufs = [p.window_buffer(W) for p in pools]
    sl, sv = to_dev(SLOTS), to_dev(SLOTS[VALID])
    print(f"bad slots: window, decay {decay}", flush=True)
    for _ in range(2):
        inp = synth.step_inputs(rng, len(SLOTS), H, D, decay, "bf16")
        out = torch.full((len(SLOTS), H, D), MARK, device="cuda")
        ref = torch.empty((len(VALID), H, D), device="cuda")
        pools[0].window_step(bufs[0], W, sl, *step_tensors(inp), out)
        pools[1].window_step(bufs[1], W, sv, *step_tensors(_sub(inp, VALID)), ref)
        torch.cuda.synchronize()
        _check_outputs(out, ref)
    pools[0].window_flush(bufs[0], W, sl)
    pools[1].window_flush(bufs[1], W, sv)
    torch.cuda.synchronize()
    assert torch.equal(pools[0].pool, pools[1].pool)
    assert torch.equal(bufs[0], bufs[1])


def test_stq_skips_out_of_range_slots():
    rng = np.random.default_rng(51)
    bits, impact = synth.stq_map(rng, H, D)
    S = synth.normal_states(rng, (len(SLOTS), H, D, D), 0.1)
    print("bad slots: STEPQuant-style pack, step and unpack", flush=True)
    st = [lib.StqState(NUM_SLOTS, H, D, bits, impact) for _ in range(2)]
    for p in st:
        p.pool.zero_()
    st[0].quantize(to_dev(S), to_dev(SLOTS))
    st[1].quantize(to_dev(S[VALID]), to_dev(SLOTS[VALID]))
    inp = synth.step_inputs(rng, len(SLOTS), H, D, synth.KDA, "bf16")
    out = torch.full((len(SLOTS), H, D), MARK, device="cuda")
    ref = torch.empty((len(VALID), H, D), device="cuda")
    st[0].decode_step(to_dev(SLOTS), *step_tensors(inp), out)
    st[1].decode_step(to_dev(SLOTS[VALID]), *step_tensors(_sub(inp, VALID)), ref)
    back = torch.full((len(SLOTS), H, D, D), MARK, device="cuda")
    st[0].dequantize(to_dev(SLOTS), back)
    torch.cuda.synchronize()
    _check_outputs(out, ref)
    assert torch.equal(st[0].pool, st[1].pool)
    assert bool((back[torch.from_numpy(BAD).cuda()] == MARK).all())
