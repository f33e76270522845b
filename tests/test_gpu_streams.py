"""Steps on caller streams: two streams (default priority) updating disjoint slot sets of one pool
at the same time give, bit for bit, the states and readouts of the same steps run one after the
other on one stream; the DAMP, per-window and STEPQuant-style steps are all stream-ordered."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from gpu_common import step_tensors, to_dev  # noqa: E402
from quantized_delta_rule_gdn_amd import lib, synth  # noqa: E402

B, H, D, r = 48, 8, 128, 24


def _inputs(seed):
    return [step_tensors(synth.step_inputs(np.random.default_rng([seed, t]), B, H, D, synth.KDA, "bf16"))
            for t in range(3)]


def _halves():
    slots = np.random.default_rng(5).choice(2 * B, B, replace=False).astype(np.int32)
    return to_dev(slots), to_dev(slots[: B // 2]), to_dev(slots[B // 2:])


def _split(x, lo):
    return x[:B // 2] if lo else x[B // 2:]


def test_damp_steps_on_two_streams():
    rows = synth.random_rows(np.random.default_rng(1), H, D, r)
    all_sl, sa, sb = _halves()
    S = torch.randn((B, H, D, D), generator=torch.Generator(device="cuda").manual_seed(3), device="cuda") * 0.1
    ref = lib.DampState(2 * B, H, D, rows)
    ref.pool.zero_()
    ref.quantize(S, all_sl)
    two = lib.DampState(2 * B, H, D, rows)
    two.pool.copy_(ref.pool)
    torch.cuda.synchronize()
    steps = _inputs(7)
    out_ref = torch.empty((B, H, D), device="cuda")
    outs = []
    for q, k, v, a, b in steps:        # one stream, the whole batch
        ref.decode_step(all_sl, q, k, v, a, b, out_ref)
        outs.append(out_ref.clone())
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    o1 = [torch.empty((B // 2, H, D), device="cuda") for _ in steps]
    o2 = [torch.empty((B // 2, H, D), device="cuda") for _ in steps]
    torch.cuda.synchronize()
    for i, (q, k, v, a, b) in enumerate(steps):
        # stream 1 in batch order, stream 2 in slot order (its own order buffer, made on it)
        with torch.cuda.stream(s1):
            two.decode_step(sa, *(_split(x, True) for x in (q, k, v, a, b)), o1[i], stream=s1)
        with torch.cuda.stream(s2):
            order = two.batch_order(sb, stream=s2)
            two.decode_step(sb, *(_split(x, False) for x in (q, k, v, a, b)), o2[i], stream=s2,
                            order=order)
    torch.cuda.synchronize()
    assert torch.equal(two.pool, ref.pool)
    for i in range(len(steps)):
        assert torch.equal(torch.cat([o1[i], o2[i]]), outs[i])


def test_window_and_stq_steps_on_two_streams():
    all_sl, sa, sb = _halves()
    gen = torch.Generator(device="cuda").manual_seed(9)
    S = torch.randn((B, H, D, D), generator=gen, device="cuda") * 0.1
    steps = _inputs(11)
    # per-window requantization, windows of 2 tokens over 3 tokens (one end, one pending)
    rows = synth.random_rows(np.random.default_rng(2), H, D, r)
    ref, two = lib.DampState(2 * B, H, D, rows), lib.DampState(2 * B, H, D, rows)
    ref.pool.zero_()
    ref.quantize(S, all_sl)
    two.pool.copy_(ref.pool)
    wr, w2 = ref.window_buffer(2), two.window_buffer(2)
    # STEPQuant-style state, new states into a second pool
    bits, impact = synth.stq_map(np.random.default_rng(4), H, D)
    qr, q2 = lib.StqState(2 * B, H, D, bits, impact), lib.StqState(2 * B, H, D, bits, impact)
    qr.quantize(S, all_sl)
    q2.pool.copy_(qr.pool)
    dr, d2 = torch.zeros_like(qr.pool), torch.zeros_like(q2.pool)
    torch.cuda.synchronize()
    out = torch.empty((B, H, D), device="cuda")
    ref_out = []
    for q, k, v, a, b in steps:
        ref.window_step(wr, 2, all_sl, q, k, v, a, b, out)
        ref_out.append(out.clone())
    qr.decode_step(all_sl, *steps[0], out, dst=dr)
    ref_out.append(out.clone())
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    got = [[torch.empty((B // 2, H, D), device="cuda") for _ in range(4)] for _ in range(2)]
    torch.cuda.synchronize()
    for j, (st, sl, lo) in enumerate(((s1, sa, True), (s2, sb, False))):
        with torch.cuda.stream(st):
            for i, x in enumerate(steps):
                two.window_step(w2, 2, sl, *(_split(y, lo) for y in x), got[j][i], stream=st)
            q2.decode_step(sl, *(_split(y, lo) for y in steps[0]), got[j][3], dst=d2, stream=st)
    torch.cuda.synchronize()
    assert torch.equal(two.pool, ref.pool) and torch.equal(w2, wr)
    assert torch.equal(d2, dr) and torch.equal(q2.pool, qr.pool)
    for i in range(4):
        assert torch.equal(torch.cat([got[0][i], got[1][i]]), ref_out[i])
