"""The processing order: damp_batch_order lists the batch positions by ascending slot bucket
(checked exactly against the bucket rule, on every kind of slot list), and the step taken in any
order -- that one, a random permutation, batch order -- gives, bit for bit, the pool and the
readouts of damp_decode_step (each unit's arithmetic does not depend on the order)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from gpu_common import SENTINEL, step_tensors, to_dev  # noqa: E402
from quantized_delta_rule_gdn_amd import lib, synth  # noqa: E402


def _shift(num_slots):
    s = 0
    while (num_slots - 1) >> s >= 4096:
        s += 1
    return s


def _check_order(slots, num_slots):
    order = lib.batch_order(to_dev(slots), num_slots).cpu().numpy()
    B = len(slots)
    assert order.dtype == np.int32 and order.shape == (B,)
    assert np.array_equal(np.sort(order), np.arange(B)), "not a permutation"
    bucket = np.clip(slots.astype(np.int64), 0, num_slots - 1) >> _shift(num_slots)
    assert np.all(np.diff(bucket[order]) >= 0), "buckets not ascending"
    return order


@pytest.mark.parametrize("num_slots,B,seed", [(4096, 1024, 1), (4096, 4096, 2), (8192, 3000, 3),
                                              (64, 64, 4), (1_000_000, 2500, 5), (7, 1, 6)])
def test_batch_order_of_unique_slots(num_slots, B, seed):
    print(f"batch order: pool {num_slots}, B {B}", flush=True)
    slots = np.random.default_rng(seed).choice(num_slots, B, replace=False).astype(np.int32)
    order = _check_order(slots, num_slots)
    if _shift(num_slots) == 0:   # an exact sort
        assert np.array_equal(slots[order], np.sort(slots))


def test_batch_order_of_repeated_and_out_of_range_slots():
    rng = np.random.default_rng(9)
    slots = rng.integers(-50, 5000, 2100).astype(np.int32)   # repeats, negatives, >= num_slots
    slots[:5] = [-2**31, 2**31 - 1, 0, 4095, 4095]
    _check_order(slots, 4096)


def test_batch_order_of_an_empty_batch():
    assert lib.batch_order(torch.empty(0, dtype=torch.int32, device="cuda"), 16).numel() == 0


B, H, D = 40, 8, 128


def _states(make, slots, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    a, b = make(), make()
    a.pool.fill_(SENTINEL)
    a.quantize(torch.randn((len(slots), H, D, D), generator=g, device="cuda") * 0.1, to_dev(slots))
    b.pool.copy_(a.pool)
    return a, b


@pytest.mark.parametrize("decay", [synth.GDN, synth.KDA])
@pytest.mark.parametrize("per_head", [None, "row steps", "any r"])
def test_ordered_step_is_bit_exact(decay, per_head):
    """Uniform layout; per-head layouts whose r are all multiples of the row step (the
    compile-time row kinds) and with one r that is not (the general instance)."""
    print(f"ordered step: decay {decay}, per-head {per_head}", flush=True)
    rng = np.random.default_rng([decay, 0 if per_head is None else len(per_head)])
    slots = rng.choice(4 * B, B, replace=False).astype(np.int32)
    if per_head:
        r_per_head = np.array([0, 8, 16, 24, 32, 24, 8, 12 if per_head == "any r" else 8], np.int32)
        row_map = np.stack([rng.permutation(D) for _ in range(H)]).astype(np.int32)
        for h in range(H):   # each head's FP16 rows ascending, then its other rows ascending
            row_map[h] = np.concatenate([np.sort(row_map[h, :r_per_head[h]]), np.sort(row_map[h, r_per_head[h]:])])
        make = lambda: lib.DampState(4 * B, H, D, row_map, r_per_head=r_per_head)
    else:
        rows = synth.random_rows(rng, H, D, 24)
        make = lambda: lib.DampState(4 * B, H, D, rows)
    ref, got = _states(make, slots, 3)
    sl = to_dev(slots)
    orders = [lib.batch_order(sl, 4 * B), to_dev(rng.permutation(B).astype(np.int32)),
              to_dev(np.arange(B, dtype=np.int32))]
    for t, order in enumerate(orders):
        x = step_tensors(synth.step_inputs(np.random.default_rng([7, t]), B, H, D, decay, "bf16"))
        o_ref = torch.empty((B, H, D), device="cuda")
        o_got = torch.full((B, H, D), float("nan"), device="cuda")
        ref.decode_step(sl, *x, o_ref)
        got.decode_step(sl, *x, o_got, order=order)
        torch.cuda.synchronize()
        assert torch.equal(o_got, o_ref), f"readout, order {t}"
        assert torch.equal(got.pool, ref.pool), f"pool, order {t}"


def test_order_entries_outside_the_batch_are_skipped():
    rng = np.random.default_rng(11)
    slots = rng.choice(4 * B, B, replace=False).astype(np.int32)
    rows = synth.random_rows(rng, H, D, 24)
    ref, got = _states(lambda: lib.DampState(4 * B, H, D, rows), slots, 5)
    before = got.blocks()[int(slots[-1])].clone()
    order = np.arange(B, dtype=np.int32)
    order[-1] = B + 5          # position B - 1 is never listed; B + 5 is no batch position
    x = step_tensors(synth.step_inputs(np.random.default_rng(12), B, H, D, synth.GDN, "bf16"))
    o_ref = torch.empty((B, H, D), device="cuda")
    o_got = torch.full((B, H, D), 7.0, device="cuda")
    ref.decode_step(to_dev(slots[:-1]), *(y[:-1] for y in x), o_ref[:-1])
    got.decode_step(to_dev(slots), *x, o_got, order=to_dev(order))
    torch.cuda.synchronize()
    assert torch.equal(o_got[:-1], o_ref[:-1])
    assert bool((o_got[-1] == 7.0).all()), "the skipped position's readout was written"
    assert torch.equal(got.blocks()[int(slots[-1])], before), "the skipped position's state changed"
    assert torch.equal(got.pool, ref.pool)


@pytest.mark.parametrize("D,r,Bn,Hn,decay", [(16, 5, 9, 2, synth.KDA), (32, 8, 7, 3, synth.GDN),
                                             (64, 4, 11, 2, synth.GDN), (128, 12, 5, 2, synth.KDA),
                                             (128, 27, 6, 3, synth.GDN)])
def test_ordered_step_every_instance(D, r, Bn, Hn, decay):
    """Every d and launch plan (general r, r % 4 == 0, compile-time kinds): a random order gives the
    batch-order step bit for bit."""
    print(f"ordered step D={D} r={r} B={Bn} H={Hn}", flush=True)
    rng = np.random.default_rng([D, r, Bn])
    slots = rng.choice(3 * Bn, Bn, replace=False).astype(np.int32)
    rows = synth.random_rows(rng, Hn, D, r)
    g = torch.Generator(device="cuda").manual_seed(D + r)
    ref, got = lib.DampState(3 * Bn, Hn, D, rows), lib.DampState(3 * Bn, Hn, D, rows)
    ref.pool.fill_(SENTINEL)
    ref.quantize(torch.randn((Bn, Hn, D, D), generator=g, device="cuda") * 0.1, to_dev(slots))
    got.pool.copy_(ref.pool)
    x = step_tensors(synth.step_inputs(np.random.default_rng([D, 1]), Bn, Hn, D, decay, "bf16"))
    o_ref = torch.empty((Bn, Hn, D), device="cuda")
    o_got = torch.empty((Bn, Hn, D), device="cuda")
    sl = to_dev(slots)
    ref.decode_step(sl, *x, o_ref)
    got.decode_step(sl, *x, o_got, order=to_dev(rng.permutation(Bn).astype(np.int32)))
    torch.cuda.synchronize()
    assert torch.equal(o_got, o_ref)
    assert torch.equal(got.pool, ref.pool)


def test_ordered_fused_and_window_steps_are_bit_exact():
    """The fused pre-step and the per-window step (windows of 2 over 3 tokens: one end, one
    pending; both decay modes) in a random order give the batch-order results bit for bit:
    readouts, pool and window buffers."""
    rng = np.random.default_rng(21)
    slots = rng.choice(4 * B, B, replace=False).astype(np.int32)
    rows = synth.random_rows(rng, H, D, 24)
    ref, got = _states(lambda: lib.DampState(4 * B, H, D, rows), slots, 13)
    sl = to_dev(slots)
    perm = to_dev(rng.permutation(B).astype(np.int32))
    o_ref = torch.empty((B, H, D), device="cuda")
    o_got = torch.empty((B, H, D), device="cuda")
    for decay in (synth.GDN, synth.KDA):
        raw = step_tensors(synth.raw_step_inputs(np.random.default_rng([22, decay]), B, H, D, decay, "bf16"))
        ref.decode_step_fused(sl, *raw, o_ref)
        got.decode_step_fused(sl, *raw, o_got, order=perm)
        torch.cuda.synchronize()
        assert torch.equal(o_got, o_ref), f"fused readout, decay {decay}"
        assert torch.equal(got.pool, ref.pool), f"fused pool, decay {decay}"
        w_ref, w_got = ref.window_buffer(2), got.window_buffer(2)
        for t in range(3):
            x = step_tensors(synth.step_inputs(np.random.default_rng([23, decay, t]), B, H, D, decay, "bf16"))
            ref.window_step(w_ref, 2, sl, *x, o_ref)
            got.window_step(w_got, 2, sl, *x, o_got, order=perm)
            torch.cuda.synchronize()
            assert torch.equal(o_got, o_ref), f"window readout, decay {decay}, token {t}"
            assert torch.equal(got.pool, ref.pool), f"window pool, decay {decay}, token {t}"
            assert torch.equal(w_got, w_ref), f"window buffer, decay {decay}, token {t}"
