"""damp_decode_step_sorted, the step for callers that cannot allocate: it lists the batch by slot
in the library-held order buffer and runs the ordered step. Checked through the C ABI against the
same step with a caller-owned order buffer (damp_batch_order, then damp_decode_step_ordered) and
against damp_decode_step in batch order, on two calls in a row, the second with a smaller batch
(and the other gate form): every byte of the pool and every readout equal."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from gpu_common import SENTINEL, step_tensors, to_dev  # noqa: E402
from quantized_delta_rule_gdn_amd import lib, synth  # noqa: E402

NUM_SLOTS, H, D, R = 3000, 8, 128, 24


def _pools(rows, slots):
    g = torch.Generator(device="cuda").manual_seed(77)
    pools = [lib.DampState(NUM_SLOTS, H, D, rows) for _ in range(3)]
    pools[0].pool.fill_(SENTINEL)
    pools[0].quantize(torch.randn((len(slots), H, D, D), generator=g, device="cuda") * 0.1, to_dev(slots))
    for p in pools[1:]:
        p.pool.copy_(pools[0].pool)
    return pools


def test_sorted_step_matches_the_ordered_step_on_two_calls():
    rng = np.random.default_rng(2026)
    rows = synth.random_rows(rng, H, D, R)
    active = rng.choice(NUM_SLOTS, 2500, replace=False).astype(np.int32)
    sorted_st, ordered_st, plain_st = _pools(rows, active)
    # call 1: 2,500 requests, GDN; call 2: a smaller batch (300 of them, reshuffled), KDA
    calls = [(active, synth.GDN), (rng.permutation(active)[:300], synth.KDA)]
    for n, (slots, decay) in enumerate(calls):
        print(f"sorted step, call {n + 1}: B {len(slots)}, decay {decay}", flush=True)
        B = len(slots)
        inp = synth.step_inputs(rng, B, H, D, decay, "bf16")
        vec = step_tensors(inp)
        sl = to_dev(slots)
        outs = [torch.full((B, H, D), float("nan"), device="cuda") for _ in range(3)]
        sorted_st.decode_step_sorted(sl, *vec, outs[0])
        ordered_st.decode_step(sl, *vec, outs[1], order=ordered_st.batch_order(sl))
        plain_st.decode_step(sl, *vec, outs[2])
        torch.cuda.synchronize()
        assert torch.equal(sorted_st.pool, ordered_st.pool), f"call {n + 1}: pool differs from the ordered step"
        assert torch.equal(sorted_st.pool, plain_st.pool), f"call {n + 1}: pool differs from the plain step"
        assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2]), f"call {n + 1}: readouts differ"
        assert torch.isfinite(outs[0]).all()


def test_sorted_step_rejects_a_batch_above_its_buffer_and_takes_an_empty_one():
    rng = np.random.default_rng(5)
    st = lib.DampState(16, H, D, synth.random_rows(rng, H, D, R))
    B = lib.SORTED_MAX_B + 1
    inp = [torch.zeros((B, H, D), device="cuda") for _ in range(3)]
    sc = [torch.zeros((B, H), device="cuda") for _ in range(2)]
    out = torch.zeros((B, H, D), device="cuda")
    with pytest.raises(lib.DampError) as e:
        st.decode_step_sorted(torch.zeros(B, dtype=torch.int32, device="cuda"), *inp, *sc, out)
    assert e.value.status == lib.DAMP_ERR_UNSUPPORTED
    empty = torch.zeros((0, H, D), device="cuda")
    st.decode_step_sorted(torch.zeros(0, dtype=torch.int32, device="cuda"), empty, empty, empty,
                          torch.zeros((0, H), device="cuda"), torch.zeros((0, H), device="cuda"), empty)
