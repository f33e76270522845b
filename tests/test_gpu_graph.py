"""The steps inside a HIP graph: one damp_decode_step (plain, and in slot order after
damp_batch_order; one in-place STEPQuant-style step; and one token of a per-window step, whose
window buffer is compared too) captured with torch.cuda.graph and replayed several times, with eager work and synchronisation
between the replays; every replay must equal, bit for bit, the same step run eagerly the same
number of times (the states evolve in place, so replay i is eager step i)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

from gpu_common import step_tensors, to_dev  # noqa: E402
from quantized_delta_rule_gdn_amd import lib, synth  # noqa: E402

B, H, D, r, REPLAYS = 24, 4, 128, 24, 4


def _run(make_state, step, replays=REPLAYS):
    inp = step_tensors(synth.step_inputs(np.random.default_rng(8), B, H, D, synth.GDN, "bf16"))
    slots = to_dev(np.random.default_rng(9).choice(2 * B, B, replace=False).astype(np.int32))
    S = torch.randn((B, H, D, D), generator=torch.Generator(device="cuda").manual_seed(10), device="cuda") * 0.1
    eager, graphed = make_state(), make_state()
    eager.quantize(S, slots)
    graphed.pool.copy_(eager.pool)
    out_e = torch.empty((B, H, D), device="cuda")
    out_g = torch.empty((B, H, D), device="cuda")
    # warm-up on a scratch state: first launches load the kernels outside the capture
    scratch = make_state()
    scratch.pool.copy_(eager.pool)
    step(scratch, slots, inp, out_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(graphed, slots, inp, out_g)
    torch.cuda.synchronize()
    noise = torch.zeros(1 << 20, device="cuda")
    for i in range(replays):
        step(eager, slots, inp, out_e)
        g.replay()
        noise.add_(1.0)                      # the program's own eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"readout of replay {i}"
        assert torch.equal(graphed.pool, eager.pool), f"state after replay {i}"
        if hasattr(eager, "wbuf"):
            assert torch.equal(graphed.wbuf, eager.wbuf), f"window buffer after replay {i}"


def test_damp_step_in_a_graph():
    rows = synth.random_rows(np.random.default_rng(7), H, D, r)

    def make():
        st = lib.DampState(2 * B, H, D, rows)
        st.pool.zero_()
        return st

    _run(make, lambda st, sl, x, out: st.decode_step(sl, *x, out))


def test_ordered_damp_step_in_a_graph():
    """The benchmark's step: damp_batch_order into a fixed buffer, then the step in that order
    (two launches captured together)."""
    rows = synth.random_rows(np.random.default_rng(7), H, D, r)
    order = torch.empty(B, dtype=torch.int32, device="cuda")

    def make():
        st = lib.DampState(2 * B, H, D, rows)
        st.pool.zero_()
        return st

    def step(st, sl, x, out):
        st.decode_step(sl, *x, out, order=st.batch_order(sl, out=order))

    _run(make, step)


def test_stq_step_in_a_graph():
    bits, impact = synth.stq_map(np.random.default_rng(6), H, D)

    def make():
        st = lib.StqState(2 * B, H, D, bits, impact)
        return st

    _run(make, lambda st, sl, x, out: st.decode_step(sl, *x, out))


def test_window_step_in_a_graph():
    """One token of a 4-token window per replay (GDN gates): the fourth replay ends the window
    and requantizes the states, the fifth and sixth start the next window."""
    rows = synth.random_rows(np.random.default_rng(7), H, D, r)
    W = 4

    def make():
        st = lib.DampState(2 * B, H, D, rows)
        st.pool.zero_()
        st.wbuf = st.window_buffer(W)
        return st

    _run(make, lambda st, sl, x, out: st.window_step(st.wbuf, W, sl, *x, out), replays=6)
