"""GPU parity of per-window requantization (damp_window_step / damp_window_flush) against the
oracle's windowed step: readouts every token, the pool untouched inside a window, and the stored
state at every window end and after a flush. Tolerances as in gpu_common. Covers the
compile-time row-kind instances, the general instance, a per-head layout, smaller d, a window of
one token, and requests at different positions of their windows."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle  # noqa: E402
import layout_ref  # noqa: E402
from gpu_common import DampPool, check_quant, check_readout, ref_vectors, step_tensors, to_dev  # noqa: E402
from quantized_delta_rule_gdn_amd import lib, synth  # noqa: E402


def _log(msg):
    print(msg, flush=True)


def _setup(seed, B, H, D, r, decay):
    rng = np.random.default_rng(seed)
    S = synth.normal_states(rng, (B, H, D, D), 0.1)
    for hh in range(H):
        S[:, hh, rng.choice(D, max(1, D // 32), replace=False), :] *= 8
    rows = synth.random_rows(rng, H, D, r)
    mask = synth.rows_to_mask(rows, D)
    maskn = np.broadcast_to(mask, (B, H, D)).reshape(B * H, D)
    h, c, s = oracle.quantize(maskn, S.reshape(B * H, D, D))
    return rng, rows, mask, maskn, h, c, s


def _resync(win, got):
    """Parity is checked from identical input states: after a window end has been compared, the
    oracle continues from the GPU's stored state (the two may differ by the few codes the
    tolerance allows, which would otherwise carry into the next window's readouts)."""
    h, c, s = got
    win.h[...] = h.reshape(win.h.shape)
    win.c[...] = c.reshape(win.c.shape)
    win.s[...] = s.reshape(win.s.shape)


def _gpu_step(pool, wbuf, W, slots_dev, inp):
    B = slots_dev.shape[0]
    q, k, v, a, b = step_tensors(inp)
    out = torch.empty((B, pool.H, pool.D), dtype=torch.float32, device="cuda")
    pool.state.window_step(wbuf, W, slots_dev, q, k, v, a, b, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("D,r,B,H,W,decay,dtype,tokens", [
    (128, 24, 9, 4, 4, synth.GDN, "bf16", 10),    # compile-time row kinds
    (128, 27, 5, 3, 8, synth.KDA, "bf16", 11),    # general instance
    (128, 16, 6, 2, 3, synth.KDA, "fp32", 7),
    (64, 8, 7, 3, 5, synth.GDN, "fp32", 7),
    (16, 2, 4, 2, 2, synth.KDA, "bf16", 5),
    (128, 24, 5, 2, 1, synth.GDN, "bf16", 3),     # one token per window: the per-token step
    # compile-time row kinds with windows over 4 tokens: the last token's update holds seven
    # terms' deltas in registers and reads the eighth from LDS (W = 8), or holds six of eight
    # with two empty (W = 6); both end mid-window and flush
    (128, 24, 7, 3, 8, synth.GDN, "bf16", 19),
    (128, 16, 5, 2, 6, synth.KDA, "fp32", 9),
])
def test_window_steps_and_flush(D, r, B, H, W, decay, dtype, tokens):
    rng, rows, mask, maskn, h, c, s = _setup(D + r + W, B, H, D, r, decay)
    win = oracle.Window(maskn, h.copy(), c.copy(), s.copy(), W)
    slots = np.random.default_rng(B + W).choice(2 * B, B, replace=False)
    pool = DampPool(rows, h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D), slots, 2 * B)
    wbuf = pool.state.window_buffer(W)
    start = pool.state.blocks().clone()
    for tok in range(tokens):
        inp = synth.step_inputs(rng, B, H, D, decay, dtype)
        out = _gpu_step(pool, wbuf, W, pool.slot_dev, inp)
        ref = win.step(*ref_vectors(inp, B, H, D))
        check_readout(out, ref.reshape(B, H, D))
        if (tok + 1) % W == 0:
            got = pool.logical()
            stats = check_quant(mask, got, (win.h.reshape(B, H, D, D), win.c.reshape(B, H, D, D),
                                            win.s.reshape(B, H, D)))
            _resync(win, got)
            start = pool.state.blocks().clone()
            _log(f"window end after token {tok + 1}: {stats}")
        else:
            assert torch.equal(pool.state.blocks(), start), "pool written inside a window"
    # flush what is pending and compare
    pool.state.window_flush(wbuf, W, pool.slot_dev)
    win.flush()
    torch.cuda.synchronize()
    check_quant(mask, pool.logical(), (win.h.reshape(B, H, D, D), win.c.reshape(B, H, D, D),
                                       win.s.reshape(B, H, D)))
    # a second flush finds nothing pending and leaves the pool as it is
    before = pool.state.blocks().clone()
    pool.state.window_flush(wbuf, W, pool.slot_dev)
    torch.cuda.synchronize()
    assert torch.equal(pool.state.blocks(), before)


@pytest.mark.parametrize("case,decay", [("identity", synth.GDN), ("identity", synth.KDA),
                                        ("full_forget", synth.GDN), ("mixed_gates", synth.KDA)])
def test_window_degenerate(case, decay):
    """One window of W = 4 tokens with degenerate gates: alpha = 1 and beta = 0 on every token
    (the window end stores the codes and FP16 rows it started from, bit for bit); alpha = 0 on
    every token (the state at the window end is k delta^T of its last token, rank one, so every
    differing code must sit at a rounding tie, X in closed form); per key row gates of exactly 0
    and 1 mixed with drawn ones."""
    B, H, D, r, W = 5, 3, 128, 24, 4
    rng, rows, mask, maskn, h, c, s = _setup(606, B, H, D, r, decay)
    win = oracle.Window(maskn, h.copy(), c.copy(), s.copy(), W)
    pool = DampPool(rows, h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D), np.arange(B), B)
    wbuf = pool.state.window_buffer(W)
    for tok in range(W):
        inp = synth.step_inputs(rng, B, H, D, decay, "bf16")
        if case == "identity":
            inp.alpha[:] = 1.0
            inp.beta[:] = 0.0
        elif case == "full_forget":
            inp.alpha[:] = 0.0
        else:
            sel = rng.integers(0, 3, inp.alpha.shape)
            inp.alpha[sel == 0] = 0.0
            inp.alpha[sel == 1] = 1.0
        out = _gpu_step(pool, wbuf, W, pool.slot_dev, inp)
        check_readout(out, win.step(*ref_vectors(inp, B, H, D)).reshape(B, H, D))
    got = pool.logical()
    ref = (win.h.reshape(B, H, D, D), win.c.reshape(B, H, D, D), win.s.reshape(B, H, D))
    stats = check_quant(mask, got, ref, min_code_eq=0.0 if case == "full_forget" else 0.999)
    _log(f"{case} (decay {decay}): {stats}")
    f16 = np.broadcast_to(mask, (B, H, D)).astype(bool)
    if case == "identity":
        assert np.array_equal(got[1][~f16], c.reshape(B, H, D, D)[~f16])
        assert np.array_equal(got[0][f16], h.reshape(B, H, D, D)[f16])
    if case == "full_forget":
        dl = inp.beta.reshape(B, H, 1).astype(np.float64) * inp.v.astype(np.float64)
        X = (inp.k.astype(np.float64)[:, :, :, None] * dl[:, :, None, :]).astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):   # FP16 rows carry scale 0 here
            qt = X.astype(np.float64) / ref[2].astype(np.float64)[..., None]
            tie = np.abs(np.abs(qt - np.floor(qt)) - 0.5)
        differ = (got[1] != ref[1]) & ~f16[..., None]
        assert (tie[differ] <= 1e-4).all(), "a code of the rank-one state differs away from a tie"
        assert stats["code_eq_frac"] >= 0.99


@pytest.mark.parametrize("decay", [synth.GDN, synth.KDA])
def test_window_count_out_of_range_reads_as_an_empty_window(decay):
    """A window buffer whose token count lies outside [0, W) (never zero-filled, or last used with
    another window length), the rest of it random bytes, behaves as a zero buffer: three tokens
    and a flush give the same readouts and the same pool, bit for bit."""
    B, H, D, r, W = 6, 3, 128, 24, 4
    rng, rows, mask, maskn, h, c, s = _setup(707, B, H, D, r, decay)
    pools = [DampPool(rows, h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D),
                      np.arange(B), B) for _ in range(2)]
    zero = pools[0].state.window_buffer(W)
    junk = pools[1].state.window_buffer(W)
    g = torch.Generator(device="cuda").manual_seed(708)
    junk.copy_(torch.randint(0, 256, junk.shape, generator=g, device="cuda", dtype=torch.int32).to(torch.uint8))
    words = junk.view(torch.int32).view(B * H, -1)        # one row of words per unit's buffer
    counts = [W, W + 1, 1000, -1, -5, 2 ** 31 - 1, -2 ** 31]
    words[:, 0] = torch.tensor([counts[u % len(counts)] for u in range(B * H)], dtype=torch.int32,
                               device="cuda")
    for tok in range(3):
        inp = synth.step_inputs(rng, B, H, D, decay, "bf16")
        o0 = _gpu_step(pools[0], zero, W, pools[0].slot_dev, inp)
        o1 = _gpu_step(pools[1], junk, W, pools[1].slot_dev, inp)
        assert np.array_equal(o0, o1), f"token {tok}: readouts differ"
    for p, wb in zip(pools, (zero, junk)):
        p.state.window_flush(wb, W, p.slot_dev)
    torch.cuda.synchronize()
    assert torch.equal(pools[0].state.blocks(), pools[1].state.blocks())


@pytest.mark.parametrize("W,tokens", [(4, 10), (8, 13)])
def test_scalar_gate_window_with_mixed_input_types(W, tokens):
    """One gate per unit: a key from bf16 inputs is buffered as bf16 (exact), one from fp32
    inputs as fp32; tokens alternate between the two input types within every window, so each
    window holds both formats (at W = 8 the last token's update also reads an LDS-held delta)."""
    D, r, B, H = 128, 24, 6, 3
    rng, rows, mask, maskn, h, c, s = _setup(500 + W, B, H, D, r, synth.GDN)
    win = oracle.Window(maskn, h.copy(), c.copy(), s.copy(), W)
    slots = np.random.default_rng(W).choice(2 * B, B, replace=False)
    pool = DampPool(rows, h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D), slots, 2 * B)
    wbuf = pool.state.window_buffer(W)
    for tok in range(tokens):
        dtype = "bf16" if tok % 3 != 1 else "fp32"
        inp = synth.step_inputs(rng, B, H, D, synth.GDN, dtype)
        out = _gpu_step(pool, wbuf, W, pool.slot_dev, inp)
        ref = win.step(*ref_vectors(inp, B, H, D))
        check_readout(out, ref.reshape(B, H, D))
        if (tok + 1) % W == 0:
            got = pool.logical()
            check_quant(mask, got, (win.h.reshape(B, H, D, D), win.c.reshape(B, H, D, D),
                                    win.s.reshape(B, H, D)))
            _resync(win, got)
    pool.state.window_flush(wbuf, W, pool.slot_dev)
    win.flush()
    torch.cuda.synchronize()
    check_quant(mask, pool.logical(), (win.h.reshape(B, H, D, D), win.c.reshape(B, H, D, D),
                                       win.s.reshape(B, H, D)))


def test_requests_at_different_window_positions():
    D, r, H, W = 128, 24, 3, 4
    B = 8
    rng, rows, mask, maskn, h, c, s = _setup(77, B, H, D, r, synth.GDN)
    first = np.arange(3)            # these slots run two tokens on their own first
    pool = DampPool(rows, h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D),
                    np.arange(B), B)
    wbuf = pool.state.window_buffer(W)
    nf = len(first) * H
    wa = oracle.Window(maskn[:nf], h[:nf].copy(), c[:nf].copy(), s[:nf].copy(), W)
    wb = oracle.Window(maskn[nf:], h[nf:].copy(), c[nf:].copy(), s[nf:].copy(), W)
    sub = torch.from_numpy(first.astype(np.int32)).cuda()
    for _ in range(2):
        inp = synth.step_inputs(rng, len(first), H, D, synth.GDN, "bf16")
        out = _gpu_step(pool, wbuf, W, sub, inp)
        check_readout(out, wa.step(*ref_vectors(inp, len(first), H, D)).reshape(len(first), H, D))
    na = len(first)
    for j in range(5):
        inp = synth.step_inputs(rng, B, H, D, synth.GDN, "bf16")
        out = _gpu_step(pool, wbuf, W, pool.slot_dev, inp)
        v = ref_vectors(inp, B, H, D)
        ra = wa.step(*(x[:nf] for x in v))
        rb = wb.step(*(x[nf:] for x in v))
        check_readout(out, np.concatenate([ra, rb]).reshape(B, H, D))
        # the first group's windows end after its 4th token (joint token 2), the others' after
        # joint token 4: compare there and continue from the GPU's stored state
        got = pool.logical()
        for wo, sl, ends in ((wa, slice(0, na), j == 1), (wb, slice(na, B), j == 3)):
            if ends:
                part = tuple(x[sl] for x in got)
                n_ = part[2].shape[0]
                check_quant(mask, part, (wo.h.reshape(n_, H, D, D), wo.c.reshape(n_, H, D, D),
                                         wo.s.reshape(n_, H, D)))
                _resync(wo, part)
    pool.state.window_flush(wbuf, W, pool.slot_dev)
    wa.flush()
    wb.flush()
    torch.cuda.synchronize()
    ref = tuple(np.concatenate([x, y]) for x, y in ((wa.h, wb.h), (wa.c, wb.c), (wa.s, wb.s)))
    check_quant(mask, pool.logical(), (ref[0].reshape(B, H, D, D), ref[1].reshape(B, H, D, D),
                                       ref[2].reshape(B, H, D)))


def test_window_on_per_head_layout():
    B, H, D, W = 6, 6, 128, 4
    r_per_head = np.array([0, 8, 16, 24, 32, 24], np.int32)
    rng = np.random.default_rng(21)
    row_map = np.empty((H, D), np.int32)
    for hh in range(H):
        f = np.sort(rng.choice(D, r_per_head[hh], replace=False))
        row_map[hh] = np.concatenate([f, np.setdiff1d(np.arange(D), f)])
    S = synth.normal_states(rng, (B, H, D, D), 0.1)
    mask = layout_ref.mask_per_head(r_per_head, row_map, D)
    maskn = np.broadcast_to(mask, (B, H, D)).reshape(B * H, D)
    h, c, s = oracle.quantize(maskn, S.reshape(B * H, D, D))
    st = lib.DampState(B, H, D, row_map, r_per_head=r_per_head)
    st.slots()[:] = to_dev(layout_ref.pack_per_head(r_per_head, row_map, h.reshape(B, H, D, D),
                                                    c.reshape(B, H, D, D), s.reshape(B, H, D)))
    wbuf = st.window_buffer(W)
    win = oracle.Window(maskn, h.copy(), c.copy(), s.copy(), W)
    slots = torch.arange(B, dtype=torch.int32, device="cuda")
    for tok in range(6):
        inp = synth.step_inputs(rng, B, H, D, synth.KDA, "bf16")
        q, k, v, a, b = step_tensors(inp)
        out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
        st.window_step(wbuf, W, slots, q, k, v, a, b, out)
        torch.cuda.synchronize()
        check_readout(out.cpu().numpy(), win.step(*ref_vectors(inp, B, H, D)).reshape(B, H, D))
        if tok + 1 == W:
            got = layout_ref.unpack_per_head(r_per_head, row_map, st.slots().cpu().numpy(), D)
            check_quant(mask, got, (win.h.reshape(B, H, D, D), win.c.reshape(B, H, D, D),
                                    win.s.reshape(B, H, D)))
            _resync(win, got)
    st.window_flush(wbuf, W, slots)
    win.flush()
    torch.cuda.synchronize()
    got = layout_ref.unpack_per_head(r_per_head, row_map, st.slots().cpu().numpy(), D)
    check_quant(mask, got, (win.h.reshape(B, H, D, D), win.c.reshape(B, H, D, D), win.s.reshape(B, H, D)))


def test_window_full_heads_gdn64_shape():
    """64 slots x 32 heads x 128, 24 FP16 rows, windows of 8 tokens: 12 tokens and a flush."""
    B, H, D, r, W = 64, 32, 128, 24, 8
    rng, rows, mask, maskn, h, c, s = _setup(64, B, H, D, r, synth.GDN)
    win = oracle.Window(maskn, h.copy(), c.copy(), s.copy(), W)
    pool = DampPool(rows, h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D), np.arange(B), B)
    wbuf = pool.state.window_buffer(W)
    for tok in range(12):
        inp = synth.step_inputs(rng, B, H, D, synth.GDN, "bf16")
        out = _gpu_step(pool, wbuf, W, pool.slot_dev, inp)
        check_readout(out, win.step(*ref_vectors(inp, B, H, D)).reshape(B, H, D))
        if (tok + 1) % W == 0:
            got = pool.logical()
            check_quant(mask, got, (win.h.reshape(B, H, D, D), win.c.reshape(B, H, D, D), win.s.reshape(B, H, D)))
            _resync(win, got)
    pool.state.window_flush(wbuf, W, pool.slot_dev)
    win.flush()
    torch.cuda.synchronize()
    _log(str(check_quant(mask, pool.logical(), (win.h.reshape(B, H, D, D), win.c.reshape(B, H, D, D),
                                                win.s.reshape(B, H, D)))))


def test_one_buffer_takes_a_scalar_gate_window_then_a_per_key_one():
    """A GDN window (scalar gate), a flush, then a KDA window (a gate per key row) and a flush on
    the same buffers: the flag that tells a flush which form the buffer holds is set by each
    window's own tokens and cleared when a window ends, so the second flush takes the per-row
    form. Each flush against the oracle."""
    B, H, D, r, W = 5, 3, 128, 24, 4
    rng, rows, mask, maskn, h, c, s = _setup(404, B, H, D, r, synth.GDN)
    win = oracle.Window(maskn, h.copy(), c.copy(), s.copy(), W)
    pool = DampPool(rows, h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D), np.arange(B), B)
    wbuf = pool.state.window_buffer(W)
    for decay in (synth.GDN, synth.KDA):
        print(f"window of two tokens, decay {decay}, then a flush", flush=True)
        for _ in range(2):
            inp = synth.step_inputs(rng, B, H, D, decay, "bf16")
            out = _gpu_step(pool, wbuf, W, pool.slot_dev, inp)
            check_readout(out, win.step(*ref_vectors(inp, B, H, D)).reshape(B, H, D))
        pool.state.window_flush(wbuf, W, pool.slot_dev)
        win.flush()
        torch.cuda.synchronize()
        got = pool.logical()
        check_quant(mask, got, (win.h.reshape(B, H, D, D), win.c.reshape(B, H, D, D), win.s.reshape(B, H, D)))
        _resync(win, got)
