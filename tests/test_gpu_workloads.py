"""GPU parity on the named workloads at their full sizes, from identical input states.

* gdn64:    64 slots x 32 GDN heads, d = 128; state warmed by 256 fp32 oracle steps from zero,
            24 FP16 rows per head chosen by the oracle's score, then one bf16 step; DAMP, fp32 and
            uniform INT8.
* kda256:   256 slots x 32 KDA heads with lognormal value-column multipliers, 24 FP16 rows by
            score with per-channel mean gates, 4 INT8 rows per head scaled x20; one step.
* pool4096: the benchmark's configuration: a 4,096-slot DAMP pool, 1,024 random active slots,
            one step with the benchmark's first input set, launched as the benchmark launches it
            (damp_batch_order, then the step in slot order); every active unit compared, every
            inactive block checked bit-identical. Then every slot of that pool at once (131,072
            units, the largest batch it takes): 64 sampled slots against the oracle, every unit
            against the properties a correct step leaves.
* drift:    the 64-slot state run for 2,048 steps in all three formats on the GPU; the oracle runs
            the same steps for a sample of units, and at sampled steps the GPU restarts from the
            oracle's state for one step (identical-input parity). The per-step readout error of
            the quantized formats against fp32 is reported (no page gives values to pin it).
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle  # noqa: E402
import layout_ref  # noqa: E402
from gpu_common import (SENTINEL, DampPool, check_fp32_state, check_quant, check_readout,  # noqa: E402
                        fp32_state_bound, gpu_fp32_step, gpu_int8_step, ref_vectors,
                        step_tensors, to_dev)
from quantized_delta_rule_gdn_amd import lib, synth  # noqa: E402


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def gdn64_warm():
    """Warmed fp32 state [64*32, 128, 128], per-head mean gate, FP16 rows [32, 24]."""
    w = synth.GDN64
    n = w.batch * w.heads
    S = np.zeros((n, w.d, w.d), np.float32)
    gate_sum = np.zeros(w.heads)
    for t in range(synth.GDN64_WARMUP_STEPS):
        inp = synth.gdn64_warmup(t)
        oracle.step_fp32(S, *ref_vectors(inp, w.batch, w.heads, w.d))
        gate_sum += inp.alpha.astype(np.float64).sum(axis=0)
    abar = gate_sum / (synth.GDN64_WARMUP_STEPS * w.batch)
    rows, _ = oracle.select_rows(S.reshape(w.batch, w.heads, w.d, w.d),
                                 np.repeat(abar[:, None], w.d, axis=1), w.fp16_rows)
    _log(f"gdn64 warmed: |S| mean {np.abs(S).mean():.3g}, max {np.abs(S).max():.3g}")
    return S, abar, rows


def test_gdn64_all_formats(gdn64_warm):
    S, _, rows = gdn64_warm
    w = synth.GDN64
    B, H, D = w.batch, w.heads, w.d
    inp = synth.gdn64_step()
    vecs = ref_vectors(inp, B, H, D)
    slots = np.arange(B)
    # DAMP
    mask = synth.rows_to_mask(rows, D)
    maskn = np.broadcast_to(mask, (B, H, D)).reshape(B * H, D)
    h, c, s = oracle.quantize(maskn, S)
    pool = DampPool(rows, h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D), slots, B)
    out = pool.step(inp)
    got = pool.logical()
    ref_out = oracle.step_quant(maskn, h, c, s, *vecs)
    check_readout(out, ref_out)
    _log(f"gdn64 DAMP: {check_quant(mask, got, (h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D)))}")
    # fp32
    S32 = S.copy()
    o32, Sg = gpu_fp32_step(S.reshape(B, H, D, D), inp, slots, B)
    r32 = oracle.step_fp32(S32, *vecs)
    check_readout(o32, r32)
    err = check_fp32_state(Sg.reshape(B * H, D, D), S32, fp32_state_bound(S, vecs[3], vecs[1], vecs[2], vecs[4], S32))
    _log(f"gdn64 fp32: state max abs err {err:.3g}")
    # uniform INT8
    z = np.zeros((B * H, D), np.uint8)
    hi, ci, si = oracle.quantize(z, S)
    oi, cg, sg = gpu_int8_step(ci.reshape(B, H, D, D), si.reshape(B, H, D), inp, slots, B)
    ri = oracle.step_quant(z, hi, ci, si, *vecs)
    check_readout(oi, ri)
    _log(f"gdn64 INT8: {check_quant(np.zeros((1, H, D), np.uint8), (np.zeros_like(cg, np.uint16), cg, sg), (hi.reshape(B, H, D, D), ci.reshape(B, H, D, D), si.reshape(B, H, D)))}")


def test_kda256_damp():
    w = synth.KDA256
    B, H, D, r = w.batch, w.heads, w.d, w.fp16_rows
    S0, _, inp = synth.kda256()
    # rows by score with per-channel mean gate (alpha is in original key order)
    abar = inp.alpha.astype(np.float64).mean(axis=0)          # [H, D]
    rows, _ = oracle.select_rows(S0, abar, r)
    mask = synth.rows_to_mask(rows, D)
    int8_rows = np.stack([np.flatnonzero(mask[h] == 0) for h in range(H)])
    out_rows = synth.kda256_outlier_rows(int8_rows)
    for h in range(H):
        S0[:, h, out_rows[h], :] *= np.float32(synth.KDA256_OUTLIER_GAIN)
    n = B * H
    maskn = np.broadcast_to(mask, (B, H, D)).reshape(n, D)
    h_, c, s = oracle.quantize(maskn, S0.reshape(n, D, D))
    del S0
    pool = DampPool(rows, h_.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D),
                    np.arange(B), B)
    out = pool.step(inp)
    got = pool.logical()
    ref_out = oracle.step_quant(maskn, h_, c, s, *ref_vectors(inp, B, H, D))
    check_readout(out, ref_out)
    _log(f"kda256 DAMP: {check_quant(mask, got, (h_.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D)))}")


def test_pool4096_full_size():
    """The benchmark's launch: 1,024 of 4,096 slots, 32 heads, d = 128, r = 24, bf16 inputs,
    the batch ordered by slot and the step taken in that order."""
    w = synth.POOL4096
    B, H, D, r = w.batch, w.heads, w.d, w.fp16_rows
    slots = synth.pool4096_slots()
    rows = synth.pool4096_rows()
    mask = synth.rows_to_mask(rows, D)
    st = lib.DampState(w.pool_slots, H, D, rows)
    st.pool.fill_(SENTINEL)
    blocks = st.blocks()
    inp = synth.pool4096_step(0)
    refs = []
    chunk = 128
    for i in range(0, B, chunk):   # quantize with the oracle, pack, upload, slot chunk by chunk
        S = synth.pool4096_states(i, chunk).reshape(chunk * H, D, D)
        maskn = np.broadcast_to(mask, (chunk, H, D)).reshape(chunk * H, D)
        h, c, s = oracle.quantize(maskn, S)
        del S
        blocks[torch.from_numpy(slots[i:i + chunk]).long().cuda()] = to_dev(
            layout_ref.pack(rows, h.reshape(chunk, H, D, D), c.reshape(chunk, H, D, D),
                            s.reshape(chunk, H, D)))
        refs.append((h, c, s))
    torch.cuda.synchronize()
    _log("pool4096 uploaded")
    q, k, v, a, b = step_tensors(inp)
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    slots_dev = to_dev(slots)
    st.decode_step(slots_dev, q, k, v, a, b, out, order=st.batch_order(slots_dev))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    inactive = torch.ones(w.pool_slots, dtype=torch.bool, device="cuda")
    inactive[torch.from_numpy(slots).long().cuda()] = False
    assert bool((blocks[inactive] == SENTINEL).all()), "an inactive slot was written"
    stats = []
    for j, i in enumerate(range(0, B, chunk)):
        h, c, s = refs[j]
        n = chunk * H
        maskn = np.broadcast_to(mask, (chunk, H, D)).reshape(n, D)
        vecs = tuple(x[i:i + chunk] for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta))
        ref_out = oracle.step_quant(maskn, h, c, s, *(x.reshape(n, -1) if x.ndim == 3 else x.reshape(n)
                                                       for x in vecs))
        check_readout(out[i:i + chunk], ref_out)
        got = layout_ref.unpack(rows, blocks[torch.from_numpy(slots[i:i + chunk]).long().cuda()].cpu().numpy(), D)
        stats.append(check_quant(mask, got, (h.reshape(chunk, H, D, D), c.reshape(chunk, H, D, D),
                                             s.reshape(chunk, H, D))))
    eq = min(x["code_eq_frac"] for x in stats)
    _log(f"pool4096: min code_eq_frac over chunks {eq:.6f}, max fp16 ulp "
         f"{max(x['fp16_max_ulp'] for x in stats)}, max scale rel {max(x['scale_max_rel'] for x in stats):.3g}")


def test_pool4096_every_slot_active():
    """The largest batch the benchmark's pool takes: all 4,096 slots (131,072 units) in one
    ordered launch, the slots in a seeded random order. The pool starts from random blocks made
    on the device (FP16 rows ~N(0, 0.05^2), INT8 codes uniform in [-100, 100], scales uniform in
    [1e-3, 2e-3)). 64 sampled slots are compared with the oracle element by element; every unit
    is checked for what any correct step leaves: each INT8 row with a nonzero scale holds a code
    of magnitude 127 (a block left unwritten still stops at 100), scales finite and >= 0, FP16
    rows and readouts finite."""
    w = synth.POOL4096
    n_slots, H, D, r = w.pool_slots, w.heads, w.d, w.fp16_rows
    rows = synth.pool4096_rows()
    mask = synth.rows_to_mask(rows, D)
    st = lib.DampState(n_slots, H, D, rows)
    blocks = st.blocks()
    o1, o2 = 2 * r * D, 2 * r * D + (D - r) * D
    g = torch.Generator(device="cuda").manual_seed(40960)
    blocks[:, :, :o1] = (torch.randn((n_slots, H, r * D), generator=g, device="cuda") * 0.05).half().view(torch.uint8)
    blocks[:, :, o1:o2] = torch.randint(-100, 101, (n_slots, H, (D - r) * D), generator=g, device="cuda",
                                        dtype=torch.int8).view(torch.uint8)
    blocks[:, :, o2:o2 + 4 * (D - r)] = (torch.rand((n_slots, H, D - r), generator=g, device="cuda") * 1e-3
                                         + 1e-3).view(torch.uint8)
    rng = np.random.default_rng([w.seed, 40])
    slots = rng.permutation(n_slots).astype(np.int32)
    B = n_slots
    inp = synth.step_inputs(rng, B, H, D, synth.GDN, "bf16")
    pick = np.sort(rng.choice(B, 64, replace=False))
    sel = torch.from_numpy(slots[pick]).long().cuda()
    h, c, s = layout_ref.unpack(rows, blocks[sel].cpu().numpy(), D)
    q, k, v, a, b = step_tensors(inp)
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    slots_dev = to_dev(slots)
    _log(f"pool4096, every slot: {B * H} units")
    st.decode_step(slots_dev, q, k, v, a, b, out, order=st.batch_order(slots_dev))
    torch.cuda.synchronize()

    n = len(pick) * H
    maskn = np.broadcast_to(mask, (len(pick), H, D)).reshape(n, D)
    vecs = tuple(x[pick] for x in (inp.q, inp.k, inp.v, inp.alpha, inp.beta))
    ref_out = oracle.step_quant(maskn, h.reshape(n, D, D), c.reshape(n, D, D), s.reshape(n, D),
                                *(x.reshape(n, -1) if x.ndim == 3 else x.reshape(n) for x in vecs))
    check_readout(out[torch.from_numpy(pick).long().cuda()].cpu().numpy(), ref_out)
    stats = check_quant(mask, layout_ref.unpack(rows, blocks[sel].cpu().numpy(), D), (h, c, s))

    codes = blocks[:, :, o1:o2].contiguous().view(torch.int8).view(n_slots, H, D - r, D)
    scales = blocks[:, :, o2:o2 + 4 * (D - r)].contiguous().view(torch.float32)
    f16 = blocks[:, :, :o1].contiguous().view(torch.float16)
    peak = codes.to(torch.int16).abs().amax(dim=-1)
    assert bool(torch.isfinite(scales).all()) and bool((scales >= 0).all()), "a scale is negative or not finite"
    live = scales > 0
    assert bool((peak[live] == 127).all()), \
        f"{int((peak[live] != 127).sum())} INT8 rows with a nonzero scale have no code of magnitude 127"
    assert bool((peak[~live] == 0).all()), "an INT8 row with scale 0 has a nonzero code"
    assert bool(torch.isfinite(f16).all()), "an FP16 row holds a non-finite value"
    assert bool(torch.isfinite(out).all()), "a readout is not finite"
    _log(f"pool4096, every slot: sample code_eq_frac {stats['code_eq_frac']:.6f}, "
         f"{int(live.sum())} live INT8 rows checked")


# ------------------------------------------------------------------------------------------
DRIFT_SAMPLE_SLOTS = (0, 41)        # oracle free-runs these slots' 32 heads (fp32 deviation)
DRIFT_CHECK_SLOTS = (0, 9, 17, 26, 33, 41, 50, 63)   # identical-input parity on these slots ...
DRIFT_CHECK_STEPS = (0, 700, 2047)                  # ... at these steps, in all three formats


def test_drift_2048_steps(gdn64_warm):
    """The drift workload: 2,048 steps in all three formats from gdn64's warmed state, the
    readout error of the quantized formats against the fp32 run per step, and identical-input
    parity along the way: at the check steps each format's GPU state of the check slots (8 slots
    x 32 heads) is handed to the oracle, which takes the same step; readouts, DAMP and uniform-INT8
    states (tolerances of gpu_common) and the fp32 state (its error bound) are compared."""
    S_warm, _, rows = gdn64_warm
    w = synth.DRIFT
    B, H, D, T = w.batch, w.heads, w.d, w.steps
    mask = synth.rows_to_mask(rows, D)
    maskn = np.broadcast_to(mask, (B, H, D)).reshape(B * H, D)
    z = np.zeros((B * H, D), np.uint8)
    # GPU states, all 64 slots
    h, c, s = oracle.quantize(maskn, S_warm)
    damp = DampPool(rows, h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D), np.arange(B), B)
    _, ci, si = oracle.quantize(z, S_warm)
    codes = to_dev(ci.reshape(B, H, D, D))
    scales = to_dev(si.reshape(B, H, D))
    pool32 = to_dev(S_warm.reshape(B, H, D, D))
    slot_dev = to_dev(np.arange(B, dtype=np.int32))
    # the oracle's free-running fp32 units
    sel = np.concatenate([np.arange(sl * H, (sl + 1) * H) for sl in DRIFT_SAMPLE_SLOTS])
    o_S = S_warm[sel].copy()
    chk = list(DRIFT_CHECK_SLOTS)
    csel = np.concatenate([np.arange(sl * H, (sl + 1) * H) for sl in chk])
    nc = len(chk)
    outs = {f: torch.empty((B, H, D), dtype=torch.float32, device="cuda") for f in ("f32", "q", "i8")}
    err_q, err_i, dev32, unit_q, unit_i = [], [], [], [], []
    for t in range(T):
        inp = synth.drift_step(t)
        vecs = ref_vectors(inp, B, H, D)
        check = t in DRIFT_CHECK_STEPS
        if check:   # the GPU's states of the check slots before this step
            _log(f"drift step {t}: identical-input check, three formats, {nc} slots")
            gq0 = [x[chk].reshape(nc * H, *x.shape[2:]).copy() for x in damp.logical()]
            gi0 = (codes[chk].cpu().numpy().reshape(nc * H, D, D), scales[chk].cpu().numpy().reshape(nc * H, D))
            g320 = pool32[chk].cpu().numpy().reshape(nc * H, D, D)
        # the GPU runs all units in all three formats
        q, k, v, a, b = step_tensors(inp)
        lib.fp32_decode_step(pool32, slot_dev, q, k, v, a, b, outs["f32"])
        damp.state.decode_step(slot_dev, q, k, v, a, b, outs["q"])
        lib.uniform_int8_decode_step(codes, scales, slot_dev, q, k, v, a, b, outs["i8"])
        o32 = outs["f32"].cpu().numpy().reshape(B * H, D)
        oq = outs["q"].cpu().numpy().reshape(B * H, D)
        oi = outs["i8"].cpu().numpy().reshape(B * H, D)
        if check:
            vc = tuple(x[csel] for x in vecs)
            hq, cq, sq = (x.copy() for x in gq0)
            ref_q = oracle.step_quant(maskn[csel], hq, cq, sq, *vc)
            check_readout(oq[csel], ref_q)
            got_q = [x[chk] for x in damp.logical()]
            check_quant(mask, got_q, (hq.reshape(nc, H, D, D), cq.reshape(nc, H, D, D), sq.reshape(nc, H, D)))
            hz = np.zeros((nc * H, D, D), np.uint16)
            ci0, si0 = (x.copy() for x in gi0)
            ref_i = oracle.step_quant(z[csel], hz, ci0, si0, *vc)
            check_readout(oi[csel], ref_i)
            hz = hz.reshape(nc, H, D, D)
            got_i = (hz, codes[chk].cpu().numpy(), scales[chk].cpu().numpy())
            check_quant(np.zeros((H, D), np.uint8), got_i, (hz, ci0.reshape(nc, H, D, D), si0.reshape(nc, H, D)))
            S32 = g320.copy()
            ref_32 = oracle.step_fp32(S32, *vc)
            check_readout(o32[csel], ref_32)
            check_fp32_state(pool32[chk].cpu().numpy().reshape(nc * H, D, D), S32,
                             fp32_state_bound(g320, vc[3], vc[1], vc[2], vc[4], S32))
        # advance the oracle's free-running fp32 units
        r32 = oracle.step_fp32(o_S, *(x[sel] for x in vecs))
        assert np.isfinite(oq).all() and np.isfinite(oi).all() and np.isfinite(o32).all()
        nrm = np.linalg.norm(o32)
        err_q.append(np.linalg.norm(oq - o32) / nrm)
        err_i.append(np.linalg.norm(oi - o32) / nrm)
        un = np.maximum(np.linalg.norm(o32, axis=1), 1e-30)      # per (slot, head) unit
        unit_q.append((np.linalg.norm(oq - o32, axis=1) / un).max())
        unit_i.append((np.linalg.norm(oi - o32, axis=1) / un).max())
        dev32.append(np.linalg.norm(o32[sel] - r32) / np.linalg.norm(r32))
    err_q, err_i, dev32, unit_q, unit_i = map(np.array, (err_q, err_i, dev32, unit_q, unit_i))
    _log(f"drift: DAMP rel readout err vs fp32 mean {err_q.mean():.3e} max {err_q.max():.3e}; "
         f"uniform INT8 mean {err_i.mean():.3e} max {err_i.max():.3e}; "
         f"worst unit per step: DAMP mean {unit_q.mean():.3e} max {unit_q.max():.3e}, "
         f"INT8 mean {unit_i.mean():.3e} max {unit_i.max():.3e}; "
         f"GPU fp32 vs oracle max {dev32.max():.3e}")
    out_dir = os.environ.get("DAMP_DRIFT_OUT")
    if out_dir:
        os.makedirs(out_dir, exist_ok=True)
        np.savez(os.path.join(out_dir, "drift_curves.npz"), damp=err_q, int8=err_i, fp32_dev=dev32,
                 damp_unit_max=unit_q, int8_unit_max=unit_i)
    assert dev32.max() < 1e-4          # the fp32 recurrence stays on the double-accumulated one
    assert err_q.mean() < err_i.mean()  # FP16 high-risk rows cut the INT8 drift


def test_drift_slow_gates(gdn64_warm):
    """The drift run with slow decay: gate logits ~ N(-4, 1), so alpha ~ 0.98 and a step's
    requantization error is retained for ~50 steps (the regime the DAMP page targets). GPU only,
    512 steps, three formats from the same warmed state; the FP16 rows must cut the error."""
    S_warm, _, rows = gdn64_warm
    w = synth.DRIFT
    B, H, D, T = w.batch, w.heads, w.d, 512
    mask = synth.rows_to_mask(rows, D)
    maskn = np.broadcast_to(mask, (B, H, D)).reshape(B * H, D)
    h, c, s = oracle.quantize(maskn, S_warm)
    damp = DampPool(rows, h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D), np.arange(B), B)
    _, ci, si = oracle.quantize(np.zeros((B * H, D), np.uint8), S_warm)
    codes, scales = to_dev(ci.reshape(B, H, D, D)), to_dev(si.reshape(B, H, D))
    pool32 = to_dev(S_warm.reshape(B, H, D, D))
    slot_dev = to_dev(np.arange(B, dtype=np.int32))
    outs = {f: torch.empty((B, H, D), dtype=torch.float32, device="cuda") for f in ("f32", "q", "i8")}
    err_q, err_i = [], []
    for t in range(T):
        q, k, v, a, b = step_tensors(synth.drift_step(t, gate_mean=-4.0))
        lib.fp32_decode_step(pool32, slot_dev, q, k, v, a, b, outs["f32"])
        damp.state.decode_step(slot_dev, q, k, v, a, b, outs["q"])
        lib.uniform_int8_decode_step(codes, scales, slot_dev, q, k, v, a, b, outs["i8"])
        o32, oq, oi = (outs[f].cpu().numpy().reshape(B * H, D) for f in ("f32", "q", "i8"))
        assert np.isfinite(oq).all() and np.isfinite(oi).all()
        nrm = np.linalg.norm(o32)
        err_q.append(np.linalg.norm(oq - o32) / nrm)
        err_i.append(np.linalg.norm(oi - o32) / nrm)
    err_q, err_i = np.array(err_q), np.array(err_i)
    _log(f"drift, slow gates: DAMP rel readout err vs fp32 mean {err_q.mean():.3e} max {err_q.max():.3e}; "
         f"uniform INT8 mean {err_i.mean():.3e} max {err_i.max():.3e}")
    out_dir = os.environ.get("DAMP_DRIFT_OUT")
    if out_dir:
        os.makedirs(out_dir, exist_ok=True)
        np.savez(os.path.join(out_dir, "drift_slow_curves.npz"), damp=err_q, int8=err_i)
    assert err_q.mean() < err_i.mean()
