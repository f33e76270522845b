"""GPU parity of the STEPQuant-style state (stq_state_*, stq_decode_step) against the oracle.

Pack fits the column scales from binary64 sums of w_i^2 X_ij^2 as the oracle does (in another
order), so from the same binary32 X they agree except where a scale's square root lies within
~1e-15 of a binary16 tie; pack starts from the caller's binary32 states and is checked byte for
byte. In the step the device's X differs from the oracle's by a few binary32 ulps (relative
~2e-7; at d = 128 it is formed as X / cs_j from the codes, with the column sums u and p taken
as exact integer sums of codes times 7-bit pieces of the row weights), and its lane sums of
(w_i X_ij)^2 are binary32 (a column scale within 5 binary32 ulps, 3e-7, of the binary64 fit of
the same values), so a column scale or a row factor whose exact value
lies that close to a binary16 tie can take either neighbour, and the row factors and codes that
follow it move with it. The step is therefore checked over every unit and every row, with each
disagreement required to be such a tie:
  FP16 pivots <= 1 ulp;
  column scales <= 1 binary16 ulp, >= 99% equal, and where they differ the oracle's
    sqrt(sum w^2 X^2 / sum w^2) (binary64, from its X) within 1e-6 (relative) of the tie between
    the two values;
  row factors against the oracle's rows fitted to the device's own column scales
    (oracle_stq_fit_rows on the oracle's binary32 X): <= 1 ulp, >= 99% equal, and where they
    differ the oracle's max_j fl32(|X_ij| / cs_j) / qmax within 1e-6 of the tie;
  codes against those rows: |delta| <= 1 everywhere and >= 99.9% equal in the rows whose row
    factor agrees (a row factor one ulp off moves X / (rf cs) by 2^-10, at most 0.13 of a code);
  against the oracle's own fit: row factors <= 2 ulps, codes |delta| <= 2;
  readout as in gpu_common; reconstruction (unpack) bit-exact.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle  # noqa: E402
import layout_ref  # noqa: E402
from gpu_common import _f16_ord, check_readout, ref_vectors, step_tensors, to_dev  # noqa: E402
from quantized_delta_rule_gdn_amd import lib, synth  # noqa: E402

TIE_REL = 1e-6   # a few binary32 ulps of X plus the step's binary32 lane sums (5 ulps), with margin


def _log(msg):
    print(msg, flush=True)


def _f16v(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _near_tie(x, a_bits, b_bits):
    """x (float64) lies within TIE_REL of the midpoint of the binary16 values a and b."""
    mid = (_f16v(a_bits) + _f16v(b_bits)) / 2
    return np.abs(x - mid) <= TIE_REL * np.abs(mid)


def check_stq_exact(got, ref):
    """Pack: the logical (h, c, rf, cs) equal byte for byte."""
    names = ("pivot values", "codes", "row factors", "column scales")
    for name, g, r in zip(names, got, ref):
        assert np.array_equal(g, r), f"{name}: {int((g != r).sum())} differ"
    return {"exact": True}


def check_stq(bits, impact, got, ref, X_ref):
    """bits, impact [H, D]; got / ref = logical (h, c, rf, cs) [n, H, ...]; X_ref the oracle's
    new states rounded to binary32 [n, H, D, D]. Every unit and row is checked (module
    docstring)."""
    hg, cg, rg, sg = got
    hr, cr, rr, sr = ref
    n, H, D, _ = cg.shape
    piv = np.broadcast_to(bits == 16, (n, H, D))
    ulp = np.abs(_f16_ord(hg[piv]) - _f16_ord(hr[piv])) if piv.any() else np.zeros(1)
    assert ulp.max() <= 1, f"pivots: {ulp.max()} ulp"
    nf = ((hg[piv] & 0x7C00) == 0x7C00) | ((hr[piv] & 0x7C00) == 0x7C00)
    assert np.array_equal(hg[piv][nf], hr[piv][nf]), "pivots: a non-finite value differs"
    dcs = np.abs(_f16_ord(sg) - _f16_ord(sr))
    cs_eq = float((dcs == 0).mean())
    assert dcs.max() <= 1 and cs_eq >= 0.99, f"column scales: max {dcs.max()}, eq {cs_eq}"
    ints = ~piv
    if not ints.any():   # every row a pivot: no codes, no row factors, the column scales are 0
        assert not sg.any() and not cg.any() and not rg.any()
        return {"cs_eq": 1.0, "rf_eq": 1.0, "code_eq": 1.0}
    X64 = X_ref.astype(np.float64)
    if (dcs > 0).any():   # each differing column scale sits at a tie of the exact value
        w = np.where(bits == 16, 0.0, impact.astype(np.float64))                 # [H, D]
        w = np.where((w ** 2).sum(axis=1, keepdims=True) > 0, w, (bits != 16).astype(np.float64))
        w2 = np.broadcast_to((w ** 2)[None, :, :, None], X64.shape)
        R = (w2 * X64 ** 2).sum(axis=2) / (w ** 2).sum(axis=1)[None, :, None]    # [n, H, D]
        d = dcs > 0
        assert _near_tie(np.sqrt(R[d]), sg[d], sr[d]).all(), "a column scale differs away from a tie"
    # the oracle's rows fitted to the device's column scales
    bb = np.broadcast_to(bits, (n, H, D)).reshape(n * H, D)
    _, cc, rc = oracle.stq_fit_rows(bb, X_ref.reshape(n * H, D, D), sg.reshape(n * H, D))
    cc, rc = cc.reshape(n, H, D, D), rc.reshape(n, H, D)
    drf_all = np.abs(_f16_ord(rg) - _f16_ord(rc))
    drf = drf_all[ints]
    rf_eq = float((drf == 0).mean())
    assert drf.max() <= 1 and rf_eq >= 0.99, f"row factors (device's column scales): max {drf.max()}, eq {rf_eq}"
    dr = (drf_all > 0) & ints
    if dr.any():   # each differing row factor sits at a tie of max fl32(|X| / cs) / qmax
        csv = _f16v(sg).astype(np.float32)                                        # [n, H, D]
        with np.errstate(divide="ignore", invalid="ignore"):
            a = np.where(csv[:, :, None, :] > 0, np.abs(X_ref) / csv[:, :, None, :], np.float32(0))
        m = a.astype(np.float32).max(axis=-1)                                      # [n, H, D]
        qm = (2.0 ** (np.broadcast_to(bits, (n, H, D)).astype(np.int64) - 1) - 1).astype(np.float32)
        q = (m / np.where(qm > 0, qm, np.float32(1))).astype(np.float64)
        assert _near_tie(q[dr], rg[dr], rc[dr]).all(), "a row factor differs away from a tie"
    m4 = np.broadcast_to(ints[..., None], cg.shape)
    dc_all = np.abs(cg.astype(np.int32) - cc.astype(np.int32))
    assert dc_all[m4].max() <= 1, f"codes (device's column scales): max {dc_all[m4].max()}"
    same = m4 & (drf_all == 0)[..., None]
    code_eq = float((dc_all[same] == 0).mean()) if same.any() else 1.0
    assert code_eq >= 0.999, f"codes (device's column scales, equal row factors): eq {code_eq}"
    # against the oracle's own fit
    assert np.abs(_f16_ord(rg) - _f16_ord(rr))[ints].max() <= 2
    assert np.abs(cg.astype(np.int32) - cr.astype(np.int32))[m4].max() <= 2
    return {"cs_eq": cs_eq, "rf_eq": rf_eq, "code_eq": code_eq,
            "units_cs_equal": float((sg == sr).all(axis=-1).mean())}


def _state(seed, n, H, D, pivots=2):
    rng = np.random.default_rng(seed)
    bits, impact = synth.stq_map(rng, H, D, pivots)
    S = synth.normal_states(rng, (n, H, D, D), 0.1)
    for h in range(H):
        S[:, h, rng.choice(D, 3, replace=False), :] *= 8
        S[:, h, :, rng.choice(D, 3, replace=False)] *= 5
    return rng, bits, impact, S


def _oracle_logical(bits, impact, S):
    n, H, D, _ = S.shape
    b = np.broadcast_to(bits, (n, H, D)).reshape(n * H, D)
    w = np.broadcast_to(impact, (n, H, D)).reshape(n * H, D)
    out = oracle.stq_quantize(b, w, S.reshape(n * H, D, D))
    return tuple(x.reshape((n, H) + x.shape[1:]) for x in out)


@pytest.mark.parametrize("D,H,n,pivots", [(128, 4, 3, 2), (64, 3, 5, 0), (128, 2, 2, 5)])
def test_pack_and_unpack(D, H, n, pivots):
    rng, bits, impact, S = _state(D + n + pivots, n, H, D, pivots)
    st = lib.StqState(2 * n, H, D, bits, impact)
    assert st.slot_bytes == sum(layout_ref.stq_block_bytes(D, bits[h]) for h in range(H))
    slots = torch.tensor(np.random.default_rng(n).choice(2 * n, n, replace=False), dtype=torch.int32, device="cuda")
    st.quantize(to_dev(S), slots)
    back = st.dequantize(slots)
    torch.cuda.synchronize()
    got = layout_ref.stq_unpack(bits, st.slots()[slots.long()].cpu().numpy(), D)
    _log(str(check_stq_exact(got, _oracle_logical(bits, impact, S))))
    # unpack reconstructs the stored bytes exactly
    b = np.broadcast_to(bits, (n, H, D)).reshape(n * H, D)
    ref = oracle.stq_dequantize(b, *(x.reshape((n * H,) + x.shape[2:]) for x in got))
    assert np.array_equal(back.cpu().numpy(), ref.reshape(n, H, D, D))


def _step_case(D, H, B, decay, dtype, pivots, seed, inplace, bits=None, impact=None):
    rng, bits0, impact0, S = _state(seed, B, H, D, pivots)
    bits = bits0 if bits is None else bits
    impact = impact0 if impact is None else impact
    num = 2 * B + 1
    st = lib.StqState(num, H, D, bits, impact)
    slots = np.random.default_rng(seed).choice(num, B, replace=False)
    sl = torch.tensor(slots, dtype=torch.int32, device="cuda")
    st.quantize(to_dev(S), sl)
    torch.cuda.synchronize()
    start = layout_ref.stq_unpack(bits, st.slots()[sl.long()].cpu().numpy(), D)   # identical input state
    inp = synth.step_inputs(rng, B, H, D, decay, dtype)
    q, k, v, a, be = step_tensors(inp)
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    before = st.pool.clone()
    dst = None if inplace else torch.zeros_like(st.pool)
    st.decode_step(sl, q, k, v, a, be, out, dst=dst)
    torch.cuda.synchronize()
    if not inplace:
        assert torch.equal(st.pool, before), "the old representation was modified"
    newp = st.pool if inplace else dst
    got = layout_ref.stq_unpack(bits, st.slots(newp)[sl.long()].cpu().numpy(), D)
    n = B * H
    bb = np.broadcast_to(bits, (B, H, D)).reshape(n, D)
    ww = np.broadcast_to(impact, (B, H, D)).reshape(n, D)
    ref_out, ref_state, X_ref = oracle.stq_step(bb, ww, *(x.reshape((n,) + x.shape[2:]) for x in start),
                                                *ref_vectors(inp, B, H, D), return_x=True)
    check_readout(out.cpu().numpy(), ref_out.reshape(B, H, D))
    return check_stq(bits, impact, got, tuple(x.reshape((B, H) + x.shape[1:]) for x in ref_state),
                     X_ref.reshape(B, H, D, D))


@pytest.mark.parametrize("D,H,B,decay,dtype,pivots,inplace", [
    (128, 4, 9, synth.KDA, "bf16", 2, True),
    (128, 3, 5, synth.KDA, "bf16", 1, False),   # the new state to a second pool
    (128, 2, 4, synth.GDN, "fp32", 0, True),
    (64, 4, 7, synth.KDA, "fp32", 3, False),
])
def test_step(D, H, B, decay, dtype, pivots, inplace):
    _log(str(_step_case(D, H, B, decay, dtype, pivots, D * 10 + B, inplace)))


def test_step_full_heads_kda():
    """64 slots x 32 KDA heads x 128 at the nominal 6-bit map (2 pivots per head)."""
    _log(str(_step_case(128, 32, 64, synth.KDA, "bf16", 2, 4242, True)))


def _edge_map(name, H, D, rng):
    """Precision maps at the edges of the layout: every kind in one row group, a single kind,
    per-head ragged counts, zero row weights."""
    impact = np.exp(rng.standard_normal((H, D))).astype(np.float32)
    bits = np.empty((H, D), np.uint8)
    for h in range(H):
        perm = rng.permutation(D)
        if name == "one_of_each":        # 1 pivot, one 8-bit and one 6-bit row, the rest 4-bit
            counts = (1, 1, 1, D - 3)
        elif name == "all16":
            counts = (D, 0, 0, 0)
        elif name == "all4":
            counts = (0, 0, 0, D)
        elif name == "many_pivots":      # more pivot rows than one 16-row step holds
            n16 = 17 + 5 * h
            counts = (n16, 13, (D - n16 - 13) // 2, D - n16 - 13 - (D - n16 - 13) // 2)
        elif name == "ragged":           # different counts in every head, none a multiple of 4
            n16 = (3 + 2 * h) % 11
            n8 = ((5 + 7 * h) % 37 + 1) * D // 128
            n6 = ((13 * h + 9) % 41 + 1) * D // 128
            counts = (n16, n8, n6, D - n16 - n8 - n6)
        else:
            raise ValueError(name)
        start = 0
        for width, c in zip((16, 8, 6, 4), counts):
            bits[h, perm[start:start + c]] = width
            start += c
    assert np.isin(bits, (16, 8, 6, 4)).all()
    if name == "ragged":
        impact[min(1, H - 1)] = 0.0      # one head with all-zero weights: the unweighted fit
    return bits, impact


@pytest.mark.parametrize("name,D,decay,inplace", [
    ("one_of_each", 128, synth.KDA, True),
    ("all16", 64, synth.GDN, True),
    ("all4", 128, synth.GDN, False),
    ("ragged", 128, synth.KDA, True),
    ("ragged", 64, synth.GDN, False),
    ("many_pivots", 128, synth.KDA, True),
])
def test_step_edge_maps(name, D, decay, inplace):
    H, B = 5, 6
    bits, impact = _edge_map(name, H, D, np.random.default_rng(len(name) + D))
    _log(f"{name} D={D}: " + str(_step_case(D, H, B, decay, "bf16", 0, 7 * D + len(name), inplace, bits, impact)))


@pytest.mark.parametrize("case", ["zero", "zero_columns", "identity", "wide_range"])
def test_step_degenerate(case):
    """Degenerate STEPQuant-style steps: a zero state with v = 0 (every stored number and the
    readout exactly 0), value columns that are zero in the state and in v (their column scales
    exactly 0 on both sides, so those columns code 0 and the row factors come from the others),
    alpha = 1 with beta = 0 (the refit of the reconstructed state), and row weights of the
    column sums gate_i rf_i k_i spread over ~5 decades (per-key gates from 1e-3 to 1, one row
    of each head 100 times the others), which the step's 7-bit pieces below the wave's largest
    weight must still carry."""
    D, H, B = 128, 4, 6
    rng, bits, impact, S = _state(91, B, H, D, 2)
    inp = synth.step_inputs(rng, B, H, D, synth.KDA, "fp32")
    zc = np.zeros(D, bool)
    if case == "zero":
        S[:] = 0.0
        inp.v[:] = 0.0
    elif case == "zero_columns":
        zc[rng.choice(D, 9, replace=False)] = True
        S[..., zc] = 0.0
        inp.v[..., zc] = 0.0
    elif case == "identity":
        inp.alpha[:] = 1.0
        inp.beta[:] = 0.0
    else:
        inp.alpha[:] = (10.0 ** rng.uniform(-3, 0, size=inp.alpha.shape)).astype(np.float32)
        for h in range(H):
            S[:, h, rng.integers(0, D), :] *= 100
    st = lib.StqState(B, H, D, bits, impact)
    sl = torch.arange(B, dtype=torch.int32, device="cuda")
    st.quantize(to_dev(S), sl)
    torch.cuda.synchronize()
    start = layout_ref.stq_unpack(bits, st.slots()[sl.long()].cpu().numpy(), D)
    q, k, v, a, be = step_tensors(inp)
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    st.decode_step(sl, q, k, v, a, be, out)
    torch.cuda.synchronize()
    got = layout_ref.stq_unpack(bits, st.slots()[sl.long()].cpu().numpy(), D)
    n = B * H
    bb = np.broadcast_to(bits, (B, H, D)).reshape(n, D)
    ww = np.broadcast_to(impact, (B, H, D)).reshape(n, D)
    ref_out, ref_state, X_ref = oracle.stq_step(bb, ww, *(x.reshape((n,) + x.shape[2:]) for x in start),
                                                *ref_vectors(inp, B, H, D), return_x=True)
    ref = tuple(x.reshape((B, H) + x.shape[1:]) for x in ref_state)
    o = out.cpu().numpy()
    check_readout(o, ref_out.reshape(B, H, D))
    stats = check_stq(bits, impact, got, ref, X_ref.reshape(B, H, D, D))
    _log(f"{case}: {stats}")
    if case == "zero":
        assert not o.any() and all(not x.any() for x in got) and all(not x.any() for x in ref)
    if case == "zero_columns":
        for x in (got[3], ref[3]):          # column scales, binary16 bits
            assert not x[..., zc].any() and x[..., ~zc].all()
        ints = np.broadcast_to(bits != 16, (B, H, D))
        assert not got[1][ints][:, zc].any(), "a code in a zero column is not 0"


def test_empty_batch_is_a_no_op():
    D, H = 128, 2
    rng, bits, impact, S = _state(3, 2, H, D)
    st = lib.StqState(2, H, D, bits, impact)
    sl = torch.arange(2, dtype=torch.int32, device="cuda")
    st.quantize(to_dev(S), sl)
    before = st.pool.clone()
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    z = torch.empty((0, H, D), dtype=torch.bfloat16, device="cuda")
    st.decode_step(e, z, z, z, torch.empty((0, H), device="cuda"), torch.empty((0, H), device="cuda"),
                   torch.empty((0, H, D), device="cuda"))
    st.quantize(torch.empty((0, H, D, D), device="cuda"), e)
    torch.cuda.synchronize()
    assert torch.equal(st.pool, before)
