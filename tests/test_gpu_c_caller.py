"""The C ABI used from C alone: tests/c/step_from_c (built with the library) packs states and
takes one DAMP step on the GPU with no Python in its process; its readouts and stored blocks are
compared with the oracle from the identical input state (the pack is bit-exact to the oracle's
quantizer). The program runs as a child process of the test."""
import os
import subprocess

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

import oracle  # noqa: E402
import layout_ref  # noqa: E402
from gpu_common import check_quant, check_readout, ref_vectors  # noqa: E402
from quantized_delta_rule_gdn_amd import synth  # noqa: E402

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "step_from_c")


@pytest.mark.parametrize("decay", [synth.GDN, synth.KDA])
def test_step_from_a_c_program(tmp_path, decay):
    assert os.path.exists(EXE), "tests/c/step_from_c is not built: run the library build"
    num_slots, H, D, r, B = 12, 3, 128, 24, 5
    rng = np.random.default_rng(808 + decay)
    S = synth.normal_states(rng, (B, H, D, D), 0.1)
    rows = synth.random_rows(rng, H, D, r)
    inp = synth.step_inputs(rng, B, H, D, decay, "fp32")
    slots = rng.choice(num_slots, B, replace=False).astype(np.int32)
    hdr = np.array([num_slots, H, D, r, B, 1 if decay == synth.KDA else 0], np.int32)
    arrays = [hdr, rows.astype(np.int32), slots] + [np.asarray(x, np.float32) for x in
                                                     (S, inp.q, inp.k, inp.v, inp.alpha, inp.beta)]
    with open(tmp_path / "in.bin", "wb") as f:
        for a in arrays:
            f.write(np.ascontiguousarray(a).tobytes())
    print(f"C caller: decay {decay}, {B} requests x {H} heads", flush=True)
    subprocess.run([EXE, str(tmp_path / "in.bin"), str(tmp_path / "out.bin")], check=True, timeout=120)
    raw = np.fromfile(tmp_path / "out.bin", np.uint8)
    n_out = B * H * D * 4
    bb = layout_ref.block_stride(D, r)
    assert raw.size == n_out + B * H * bb
    out = raw[:n_out].view(np.float32).reshape(B, H, D)
    got = layout_ref.unpack(rows, raw[n_out:].reshape(B, H, bb), D)
    mask = synth.rows_to_mask(rows, D)
    maskn = np.broadcast_to(mask, (B, H, D)).reshape(B * H, D)
    h, c, s = oracle.quantize(maskn, S.reshape(B * H, D, D))
    ref_out = oracle.step_quant(maskn, h, c, s, *ref_vectors(inp, B, H, D))
    check_readout(out, ref_out.reshape(B, H, D))
    print(check_quant(mask, got, (h.reshape(B, H, D, D), c.reshape(B, H, D, D), s.reshape(B, H, D))),
          flush=True)
