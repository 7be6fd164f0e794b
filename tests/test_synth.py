"""Checks of the seeded input generators (not of the layer's arithmetic)."""
import numpy as np

import synth
from oracle import formats as F


def test_philox_known_answers(golden):
    for r in golden("philox_kat.txt"):
        w = [int(v, 16) for v in r.split()]
        assert synth.philox4x32_10(w[:4], w[4:6]).tolist() == w[6:10]


def test_normal_moments_and_determinism():
    z = synth.normal_f32(0, 123, 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    assert np.array_equal(z, synth.normal_f32(0, 123, 1 << 20))
    assert not np.array_equal(z[:100], synth.normal_f32(0, 124, 100))


def test_formats_encode_the_same_draws():
    H, I = 256, 128
    b = synth.expert("bf16", H, I, config=50, expert_id=3)
    m = synth.expert("mxfp4", H, I, config=50, expert_id=3)
    n = synth.expert("nvfp4", H, I, config=50, expert_id=3)
    wb = F.bf16_to_f64(b.gate.w)
    assert abs(wb.std() - 0.02) < 1e-3
    for ex in (m, n):
        wq = F.dequant(ex.gate, ex.fmt)
        rel = np.linalg.norm(wq - wb) / np.linalg.norm(wb)
        assert rel < 0.15, (ex.fmt, rel)  # 4-bit block formats on Gaussian data


def test_mxfp4_block_max_in_range():
    m = synth.expert("mxfp4", 256, 128, config=51, expert_id=0)
    raw = synth.normal_f32(0, synth.stream_id(51, 0, 0, 0), 128 * 256, 0.02).reshape(128, 256)
    amax = np.abs(raw.astype(np.float64)).reshape(128, 8, 32).max(-1)
    q = amax / 2.0 ** (m.gate.s.astype(np.float64) - 127)
    assert np.all((q >= 4) & (q < 8))


def test_workload_shapes():
    L = synth.tiny_layer()
    assert L["x"].shape == (16, 256) and L["w_router"].shape == (8, 256) and len(L["experts"]) == 8
    d = synth.decode_batch(16)
    assert d["x"].shape == (16, 2048) and d["logits"].shape == (16, 128)
    p = synth.prefill_batch(256)
    assert p["logits"].shape == (256, 128) and len(p["masked"]) == 8
    assert np.all(p["logits"][:, p["masked"]] == np.float32(-1e4))
    s = synth.stream_routing(tokens=6, layers=3)
    assert s.shape == (6, 3, 128)
