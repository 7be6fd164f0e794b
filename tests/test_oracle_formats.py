"""Pins for the oracle's decode tables and dequantisation.

Independent references: the OCP MX v1.0 E2M1 table (golden fixture) and
torch's float8_e8m0fnu / float8_e4m3fn dtypes, decoded by torch itself."""
import itertools
import math

import numpy as np
import torch

import synth
from oracle import formats as F


def test_e2m1_matches_ocp_table(golden):
    rows = golden("e2m1_ocp_mx.txt")
    assert len(rows) == 16
    for r in rows:
        code, val = r.split()
        v = float(val)
        assert F.E2M1[int(code)] == v
        assert math.copysign(1.0, F.E2M1[int(code)]) == math.copysign(1.0, v)


def test_e8m0_matches_torch_exhaustive():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for c in range(256):
        if math.isnan(ref[c]):
            assert math.isnan(F.E8M0[c]) and c == 255
        else:
            assert F.E8M0[c] == ref[c], c
    assert F.E8M0[0] == 2.0 ** -127 and F.E8M0[0] > 0  # subnormal in fp32, kept


def test_e4m3fn_matches_torch_exhaustive():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        if math.isnan(ref[c]):
            assert math.isnan(F.E4M3[c])
        else:
            assert F.E4M3[c] == ref[c], c
            assert math.copysign(1, F.E4M3[c]) == math.copysign(1, ref[c])
    assert F.E4M3[0x7E] == 448.0 and F.E4M3[0x08] == 2.0 ** -6 and F.E4M3[0x01] == 2.0 ** -9


def _torch_e8m0(c):
    return torch.tensor([c], dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).item()


def _torch_e4m3(c):
    return torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).item()


def test_dequant_every_mxfp4_pair():
    # one byte holds (lo, hi); one E8M0 scale per 32 elements
    ocp = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    ocp = ocp + [-v for v in ocp]
    for s in range(255):
        q = np.array([[lo | (hi << 4) for lo, hi in itertools.product(range(16), range(16))]], np.uint8)
        q = q[:, :16]  # 32 elements: a single block
        from synth import Proj
        p = Proj(1, 32, q=q, s=np.array([[s]], np.uint8))
        got = F.dequant(p, "mxfp4")[0]
        codes = [(b & 15, b >> 4) for b in q[0]]
        exp = [v for lo, hi in codes for v in (ocp[lo], ocp[hi])]
        want = np.array(exp) * _torch_e8m0(s)
        assert np.array_equal(got, want), s


def test_dequant_every_nvfp4_pair():
    ocp = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    ocp = ocp + [-v for v in ocp]
    from synth import Proj
    g = np.float32(3.7e-5)
    codes = np.arange(16, dtype=np.uint8)
    q = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, :]  # 16 elements, element 2i low nibble
    for s in range(256):
        if s in (0x7F, 0xFF):
            continue
        p = Proj(1, 16, q=q, s=np.array([[s]], np.uint8), g=float(g))
        got = F.dequant(p, "nvfp4")[0]
        want = np.array([ocp[c] * _torch_e4m3(s) * float(g) for c in range(16)])
        assert np.array_equal(got, want), s


def test_nibble_order_low_first():
    from synth import Proj
    q = np.array([[0x72] + [0] * 15], np.uint8)  # byte 0: low nibble 2 (1.0), high nibble 7 (6.0)
    p = Proj(1, 32, q=q, s=np.array([[127]], np.uint8))
    d = F.dequant(p, "mxfp4")[0]
    assert d[0] == 1.0 and d[1] == 6.0


def test_bf16_decode_and_round():
    vals = np.array([1.0, -2.5, 3.140625, 1e-3, 65504.0], np.float32)
    bits = F.round_f32_to_bf16(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = F.bf16_to_f64(bits)
    assert np.array_equal(back, torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy())
    rnd = np.random.default_rng(3).standard_normal(10000).astype(np.float32) * 100
    assert np.array_equal(F.round_f32_to_bf16(rnd),
                          torch.from_numpy(rnd).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_dequant_every_fp8_code():
    """FP8 weights: every E4M3FN code (a [1, 256] tensor of all codes, each
    row scaled by its own per-tensor multiplier) against torch's
    float8_e4m3fn decode times g in float64: exact, NaN at 0x7F / 0xFF."""
    codes = np.arange(256, dtype=np.uint8)[None, :]
    for g in (1.0, 0.000202275623, 3.5, 2.0 ** -20):
        proj = synth.Proj(1, 256, q=codes.copy(), g=g)
        got = F.dequant(proj, "fp8")[0]
        ref = torch.from_numpy(codes[0]).view(torch.float8_e4m3fn).to(torch.float64).numpy() * float(np.float32(g))
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
        assert np.array_equal(got[~nan], ref[~nan])


def test_fp8_generator_codes_round_to_nearest():
    """The synthetic FP8 weights (input generation, gen.c) hold the E4M3 code
    nearest to w / g for each drawn w (g = amax / 448): decoding them by
    torch's float8_e4m3fn is within half a grid step of w / g."""
    ex = synth.expert("fp8", 256, 128, config=5)
    w = synth.normal_f32(0, synth.stream_id(5, 0, 0, 0), 128 * 256, 0.02).reshape(128, 256).astype(np.float64)
    q = ex.gate.q
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    v = w / float(np.float32(ex.gate.g))
    # g is rounded to float32, so |w / g| may pass 448 by a hair: the code saturates there
    assert np.abs(v).max() <= 448.0 * (1 + 2.0 ** -22)
    v = np.clip(v, -448.0, 448.0)
    # grid step of E4M3 at |v|: 2^(floor(log2 |v|) - 3), 2^-9 below 2^-6
    step = np.where(np.abs(v) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 1e-300))) - 3))
    assert np.all(np.abs(dec - v) <= step / 2 + 1e-12)
