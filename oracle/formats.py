"""Element and scale decode tables, and dequantisation of expert weights.

The FreeToken pages name the weight formats only (page "FreeToken量子化：MoE推論の
セットアップガイド", third paragraph: MXFP4, NVFP4 and BF16 checkpoints; page
"VRAM高騰時代の救世主? ...", section "FreeTokenとは何か", bullet on formats).
The bit layouts are the public specifications:

* E2M1 (OCP Microscaling Formats v1.0, element type FP4): sign bit 3, exponent
  bits 2..1 (bias 1), mantissa bit 0; exponent 0 is subnormal (0.5 * m);
  no infinities or NaN.
* E8M0 (OCP MX v1.0 scale): value 2^(e-127); code 255 is NaN.
* E4M3FN (OCP 8-bit floating point, E4M3): bias 7, subnormals m/8 * 2^-6,
  S.1111.111 is NaN, no infinities, max 448.
* MXFP4: 32 E2M1 elements share one E8M0 scale.
* NVFP4: 16 E2M1 elements share one E4M3 scale, times one fp32 per-tensor
  multiplier g.
* FP8 (page "「8GBのGPUで35Bモデルが動く」…" on the bhrtaym blog, section on
  models and quantisation formats, names FP8 without its scaling; this is
  the plainest reading): E4M3FN elements times one fp32 per-tensor
  multiplier g.

Packing (canonical layout produced by ``synth``): [rows, cols/2] bytes, element
2i in the low nibble of byte i; scales [rows, cols/B] with B = 32 or 16.
FP8: one E4M3FN code per byte, [rows, cols].
"""
from __future__ import annotations

import math

import numpy as np


def e2m1_value(code: int) -> float:
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return sign * mag


def e8m0_value(code: int) -> float:
    return math.nan if code == 255 else 2.0 ** (code - 127)


def e4m3fn_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return sign * mag


E2M1 = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E8M0 = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)
E4M3 = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def unpack_e2m1(q: np.ndarray) -> np.ndarray:
    """[rows, cols/2] packed bytes -> [rows, cols] codes (0..15)."""
    q = np.asarray(q, dtype=np.uint8)
    codes = np.empty((q.shape[0], q.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = q & 0x0F
    codes[:, 1::2] = q >> 4
    return codes


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequant(proj, fmt: str) -> np.ndarray:
    """Exact dequantised weights [rows, cols] in float64.

    MXFP4: E2M1 * E8M0.  NVFP4: (E2M1 * E4M3) * g.  FP8: E4M3 * g.  BF16:
    the bf16 value.  Every product is exact in float64."""
    if fmt == "bf16":
        return bf16_to_f64(proj.w)
    if fmt == "fp8":
        return E4M3[np.asarray(proj.q, dtype=np.uint8)] * float(np.float32(proj.g))
    vals = E2M1[unpack_e2m1(proj.q)]
    if fmt == "mxfp4":
        return vals * np.repeat(E8M0[proj.s], 32, axis=1)
    if fmt == "nvfp4":
        return (vals * np.repeat(E4M3[proj.s], 16, axis=1)) * float(np.float32(proj.g))
    raise ValueError(fmt)


def round_f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """float -> bf16 bits by round-to-nearest-even of the float32 value (finite inputs)."""
    f = np.asarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
