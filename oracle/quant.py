"""MXFP4 activation quantiser (used only in the FP4-MFMA prefill mode).

The pages do not say how activations meet 4-bit weights in the expert GEMM;
the reading taken here is the OCP Microscaling Formats v1.0 conversion applied
to activations: per row, per block of 32 consecutive values along the
contraction axis,

    X = 2^(floor(log2(amax)) - emax_elem),   emax_elem = 2 for E2M1,
    element codes = E2M1 value nearest to v / X (ties to the even code),
                    saturating at +-6, sign taken from v,

with the E8M0 code of X clamped to [0, 254] and code 127 for an all-zero block.
This file writes that definition out directly: the nearest grid point is found
by comparing against all eight E2M1 magnitudes, not by thresholds.
"""
from __future__ import annotations

import math

import numpy as np

from .formats import E2M1

_GRID = E2M1[:8]  # 0, 0.5, 1, 1.5, 2, 3, 4, 6


def _nearest_e2m1(q: float) -> int:
    """Code of the E2M1 value nearest to q; ties -> even code (mantissa bit 0); saturate."""
    sign = 8 if math.copysign(1.0, q) < 0 else 0
    a = abs(q)
    d = np.abs(_GRID - a)
    best = d.min()
    cands = [c for c in range(8) if d[c] == best]
    even = [c for c in cands if c % 2 == 0]
    code = even[0] if even else cands[0]
    return sign | code


def block_exponent(amax: float) -> int:
    """floor(log2(amax)) - 2, clamped to the E8M0 range [-127, 127]; 0 for amax == 0."""
    if amax == 0.0:
        return 0
    _, e = math.frexp(amax)  # amax = f * 2^e, f in [0.5, 1)
    return max(-127, min(127, (e - 1) - 2))


def block_exponents(amax: np.ndarray) -> np.ndarray:
    """``block_exponent`` of every element of amax (int64, same shape):
    frexp gives amax = f * 2^e with f in [0.5, 1), so floor(log2 amax) = e - 1."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)
    ex = np.clip(e.astype(np.int64) - 1 - 2, -127, 127)
    return np.where(amax == 0.0, 0, ex)


def nearest_e2m1_codes(q: np.ndarray) -> np.ndarray:
    """Vectorised _nearest_e2m1: distance to each of the 8 magnitudes, minimum, ties -> even code."""
    q = np.asarray(q, dtype=np.float64)
    a = np.abs(q)
    d = np.abs(a[..., None] - _GRID)                  # [..., 8]
    is_best = d == d.min(axis=-1, keepdims=True)
    even = (np.arange(8) % 2 == 0)
    cand_even = is_best & even
    code = np.where(cand_even.any(axis=-1), cand_even.argmax(axis=-1), is_best.argmax(axis=-1))
    sign = np.where(np.signbit(q), 8, 0)
    return (code | sign).astype(np.uint8)


def quantize_mxfp4_rows(v: np.ndarray):
    """v [rows, cols] (float32 values; cols % 32 == 0) -> (codes uint8 [rows, cols], e8m0 uint8 [rows, cols/32])."""
    v = np.asarray(v, dtype=np.float32)
    rows, cols = v.shape
    assert cols % 32 == 0
    blk = v.astype(np.float64).reshape(rows, cols // 32, 32)
    amax = np.abs(blk).max(axis=-1)
    ex = block_exponents(amax)
    scales = (ex + 127).astype(np.uint8)
    scaled = np.ldexp(blk, -ex[..., None])           # exact: power-of-two scaling in float64
    codes = nearest_e2m1_codes(scaled).reshape(rows, cols)
    return codes, scales


def dequantize_mxfp4_codes(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return E2M1[codes] * np.repeat(2.0 ** (scales.astype(np.float64) - 127.0), 32, axis=1)


def quant_dequant(v: np.ndarray) -> np.ndarray:
    """float64 values of the MXFP4 encoding of float32 v [rows, cols]."""
    c, s = quantize_mxfp4_rows(v)
    return dequantize_mxfp4_codes(c, s)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """[rows, cols] codes -> [rows, cols/2] bytes, element 2i in the low nibble."""
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
