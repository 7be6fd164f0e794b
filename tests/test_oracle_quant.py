"""Pins for the oracle's MXFP4 activation quantiser."""
import math

import numpy as np

from oracle import quant as Q
from oracle.formats import E2M1


def test_hand_built_rounding_cases(golden):
    for r in golden("e2m1_rounding.txt"):
        v, code = r.split()
        assert Q._nearest_e2m1(float(v)) == int(code), v
        assert Q.nearest_e2m1_codes(np.array([float(v)]))[0] == int(code), v


def test_nearest_grid_brute_force_sweep():
    # every representable grid point and every midpoint, plus a dense sweep
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    mids = (grid[1:] + grid[:-1]) / 2
    xs = np.concatenate([np.linspace(-8, 8, 20001), grid, -grid, mids, -mids,
                         np.nextafter(mids, 0), np.nextafter(mids, 10)])
    codes = Q.nearest_e2m1_codes(xs)
    for x, c in zip(xs, codes):
        a = min(abs(x), 6.0)
        err = abs(abs(E2M1[c]) - a)
        # no grid point is strictly closer
        assert err <= np.min(np.abs(grid - a)) + 0.0
        assert (c >= 8) == bool(np.signbit(x))
    # ties land on the even-mantissa neighbour
    for m in mids:
        c = Q._nearest_e2m1(m)
        assert c % 2 == 0, m


def test_block_exponent_closed_form():
    for amax, e in [(1.0, -2), (6.0, 0), (4.0, 0), (7.99, 0), (8.0, 1), (0.5, -3), (2.0 ** -130, -127),
                    (3e38, 125), (0.0, 0)]:
        assert Q.block_exponent(amax) == e, amax


def test_quantize_idempotent_and_error_bound():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal((8, 128)) * rng.uniform(1e-3, 1e3, (8, 1))).astype(np.float32)
    c, s = Q.quantize_mxfp4_rows(v)
    d = Q.dequantize_mxfp4_codes(c, s)
    c2, s2 = Q.quantize_mxfp4_rows(d.astype(np.float32))
    assert np.array_equal(c, c2) and np.array_equal(s, s2)
    # error: at most half the local grid step (step <= 2 * scale for |q| <= 6) unless saturated
    scale = np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)
    q = v / scale
    ok = np.abs(q) <= 6
    assert np.all(np.abs(d - v)[ok] <= 1.0 * scale[ok] + 0)
    # the block max always lands in [4, 8) before rounding
    blk = np.abs(v.astype(np.float64)).reshape(8, 4, 32).max(-1)
    qb = blk / (2.0 ** (s.astype(np.float64) - 127))
    assert np.all((qb >= 4) & (qb < 8))


def test_zero_block_and_pack():
    v = np.zeros((1, 64), np.float32)
    v[0, 33] = -1.5
    c, s = Q.quantize_mxfp4_rows(v)
    assert s[0, 0] == 127 and np.all(c[0, :32] == 0)
    # -1.5 with block amax 1.5: floor(log2 1.5) - 2 = -2, so q = -1.5 / 0.25 = -6 -> code 8|7
    assert s[0, 1] == 127 - 2 and c[0, 33] == (8 | 7)
    packed = Q.pack_codes(c)
    assert packed.shape == (1, 32)
    assert packed[0, 16] == (c[0, 32] | (c[0, 33] << 4))


def test_vectorised_block_exponents_equal_the_scalar_definition():
    """block_exponents (frexp over an array) equals block_exponent element by
    element: powers of two and their neighbours, subnormals, zero, the clamp
    at both ends and a random sweep."""
    vals = [0.0, 5.877471754111438e-39, 1.401298464324817e-45, 2.0 ** -149, 2.0 ** -127, 2.0 ** 127, 3.0e38]
    for e in range(-140, 128, 3):
        p = 2.0 ** e
        vals += [p, np.nextafter(p, 0.0), np.nextafter(p, np.inf), 1.5 * p]
    vals += list(np.abs(np.random.default_rng(0).standard_normal(2000)) * 10.0 ** np.random.default_rng(1).integers(-30, 30, 2000))
    a = np.array(vals, np.float64)
    got = Q.block_exponents(a)
    want = np.array([Q.block_exponent(float(v)) for v in a])
    assert np.array_equal(got, want)
