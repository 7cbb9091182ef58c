"""Pins the oracle's q8_0 / q4_0 / q5_0 block quantizers to what the
definitions and the mathematics fix (the pages print no worked example of a
block; q5_0's format is not on the pages at all, so it is pinned only by
these invariants, and its parity with llama.cpp's q5_0 is unpinned):

- integer-grid blocks round-trip exactly with known codes and scales;
- brute force: each code is the nearest grid point of the stored scale
  (q8_0, ties away from zero) / the truncation rule with clamp (q4_0),
  checked in float64 against the exact binary16 scale;
- round-trip error bounds |x - x^| <= d/2 (q8_0) and <= |d| (q4_0, q5_0);
- invariants and special cases (all-zero blocks, sign ties, clamps).
"""
import numpy as np
import pytest


def f16(vals):
    return np.asarray(vals, dtype=np.float16).view(np.uint16).reshape(-1, 32)


def dval(d_bits):
    return np.asarray(d_bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def q8_codes(codes):
    return codes.view(np.int8).astype(np.int64)


def q4_codes(codes):
    lo = (codes & 0x0F).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    return np.concatenate([lo, hi], axis=1)  # element i (i<16) low nibble, i+16 high


@pytest.mark.parametrize("k", [-8, -3, 0, 2, 5])
def test_q8_0_integer_grid(orc, k):
    rng = np.random.default_rng(k + 100)
    n = rng.integers(-127, 128, size=(64, 32))
    n[:, 5] = np.where(rng.random(64) < 0.5, 127, -127)  # max |n| = 127
    x = n * 2.0**k
    d, codes = orc.quantize_blocks("q8_0", f16(x))
    assert (dval(d) == 2.0**k).all()
    assert (q8_codes(codes) == n).all()
    assert (orc.dequantize_blocks("q8_0", d, codes) == x).all()


@pytest.mark.parametrize("k", [-6, -1, 0, 3])
def test_q4_0_integer_grid(orc, k):
    rng = np.random.default_rng(k + 200)
    n = rng.integers(-7, 8, size=(64, 32))
    n[:, 9] = -8  # the signed maximum is -8*2^k  ->  d = 2^k
    x = n * 2.0**k
    d, codes = orc.quantize_blocks("q4_0", f16(x))
    assert (dval(d) == 2.0**k).all()
    assert (q4_codes(codes) == n + 8).all()
    assert (orc.dequantize_blocks("q4_0", d, codes) == x).all()
    # mirrored block: the signed max is +8*2^k -> d = -2^k, codes 8 - n
    d2, codes2 = orc.quantize_blocks("q4_0", f16(-x))
    assert (dval(d2) == -(2.0**k)).all()
    c2 = q4_codes(codes2)
    assert (c2 == np.minimum(15, n + 8)).all()  # -x/(-2^k) = n; element -8 -> 16 -> clamped


def _random_blocks(seed, n=20000):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 32)) * np.exp(rng.uniform(-2, 6, size=(n, 1)))
    x[: n // 10] *= rng.standard_t(3, size=(n // 10, 32))  # heavy tails
    x = np.clip(x, -60000, 60000)
    keep = np.abs(x).max(1) / 127 >= 2.0**-14  # binary16 scale in the normal range
    return f16(x[keep].astype(np.float16))


def test_q8_0_nearest_grid_and_bound(orc):
    xb = _random_blocks(1)
    x = xb.view(np.float16).astype(np.float64)
    d, codes = orc.quantize_blocks("q8_0", xb)
    dv = dval(d)[:, None]
    q = q8_codes(codes)
    amax = np.abs(x).max(1, keepdims=True)
    # scale: binary16 rounding of amax/127 (within half an ulp of binary16)
    rel = np.abs(dv - amax / 127) / (amax / 127)
    assert (rel <= 2.0**-11 * (1 + 1e-6)).all()
    r = x / dv
    nearest = np.sign(r) * np.floor(np.abs(r) + 0.5)  # ties away from zero
    near_tie = np.abs(np.abs(r) - np.floor(np.abs(r)) - 0.5) < 2.0**-20
    assert ((q == nearest) | near_tie).all()
    assert near_tie.sum() < 1e-3 * q.size  # exact half-way points of binary16 inputs
    assert q.min() >= -127 and q.max() <= 127
    xh = orc.dequantize_blocks("q8_0", d, codes)
    assert (np.abs(x - xh) <= dv / 2 * (1 + 2.0**-20)).all()


def test_q4_0_rule_and_bound(orc):
    xb = _random_blocks(2)
    x = xb.view(np.float16).astype(np.float64)
    d, codes = orc.quantize_blocks("q4_0", xb)
    dv = dval(d)[:, None]
    c = q4_codes(codes)
    # signed max, lowest index on ties
    idx = np.argmax(np.abs(x), axis=1)  # argmax returns the first maximum
    m = x[np.arange(len(x)), idx][:, None]
    assert (dv == m / -8).all()  # exact: |m| >= 2^-11 here
    u = x / dv + 8.5
    rule = np.clip(np.floor(u), 0, 15)
    near = np.abs(u - np.round(u)) < 2.0**-18
    assert ((c == rule) | near).all()
    # the element holding m gets code 0 and is reproduced exactly
    assert (c[np.arange(len(x)), idx] == 0).all()
    xh = orc.dequantize_blocks("q4_0", d, codes)
    err = np.abs(x - xh)
    assert (err <= np.abs(dv) * (1 + 2.0**-20)).all()
    big = err > np.abs(dv) / 2 * (1 + 2.0**-20)
    assert (c[big] == 15).all()  # beyond d/2 only where the top code clamps


def test_all_zero_blocks(orc):
    z = np.zeros((2, 32), dtype=np.float16)
    z[1] = -0.0
    d8, c8 = orc.quantize_blocks("q8_0", f16(z))
    assert (d8 == 0x0000).all() and (c8 == 0).all()
    d4, c4 = orc.quantize_blocks("q4_0", f16(z))
    assert (d4 == 0x8000).all() and (c4 == 0x88).all()  # m = +0 -> d = -0, codes 8
    assert (orc.dequantize_blocks("q4_0", d4, c4) == 0).all()


def test_q4_0_sign_tie_lowest_index(orc):
    x = np.zeros(32)
    x[3], x[7] = -5.0, 5.0
    d, _ = orc.quantize_blocks("q4_0", f16(x))
    assert dval(d)[0] == 0.625  # m = x[3] = -5
    d, _ = orc.quantize_blocks("q4_0", f16(-x))
    assert dval(d)[0] == -0.625


def test_q8_0_rounds_half_away_from_zero(orc):
    x = np.zeros(32)
    x[0] = 127 / 16  # d = 1/16
    x[1], x[2], x[3], x[4] = 2.5 / 16, -2.5 / 16, 0.5 / 16, -3.5 / 16
    d, codes = orc.quantize_blocks("q8_0", f16(x))
    assert dval(d)[0] == 1 / 16
    assert list(q8_codes(codes)[0, :5]) == [127, 3, -3, 1, -4]


def test_q8_0_subnormal_scale_clamps(orc):
    # amax/127 rounds DOWN to one binary16 ulp (2^-24): amax/d ~ 190 > 127
    x = np.zeros(32)
    x[0] = 1.49 * 127 * 2.0**-24
    x = x.astype(np.float16)
    d, codes = orc.quantize_blocks("q8_0", f16(x))
    assert d[0] == 1 and q8_codes(codes)[0, 0] == 127
    # amax so small that d underflows to zero: reciprocal 0, codes 0
    y = np.zeros(32, dtype=np.float16)
    y[0] = np.float16(2.0**-24)
    d, codes = orc.quantize_blocks("q8_0", f16(y))
    assert d[0] == 0 and (codes == 0).all()


def test_f16_blocks_are_copies(orc):
    xb = _random_blocks(3, 100)
    d, codes = orc.quantize_blocks("f16", xb)
    assert (codes.view(np.uint16) == xb).all()
    assert (orc.dequantize_blocks("f16", d, codes) == xb.view(np.float16).astype(np.float64)).all()


def q5_codes(codes):
    """Codes [n, 32] of q5_0 blocks (16 nibble bytes, then 4 bytes of high bits)."""
    lo = q4_codes(codes[:, :16])
    qh = codes[:, 16:20].copy().view("<u4").astype(np.int64)  # [n, 1]
    hi = (qh >> np.arange(32)) & 1
    return lo | (hi << 4)


@pytest.mark.parametrize("k", [-6, -1, 0, 3])
def test_q5_0_integer_grid(orc, k):
    rng = np.random.default_rng(k + 300)
    n = rng.integers(-15, 16, size=(64, 32))
    n[:, 11] = -16  # the signed maximum is -16*2^k  ->  d = 2^k
    x = n * 2.0**k
    d, codes = orc.quantize_blocks("q5_0", f16(x))
    assert (dval(d) == 2.0**k).all()
    assert (q5_codes(codes) == n + 16).all()
    assert (orc.dequantize_blocks("q5_0", d, codes) == x).all()
    # mirrored block: the signed max is +16*2^k -> d = -2^k; element -16 -> 32 -> clamped
    d2, codes2 = orc.quantize_blocks("q5_0", f16(-x))
    assert (dval(d2) == -(2.0**k)).all()
    assert (q5_codes(codes2) == np.minimum(31, n + 16)).all()


def test_q5_0_rule_and_bound(orc):
    xb = _random_blocks(4)
    x = xb.view(np.float16).astype(np.float64)
    d, codes = orc.quantize_blocks("q5_0", xb)
    dv = dval(d)[:, None]
    c = q5_codes(codes)
    idx = np.argmax(np.abs(x), axis=1)
    m = x[np.arange(len(x)), idx][:, None]
    assert (dv == m / -16).all()  # exact: |m|/16 stays in binary16's normal range here
    u = x / dv + 16.5
    rule = np.clip(np.floor(u), 0, 31)
    near = np.abs(u - np.round(u)) < 2.0**-18
    assert ((c == rule) | near).all()
    assert (c[np.arange(len(x)), idx] == 0).all()
    xh = orc.dequantize_blocks("q5_0", d, codes)
    err = np.abs(x - xh)
    assert (err <= np.abs(dv) * (1 + 2.0**-20)).all()
    big = err > np.abs(dv) / 2 * (1 + 2.0**-20)
    assert (c[big] == 31).all()
    # one more bit than q4_0 halves the typical error on the same blocks
    d4, c4 = orc.quantize_blocks("q4_0", xb)
    e4 = np.abs(x - orc.dequantize_blocks("q4_0", d4, c4))
    assert 0.4 < err.mean() / e4.mean() < 0.6


def test_q5_0_all_zero_and_sign_tie(orc):
    z = np.zeros((2, 32), dtype=np.float16)
    z[1] = -0.0
    d, c = orc.quantize_blocks("q5_0", f16(z))
    assert (d == 0x8000).all()  # m = +0 -> d = -0
    assert (c[:, :16] == 0).all() and (c[:, 16:] == 0xFF).all()  # every code is 16: nibble 0, high bit 1
    assert (orc.dequantize_blocks("q5_0", d, c) == 0).all()
    x = np.zeros(32)
    x[4], x[9] = -6.0, 6.0
    d, _ = orc.quantize_blocks("q5_0", f16(x))
    assert dval(d)[0] == 0.375  # m = x[4] = -6, the lower index
