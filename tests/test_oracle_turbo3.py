"""Pins the oracle's turbo3 values-only type (the TurboQuant page, "Benchmark
TurboQuant en Apple Silicon", section "Que es TurboQuant?": a random
Walsh-Hadamard rotation to make the data Gaussian, then an optimal scalar
quantizer at 3 bits).  The page prints no format, so only what the
mathematics fixes is pinned; parity with the TurboQuant fork is unpinned:

- the rotation is the Sylvester Hadamard matrix built from its definition,
  orthogonal up to 32, applied with the documented sign pattern;
- the codebook equals the 8-level Lloyd-Max quantizer of N(0,1) (centroid and
  midpoint conditions solved here with scipy), rounded to binary16;
- codes are the nearest level of the scaled rotated value (brute force), the
  block maximum lands on the outermost level, and the error obeys Parseval;
- the all-zero block, the byte cost and the page's KV sizes for a 70B model.
"""
import numpy as np
import pytest
from scipy.stats import norm

SIGNS = 0x9E3779B9  # the format's rotation signs: element i negated where bit i is set


def sylvester(n=32):
    k = np.arange(n)
    return np.array([[(-1) ** bin(a & b).count("1") for b in k] for a in k], dtype=np.float64)


def lloyd_max_gaussian(levels=8, iters=3000):
    L = np.linspace(-2, 2, levels)
    for _ in range(iters):
        e = np.concatenate([[-np.inf], (L[1:] + L[:-1]) / 2, [np.inf]])
        L = (norm.pdf(e[:-1]) - norm.pdf(e[1:])) / (norm.cdf(e[1:]) - norm.cdf(e[:-1]))
    return L


def signs():
    return np.array([-1.0 if (SIGNS >> i) & 1 else 1.0 for i in range(32)])


def decode_codes(codes):
    """[n, 12] turbo3 block bytes -> codes [n, 32] (0..7)."""
    lo = np.stack([(codes[:, k % 8] >> (2 * (k // 8))) & 3 for k in range(32)], axis=1).astype(np.int64)
    hi = codes[:, 8:12].copy().view("<u4").astype(np.int64)
    return lo | (((hi >> np.arange(32)) & 1) << 2)


def f16(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16).reshape(-1, 32)


def test_rotation_is_sylvester_hadamard(orc):
    H = np.stack([orc.wht32(e) for e in np.eye(32)], axis=1)  # column i = H e_i
    assert (H == sylvester()).all()
    assert (H @ H == 32 * np.eye(32)).all()


def levels_from_oracle(orc):
    """L[c] recovered through the public dequantizer: a block whose codes are all
    c and whose scale is 1 decodes to x^ = (1/32) s.(H (L[c] 1)); rotating back
    gives L[c] in every element."""
    H, s = sylvester(), signs()
    out = []
    for c in range(8):
        codes = np.zeros((1, 12), np.uint8)
        for k in range(8):
            codes[0, k] = (c & 3) * 0b01010101
        codes[0, 8:12] = 0xFF if c >> 2 else 0
        xh = orc.dequantize_blocks("turbo3", np.array([0x3C00], np.uint16), codes)[0]  # d = 1
        y = H @ (s * xh)
        assert np.allclose(y, y[0], atol=1e-12)
        out.append(y[0])
    return np.array(out)


def test_codebook_is_lloyd_max_in_binary16(orc):
    L = levels_from_oracle(orc)
    want = lloyd_max_gaussian()
    assert (L == want.astype(np.float16).astype(np.float64)).all()
    # the conditions themselves: each level is the mean of N(0,1) over its cell
    e = np.concatenate([[-np.inf], (want[1:] + want[:-1]) / 2, [np.inf]])
    cm = (norm.pdf(e[:-1]) - norm.pdf(e[1:])) / (norm.cdf(e[1:]) - norm.cdf(e[:-1]))
    assert np.abs(cm - want).max() < 1e-9
    assert np.abs(L + L[::-1]).max() == 0  # symmetric


def test_codes_are_the_nearest_level(orc):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((5000, 32)) * np.exp(rng.uniform(-4, 4, (5000, 1)))
    x[:500] *= rng.standard_t(3, size=(500, 32))
    xb = f16(x.astype(np.float16))
    xv = xb.view(np.float16).astype(np.float64)
    d, codes = orc.quantize_blocks("turbo3", xb)
    c = decode_codes(codes)
    L = lloyd_max_gaussian().astype(np.float16).astype(np.float32)
    y = (xv * signs()) @ sylvester().T  # exact in binary64 for binary16 inputs
    m = np.abs(y).max(1)
    d_want = (m.astype(np.float32) / L[7]).astype(np.float16)
    assert (d.view(np.float16) == d_want).all()
    dv = d.view(np.float16).astype(np.float32)
    idv = np.where(dv != 0, np.float32(1) / dv, np.float32(0))
    t = y.astype(np.float32) * idv[:, None]
    mids = (L[1:] + L[:-1]) / 2
    rule = (t[..., None] >= mids).sum(-1)
    assert (c == rule).all()
    # nearest level (brute force); ties are vanishingly rare and excluded
    dist = np.abs(t[..., None].astype(np.float64) - L.astype(np.float64))
    near = np.sort(dist, -1)
    unique = near[..., 1] - near[..., 0] > 1e-6
    assert (c[unique] == dist.argmin(-1)[unique]).all()
    # the block maximum maps to an outermost level
    km = np.abs(y).argmax(1)
    cm = c[np.arange(len(c)), km]
    assert ((cm == 0) | (cm == 7)).all()


def test_round_trip_error_and_parseval(orc):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3000, 32)).astype(np.float16)
    xb = f16(x)
    xv = x.astype(np.float64)
    d, codes = orc.quantize_blocks("turbo3", xb)
    xh = orc.dequantize_blocks("turbo3", d, codes)
    H, s = sylvester(), signs()
    y, yh = (xv * s) @ H.T, (xh * s) @ H.T
    # orthogonal up to sqrt(32): the error in x is the rotated-domain error / 32
    np.testing.assert_allclose(((xv - xh) ** 2).sum(1), ((y - yh) ** 2).sum(1) / 32, rtol=1e-9, atol=1e-20)
    # every rotated value lies within half the widest gap of its level (scaled)
    L = lloyd_max_gaussian().astype(np.float16).astype(np.float64)
    dv = d.view(np.float16).astype(np.float64)[:, None]
    assert (np.abs(y - yh) <= np.abs(dv) * (np.diff(L).max() / 2) * (1 + 1e-3)).all()
    # a Gaussian source at 3 bits: relative RMS error near the Lloyd-Max 0.186
    rel = np.sqrt(((xv - xh) ** 2).mean() / (xv ** 2).mean())
    assert 0.15 < rel < 0.22


def test_all_zero_block(orc):
    d, codes = orc.quantize_blocks("turbo3", np.zeros((1, 32), np.uint16))
    assert d[0] == 0 and (codes[0, :8] == 0).all() and (codes[0, 8:] == 0xFF).all()  # every code 4
    assert (orc.dequantize_blocks("turbo3", d, codes) == 0).all()


def test_turbo3_bytes_and_the_pages_70b_sizes(orc):
    """14 B per 32 values (3.5 bits).  The page prints a 32K-token KV cache of
    "~4 GB (turbo3)" and "~16 GB" at 128K for Llama-3.1-70B (80 layers, 8 kv
    heads of 128) with q8_0 keys: 4.03 GB and 16.1 GB here."""
    c, s = orc.plane_bytes("turbo3", 1, 8, 128, 32768)
    assert (c + s) * 32 == 14 * 8 * 128 * 32768
    for ctx, printed in ((32768, 4e9), (131072, 16e9)):
        kq = sum(orc.plane_bytes("q8_0", 1, 8, 128, ctx))
        vt = sum(orc.plane_bytes("turbo3", 1, 8, 128, ctx))
        total = 80 * (kq + vt)
        assert abs(total / printed - 1) < 0.05, (ctx, total)


def test_keys_reject_turbo3(orc):
    with pytest.raises(AssertionError):
        orc.OracleLayer("turbo3", "q8_0", 1, 4, 2, 64, 64)
