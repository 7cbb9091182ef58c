"""Pins the oracle's IEEE 754 binary16 conversion against numpy's (an
independent implementation of the same standard, round to nearest even)."""
import numpy as np


def test_f16_to_f32_all_bit_patterns(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan].view(np.uint32) == ref[~nan].view(np.uint32)).all()  # also signs of zero


def test_f32_to_f16_exact_values_and_midpoints(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = h.view(np.float16).astype(np.float32)
    finite = np.isfinite(f)
    # every binary16 value converts back to itself
    assert (orc.f32_to_f16_bits(f[finite]) == h[finite]).all()
    # midpoints between neighbours (exact in binary32): ties go to even
    pos = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = pos.view(np.float16).astype(np.float64)
    hi = (pos + 1).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert (mid.astype(np.float64) == (lo + hi) / 2).all()
    for x in (mid, -mid):
        assert (orc.f32_to_f16_bits(x) == x.astype(np.float16).view(np.uint16)).all()


def test_f32_to_f16_random_and_edges(orc):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert (orc.f32_to_f16_bits(x) == ref).all()
    edges = np.array([65504, 65519.996, 65520, 65536, 1e30, 2.0**-14, 2.0**-24, 2.0**-25,
                      2.0**-25 * 1.0000001, 2.0**-26, 5.9604645e-08, 0.0, -0.0, 3.0e-5],
                     dtype=np.float32)
    edges = np.concatenate([edges, -edges])
    with np.errstate(over="ignore"):
        assert (orc.f32_to_f16_bits(edges) == edges.astype(np.float16).view(np.uint16)).all()


def test_f32_to_f16_infinities(orc):
    # IEEE 754: an infinite binary32 value converts to the infinity of the
    # same sign (found by the sanitized oracle run, where +inf had come back
    # as 1.0 through frexp of an infinity)
    x = np.array([np.inf, -np.inf], dtype=np.float32)
    assert (orc.f32_to_f16_bits(x) == x.astype(np.float16).view(np.uint16)).all()
