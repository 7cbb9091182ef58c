"""Helpers for the GPU parity tests: build the same cache through the HIP
library and through the oracle from one seeded input, and compare.

Tolerance for attention (floating point): elementwise
    |gpu - oracle| <= 2e-3 + 1e-2 * |oracle|
(max-abs 2e-3 and max-rel 1e-2 read as one allclose-style bound; the oracle
is binary64 over the same dequantized values).  Quantization is compared
bit for bit (codes and binary16 scales)."""
from __future__ import annotations

import numpy as np

ATOL, RTOL = 2e-3, 1e-2


def torch():
    import torch as t

    return t


def assert_attn_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU output"
    err = np.abs(gpu - ref)
    bound = ATOL + RTOL * np.abs(ref)
    big = np.abs(ref) >= 0.2
    rel = (err[big] / np.abs(ref[big])).max() if big.any() else 0.0
    info = f"{what}: max-abs {err.max():.3e}, max-rel(|ref|>=0.2) {rel:.3e}, worst err/bound {(err / bound).max():.3f}"
    assert (err <= bound).all(), info
    return info


def bits(t):
    """binary16 torch tensor -> numpy uint16 bits (host)."""
    return t.detach().cpu().contiguous().view(torch().int16).numpy().view(np.uint16)


def gpu_planes(cache, layer):
    kc, ks, vc, vs = cache.plane_tensors(layer)
    f = lambda x: None if x is None else x.cpu().numpy()
    return f(kc), (None if ks is None else f(ks).view(np.uint16)), f(vc), (None if vs is None else f(vs).view(np.uint16))


def zero_cache(cache):
    for bufs in cache.buffers:
        for b in bufs:
            if b is not None:
                b.zero_()


def assert_planes_equal(cache, layer, orc_layer, seq=None, n_seqs=None):
    """GPU planes of `layer` equal the oracle layer's, byte for byte.  With
    seq given, the oracle layer holds that one sequence and is compared with
    the sequence's contiguous slice of the GPU planes."""
    kc, ks, vc, vs = gpu_planes(cache, layer)
    pairs = [(kc, orc_layer.k_codes, "K codes"), (vc, orc_layer.v_codes, "V codes")]
    if ks is not None:
        pairs.append((ks, orc_layer.k_scales, "K scales"))
    if vs is not None:
        pairs.append((vs, orc_layer.v_scales, "V scales"))
    for g, o, name in pairs:
        if seq is not None:
            per = g.size // n_seqs
            g = g[seq * per:(seq + 1) * per]
        assert g.shape == o.shape, name
        bad = np.flatnonzero(g != o)
        assert bad.size == 0, f"{name}: {bad.size} of {g.size} differ, first at {bad[:8]}"
