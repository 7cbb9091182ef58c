"""Pins the oracle's attention (decode and causal chunked prefill) to
independent implementations and closed forms.

- f16/f16 decode equals torch's scaled_dot_product_attention run in float64
  on the CPU (the llama.cpp guide's "Flash Attention" section: flash
  attention is exactly standard attention), GQA via repeat_interleave;
- quantized pairs equal the same SDPA over the dequantized cache;
- closed forms: ctx=1 gives V^_0 exactly; equal keys or Q=0 give the mean of
  V^; token order does not matter; heads of a GQA group with equal queries
  agree; query head hq reads kv head hq // G;
- causal prefill row i equals decode with ctx = p0 + i + 1;
- tiny shapes: a loop-free numpy reading of the planes (layout formula from
  the header) plus numpy softmax attention agrees to 1e-12.
"""
import itertools

import numpy as np
import pytest
import torch

PAIRS = list(itertools.product(["f16", "q8_0", "q4_0", "q5_0"], repeat=2))
# turbo3 is a values-only type
PAIRS += [(k, "turbo3") for k in ["f16", "q8_0", "q4_0", "q5_0"]]


def rand_f16(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16).view(np.uint16)


def build(orc, kt, vt, S, Hq, Hkv, D, T, rng, kscale=1.0, fill=None):
    lay = orc.OracleLayer(kt, vt, S, Hq, Hkv, D, T)
    n = T if fill is None else fill
    K = rand_f16(rng, (S, n, Hkv, D), kscale)
    V = rand_f16(rng, (S, n, Hkv, D))
    lay.append(K, V, np.zeros(S, np.int32))
    return lay, K, V


def sdpa_ref(q, Kd, Vd, ctx, scale, G):
    """q [Hq][D]; Kd, Vd [Hkv][T][D] float64 -> [Hq][D] via torch SDPA."""
    k = torch.from_numpy(Kd[:, :ctx]).repeat_interleave(G, dim=0)[None]
    v = torch.from_numpy(Vd[:, :ctx]).repeat_interleave(G, dim=0)[None]
    qq = torch.from_numpy(q)[None, :, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qq, k, v, scale=scale)[0, :, 0].numpy()


def deq_cache(lay, s, ctx):
    H = lay.shape.n_kv_heads
    K = np.stack([lay.read_rows(0, s, h, 0, ctx) for h in range(H)])
    V = np.stack([lay.read_rows(1, s, h, 0, ctx) for h in range(H)])
    return K, V


def test_f16_decode_equals_sdpa(orc):
    rng = np.random.default_rng(0)
    S, Hq, Hkv, D, T = 3, 8, 2, 64, 100
    lay, K, V = build(orc, "f16", "f16", S, Hq, Hkv, D, T, rng)
    Q = rand_f16(rng, (S, Hq, D))
    ctx = np.array([100, 1, 37], np.int32)
    out = lay.attn_decode(Q, ctx, 0.125)
    for s in range(S):
        Kd = K[s].view(np.float16).astype(np.float64).transpose(1, 0, 2)
        Vd = V[s].view(np.float16).astype(np.float64).transpose(1, 0, 2)
        q = Q[s].view(np.float16).astype(np.float64)
        ref = sdpa_ref(q, Kd, Vd, ctx[s], 0.125, Hq // Hkv)
        np.testing.assert_allclose(out[s], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kt,vt", PAIRS)
def test_quantized_decode_equals_sdpa_over_dequantized(orc, kt, vt):
    rng = np.random.default_rng(1)
    S, Hq, Hkv, D, T = 2, 4, 2, 64, 70
    lay, K, V = build(orc, kt, vt, S, Hq, Hkv, D, T, rng, kscale=3.0)
    Q = rand_f16(rng, (S, Hq, D))
    ctx = np.array([70, 33], np.int32)
    out = lay.attn_decode(Q, ctx, 0.125)
    for s in range(S):
        Kd, Vd = deq_cache(lay, s, T)
        q = Q[s].view(np.float16).astype(np.float64)
        np.testing.assert_allclose(out[s], sdpa_ref(q, Kd, Vd, ctx[s], 0.125, Hq // Hkv), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("t,typ", [(t, typ) for t in ("K", "V") for typ in ("f16", "q8_0", "q4_0", "q5_0")]
                         + [("V", "turbo3")])
def test_rows_read_back_as_their_blocks(orc, t, typ):
    """append writes each row's blocks; read_rows returns their dequantized
    values (block quantizer applied row by row, independent of layout)."""
    rng = np.random.default_rng(2)
    S, Hkv, D, T = 2, 3, 64, 40
    lay, K, V = build(orc, "q8_0" if typ == "turbo3" else typ, typ, S, 3, Hkv, D, T, rng)
    X = K if t == "K" else V
    for s in range(S):
        for h in range(Hkv):
            d, c = orc.quantize_blocks(typ, X[s, :, h, :].reshape(-1, 32))
            want = orc.dequantize_blocks(typ, d, c).reshape(T, D)
            assert (lay.read_rows(0 if t == "K" else 1, s, h, 0, T) == want).all()


def numpy_read_plane(codes, scales, typ, role, S, H, D, max_ctx):
    """Loop-free numpy reading of a plane from the header's layout formula."""
    Tc = (max_ctx + 31) // 32 * 32
    nb = D // 32
    R = {"f16": 2 * D, "q8_0": D, "q4_0": D // 2, "q5_0": D // 2, "turbo3": D // 4}[typ]
    qh = None
    if typ in ("q5_0", "turbo3"):
        # the nibble rows, then one 32-bit high-bit word per (row, block),
        # indexed like the scales
        n_rows = S * H * Tc
        qh = codes[n_rows * R:].view(np.uint32)
        codes = codes[:n_rows * R]
        qh = qh.reshape(S, H, Tc, nb) if role == "K" else \
            qh.reshape(S, H, Tc // 8, nb, 8).transpose(0, 1, 2, 4, 3).reshape(S, H, Tc, nb)
    if role == "K":
        rows = codes.reshape(S, H, Tc, R)
        sc = None if typ == "f16" else scales.reshape(S, H, Tc, nb)
    else:
        w = 2 if typ == "f16" else 1
        U = R // w
        unit = codes.view(np.uint16) if w == 2 else codes
        g = unit.reshape(S, H, Tc // 8, U, 8)
        rows = g.transpose(0, 1, 2, 4, 3).reshape(S, H, Tc, U)
        if w == 2:
            rows = rows.view(np.uint8)
        sc = None if typ == "f16" else scales.reshape(S, H, Tc // 8, nb, 8).transpose(0, 1, 2, 4, 3).reshape(S, H, Tc, nb)
    if typ == "f16":
        return rows.view(np.float16).astype(np.float64)
    d = sc.view(np.float16).astype(np.float64)
    blk = rows.reshape(S, H, Tc, nb, R // nb)
    if typ == "q8_0":
        q = blk.view(np.int8).astype(np.float64)
    elif typ == "q4_0":
        q = np.concatenate([(blk & 0xF), (blk >> 4)], axis=-1).astype(np.float64) - 8
    elif typ == "turbo3":
        # element k: 2 bits at (byte k%8, bits 2*(k//8)), third bit k of the word
        lo = np.stack([(blk[..., k % 8] >> (2 * (k // 8))) & 3 for k in range(32)], axis=-1).astype(np.int64)
        hi = (qh[..., None].astype(np.int64) >> np.arange(32)) & 1
        levels = np.array([-2.152, -1.344, -0.756, -0.2451, 0.2451, 0.756, 1.344, 2.152], np.float16)
        yh = levels.astype(np.float64)[lo | (hi << 2)] * d[..., None]
        k = np.arange(32)
        Hm = (-1.0) ** np.array([[bin(a & b).count("1") for b in k] for a in k])  # Sylvester Hadamard
        sg = np.array([-1.0 if (0x9E3779B9 >> i) & 1 else 1.0 for i in range(32)])  # rotation signs
        return ((yh @ Hm.T) * sg / 32).reshape(S, H, Tc, D)
    else:
        lo = np.concatenate([(blk & 0xF), (blk >> 4)], axis=-1).astype(np.int64)
        hi = (qh[..., None].astype(np.int64) >> np.arange(32)) & 1
        q = (lo | (hi << 4)).astype(np.float64) - 16
    return (q * d[..., None]).reshape(S, H, Tc, D)


@pytest.mark.parametrize("kt,vt", PAIRS)
@pytest.mark.parametrize("G", [1, 2])
def test_tiny_brute_force(orc, kt, vt, G):
    rng = np.random.default_rng(3 + G)
    S, Hkv, D, T = 2, 2, 32, 8
    Hq = Hkv * G
    lay, _, _ = build(orc, kt, vt, S, Hq, Hkv, D, T, rng, kscale=2.0)
    Q = rand_f16(rng, (S, Hq, D))
    for ctx in ([8, 1], [3, 8], [5, 6]):
        ctx = np.array(ctx, np.int32)
        out = lay.attn_decode(Q, ctx, 0.3)
        Kd = numpy_read_plane(lay.k_codes, lay.k_scales, kt, "K", S, Hkv, D, T)
        Vd = numpy_read_plane(lay.v_codes, lay.v_scales, vt, "V", S, Hkv, D, T)
        q = Q.view(np.float16).astype(np.float64).reshape(S, Hkv, G, D)
        sc = 0.3 * np.einsum("shgd,shtd->shgt", q, Kd)
        mask = np.arange(Kd.shape[2])[None, :] < ctx[:, None]
        sc = np.where(mask[:, None, None, :], sc, -np.inf)
        p = np.exp(sc - sc.max(-1, keepdims=True))
        p /= p.sum(-1, keepdims=True)
        ref = np.einsum("shgt,shtd->shgd", p, Vd).reshape(S, Hq, D)
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_ctx1_returns_first_value_row_exactly(orc):
    rng = np.random.default_rng(4)
    for kt, vt in PAIRS:
        lay, _, _ = build(orc, kt, vt, 1, 4, 2, 64, 32, rng, fill=5)
        Q = rand_f16(rng, (1, 4, 64))
        out = lay.attn_decode(Q, np.array([1], np.int32), 0.125)
        for hq in range(4):
            assert (out[0, hq] == lay.read_rows(1, 0, hq // 2, 0, 1)[0]).all()


def test_equal_keys_and_zero_query_give_mean(orc):
    rng = np.random.default_rng(5)
    S, Hq, Hkv, D, T = 1, 2, 1, 64, 50
    for kt, vt in PAIRS:
        lay = orc.OracleLayer(kt, vt, S, Hq, Hkv, D, T)
        krow = rand_f16(rng, (1, 1, 1, D))
        K = np.broadcast_to(krow, (S, T, Hkv, D)).copy()
        V = rand_f16(rng, (S, T, Hkv, D))
        lay.append(K, V, np.zeros(1, np.int32))
        Q = rand_f16(rng, (S, Hq, D))
        Q[0, 1] = 0
        out = lay.attn_decode(Q, np.array([T], np.int32), 0.125)
        mean = lay.read_rows(1, 0, 0, 0, T).mean(0)
        np.testing.assert_allclose(out[0, 0], mean, rtol=1e-13, atol=1e-13)
        # zero query with distinct keys
        lay2, _, _ = build(orc, kt, vt, S, Hq, Hkv, D, T, rng)
        Q2 = np.zeros((S, Hq, D), np.uint16)
        out2 = lay2.attn_decode(Q2, np.array([T], np.int32), 0.125)
        np.testing.assert_allclose(out2[0, 1], lay2.read_rows(1, 0, 0, 0, T).mean(0), rtol=1e-13, atol=1e-13)


def test_token_order_does_not_matter(orc):
    rng = np.random.default_rng(6)
    S, Hq, Hkv, D, T = 1, 4, 2, 64, 64
    K = rand_f16(rng, (S, T, Hkv, D), 2.0)
    V = rand_f16(rng, (S, T, Hkv, D))
    Q = rand_f16(rng, (S, Hq, D))
    perm = rng.permutation(T)
    for kt, vt in PAIRS:
        a = orc.OracleLayer(kt, vt, S, Hq, Hkv, D, T)
        a.append(K, V, np.zeros(1, np.int32))
        b = orc.OracleLayer(kt, vt, S, Hq, Hkv, D, T)
        for i, t in enumerate(perm):  # token i written at position perm[i]
            b.append(K[:, i:i + 1], V[:, i:i + 1], np.array([t], np.int32))
        ctx = np.array([T], np.int32)
        np.testing.assert_allclose(a.attn_decode(Q, ctx, 0.125), b.attn_decode(Q, ctx, 0.125), rtol=1e-12, atol=1e-13)


def test_gqa_mapping(orc):
    rng = np.random.default_rng(7)
    S, Hq, Hkv, D, T = 1, 8, 2, 64, 20
    G = Hq // Hkv
    K = rand_f16(rng, (S, T, Hkv, D))
    V = np.zeros((S, T, Hkv, D), np.float16)
    V[..., 0, :] = 1.0
    V[..., 1, :] = 2.0
    lay = orc.OracleLayer("q8_0", "q4_0", S, Hq, Hkv, D, T)
    lay.append(K, V.view(np.uint16), np.zeros(1, np.int32))
    Q = rand_f16(rng, (S, Hq, D))
    Q[0, 1] = Q[0, 0]
    out = lay.attn_decode(Q, np.array([T], np.int32), 0.125)
    assert (out[0, 0] == out[0, 1]).all()
    for hq in range(Hq):
        np.testing.assert_allclose(out[0, hq], hq // G + 1.0, rtol=1e-14)


@pytest.mark.parametrize("kt,vt", [("q8_0", "q4_0"), ("q4_0", "q4_0"), ("f16", "q8_0")])
def test_prefill_row_equals_decode(orc, kt, vt):
    rng = np.random.default_rng(8)
    S, Hq, Hkv, D, T, n_tok = 2, 4, 2, 64, 96, 24
    p0 = np.array([50, 72], np.int32)
    lay = orc.OracleLayer(kt, vt, S, Hq, Hkv, D, T)
    K = rand_f16(rng, (S, T, Hkv, D), 2.0)
    V = rand_f16(rng, (S, T, Hkv, D))
    lay.append(K, V, np.zeros(S, np.int32))
    Qc = rand_f16(rng, (S, n_tok, Hq, D))
    pre = lay.attn_prefill(Qc, p0, 0.125)
    for i in (0, 5, n_tok - 1):
        dec = lay.attn_decode(Qc[:, i], p0 + i + 1, 0.125)
        np.testing.assert_allclose(pre[:, i], dec, rtol=1e-14, atol=1e-14)
    # the want mask computes only the selected outputs
    want = np.zeros((S, n_tok, Hq), np.uint8)
    want[1, 3, 2] = 1
    sel = lay.attn_prefill(Qc, p0, 0.125, want=want)
    assert (sel[1, 3, 2] == pre[1, 3, 2]).all() and np.isnan(sel[0]).all()
