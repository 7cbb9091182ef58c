"""GPU parity at the boundary's limits: the most sequences a call takes
(KVQ_MAX_SEQS = 256, whose per-sequence contexts, positions and first waves
travel in the kernel arguments) with ragged contexts from 1 token up, and the
largest GQA group (16 query heads per kv head).  Decode (automatic and fixed
splits, so that both the uniform and the per-sequence wave maps run), the
fused append + decode, and the chunked prefill, each against the binary64
oracle."""
import numpy as np
import pytest

import oracle
from kvq_testutil import assert_attn_close, assert_planes_equal, bits, zero_cache

pytestmark = pytest.mark.gpu

S_MAX, G_MAX = 256, 16


def _inputs(rng, S, T, Hq, Hkv, D):
    import torch

    K = torch.from_numpy((rng.standard_t(4, (S, T, Hkv, D)) * 3).astype(np.float16)).cuda()
    V = torch.from_numpy(rng.standard_normal((S, T, Hkv, D)).astype(np.float16)).cuda()
    Q = torch.from_numpy(rng.standard_normal((S, Hq, D)).astype(np.float16)).cuda()
    return K, V, Q


@pytest.mark.parametrize("kt,vt", [("q8_0", "q4_0"), ("q4_0", "q5_0"), ("q8_0", "turbo3")])
def test_decode_max_sequences_max_group(kt, vt):
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    print(f"decode {S_MAX} sequences, group {G_MAX}, {kt}/{vt}", flush=True)
    rng = np.random.default_rng(71)
    S, Hkv, D, T = S_MAX, 1, 64, 96
    Hq = G_MAX * Hkv
    ctx = rng.integers(1, T + 1, S).astype(np.int32)
    ctx[0], ctx[1], ctx[-1] = 1, T, 33
    cache = kvq.KVCache(1, S, Hq, Hkv, D, T, (kt, vt))
    zero_cache(cache)
    K, V, Q = _inputs(rng, S, T, Hq, Hkv, D)
    cache.append(0, K, V, [0] * S)
    orc = oracle.OracleLayer(kt, vt, S, Hq, Hkv, D, T)
    orc.append(bits(K), bits(V), np.zeros(S, np.int32))
    assert_planes_equal(cache, 0, orc)
    ref = orc.attn_decode(bits(Q), ctx, 0.125)
    for ns in (0, 2, 7):
        out = cache.decode(0, Q, [int(c) for c in ctx], 0.125, n_splits=ns)
        torch.cuda.synchronize()
        assert_attn_close(out.cpu().numpy(), ref, f"{S} seqs {kt}/{vt} splits={ns}")


def test_decode_append_max_sequences():
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    print(f"decode_append {S_MAX} sequences", flush=True)
    rng = np.random.default_rng(72)
    S, Hkv, D, T = S_MAX, 2, 64, 70
    Hq = 8 * Hkv
    kt, vt = "q8_0", "q4_0"
    ctx = rng.integers(1, T + 1, S).astype(np.int32)
    ctx[0], ctx[1] = 1, T
    pos = ctx - 1
    K, V, Q = _inputs(rng, S, T, Hq, Hkv, D)
    Kn = torch.from_numpy((rng.standard_t(4, (S, Hkv, D)) * 3).astype(np.float16)).cuda()
    Vn = torch.from_numpy(rng.standard_normal((S, Hkv, D)).astype(np.float16)).cuda()
    two = kvq.KVCache(1, S, Hq, Hkv, D, T, (kt, vt))
    one = kvq.KVCache(1, S, Hq, Hkv, D, T, (kt, vt))
    for c in (two, one):
        zero_cache(c)
        c.append(0, K, V, [0] * S)
    two.append(0, Kn[:, None].contiguous(), Vn[:, None].contiguous(), [int(p) for p in pos])
    o2 = two.decode(0, Q, [int(c) for c in ctx], 0.125)
    o1 = one.decode_append(0, Kn, Vn, Q, [int(c) for c in ctx], 0.125)
    torch.cuda.synchronize()
    for a, b in zip(two.plane_tensors(0), one.plane_tensors(0)):
        if a is not None:
            assert torch.equal(a, b), "planes differ from append + decode"
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)), "output differs from append + decode"
    orc = oracle.OracleLayer(kt, vt, S, Hq, Hkv, D, T)
    orc.append(bits(K), bits(V), np.zeros(S, np.int32))
    orc.append(bits(Kn)[:, None], bits(Vn)[:, None], pos.astype(np.int32))
    assert_planes_equal(one, 0, orc)
    assert_attn_close(o1.cpu().numpy(), orc.attn_decode(bits(Q), ctx, 0.125), f"{S} seqs decode_append")


@pytest.mark.parametrize("kt,vt", [("q8_0", "q4_0"), ("q4_0", "turbo3")])
def test_prefill_max_sequences_max_group(kt, vt):
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    print(f"prefill {S_MAX} sequences, group {G_MAX}, {kt}/{vt}", flush=True)
    rng = np.random.default_rng(73)
    S, Hkv, D, T, n_tok = S_MAX, 1, 64, 48, 5
    Hq = G_MAX * Hkv
    q_pos0 = rng.integers(0, T - n_tok + 1, S).astype(np.int32)
    q_pos0[0], q_pos0[1] = 0, T - n_tok
    cache = kvq.KVCache(1, S, Hq, Hkv, D, T, (kt, vt))
    zero_cache(cache)
    K = torch.from_numpy((rng.standard_t(4, (S, T, Hkv, D)) * 3).astype(np.float16)).cuda()
    V = torch.from_numpy(rng.standard_normal((S, T, Hkv, D)).astype(np.float16)).cuda()
    Q = torch.from_numpy(rng.standard_normal((S, n_tok, Hq, D)).astype(np.float16)).cuda()
    cache.append(0, K, V, [0] * S)
    orc = oracle.OracleLayer(kt, vt, S, Hq, Hkv, D, T)
    orc.append(bits(K), bits(V), np.zeros(S, np.int32))
    ref = orc.attn_prefill(bits(Q), q_pos0, 0.125)
    out = cache.prefill(0, Q, [int(p) for p in q_pos0], 0.125)
    torch.cuda.synchronize()
    assert_attn_close(out.cpu().numpy(), ref, f"prefill {S} seqs {kt}/{vt}")
