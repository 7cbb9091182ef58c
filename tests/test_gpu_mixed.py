"""GPU parity for caches whose precision differs per layer and for batches
whose contexts differ per sequence.

Per-layer types follow the KVSplit roadmap's separate quantization per layer:
one cache holds layers of different (K, V) type pairs, each layer is appended
and decoded through the same C-ABI calls, and each is compared with an
oracle layer of its own types.  The ragged batch mixes contexts from 1 to
32768 tokens at the Llama-3-8B decode shape, so that the automatic work split
gives sequences very different numbers of waves per (sequence, kv head)."""
import numpy as np
import pytest

import oracle
from kvq_testutil import assert_attn_close, assert_planes_equal, bits, zero_cache

pytestmark = pytest.mark.gpu


def test_per_layer_type_mix():
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    print("per-layer type mix", flush=True)
    types = [("q8_0", "q4_0"), ("f16", "f16"), ("q4_0", "q4_0"), ("q8_0", "q8_0"), ("q4_0", "f16"), ("q5_0", "q5_0"),
             ("q8_0", "turbo3")]
    S, Hq, Hkv, D, T = 2, 16, 2, 128, 300
    ctx = [300, 133]
    cache = kvq.KVCache(len(types), S, Hq, Hkv, D, T, types)
    zero_cache(cache)
    rng = np.random.default_rng(41)
    for layer, (kt, vt) in enumerate(types):
        K = torch.from_numpy((rng.standard_t(4, (S, T, Hkv, D)) * 2).astype(np.float16)).cuda()
        V = torch.from_numpy(rng.standard_normal((S, T, Hkv, D)).astype(np.float16)).cuda()
        Q = torch.from_numpy(rng.standard_normal((S, Hq, D)).astype(np.float16)).cuda()
        cache.append(layer, K, V, [0] * S)
        out = cache.decode(layer, Q, ctx, 0.0883883)
        torch.cuda.synchronize()
        orc = oracle.OracleLayer(kt, vt, S, Hq, Hkv, D, T)
        orc.append(bits(K), bits(V), np.zeros(S, np.int32))
        assert_planes_equal(cache, layer, orc)
        ref = orc.attn_decode(bits(Q), np.array(ctx, np.int32), 0.0883883)
        assert_attn_close(out.cpu().numpy(), ref, f"layer {layer} {kt}/{vt}")
        # each layer's planes have the byte size of its own types
        kc, ks, vc, vs = cache.plane_tensors(layer)
        sh = cache.shape
        assert kc.numel() == kvq.kvq_plane_bytes(sh, kt)[0] and vc.numel() == kvq.kvq_plane_bytes(sh, vt)[0]


def test_ragged_batch_full_shape():
    """Six sequences at the Llama-3-8B decode shape (32 query / 8 kv heads,
    head_dim 128, K8V4) with contexts 32768, 1, 5000, 31, 12000 and 77:
    every output against the oracle, with the automatic split and with a
    fixed split count."""
    import torch

    import mixed_precision_quantized_quantize_amd as kvq
    from mixed_precision_quantized_quantize_amd import synth

    w = synth.WORKLOADS["llama3_8b_32k"]
    ctx = [32768, 1, 5000, 31, 12000, 77]
    S = len(ctx)
    print(f"ragged batch {ctx}", flush=True)
    cache = kvq.KVCache(1, S, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, ("q8_0", "q4_0"))
    zero_cache(cache)
    orc = oracle.OracleLayer("q8_0", "q4_0", S, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx)
    for t0 in range(0, w.ctx, 4096):
        K, V = synth.kv_batch(w, 0, t0, 4096, device="cuda", seqs=range(S))
        cache.append(0, K, V, [t0] * S)
        orc.append(bits(K), bits(V), np.full(S, t0, np.int32))
        del K, V
    g = torch.Generator(device="cuda").manual_seed(7)
    Q = torch.randn((S, w.n_q_heads, w.head_dim), generator=g, device="cuda").to(torch.float16)
    ref = orc.attn_decode(bits(Q), np.array(ctx, np.int32), w.scale)
    for ns in (0, 3):
        out = cache.decode(0, Q, ctx, w.scale, n_splits=ns)
        torch.cuda.synchronize()
        print(assert_attn_close(out.cpu().numpy(), ref, f"ragged splits={ns}"), flush=True)
