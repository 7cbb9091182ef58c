"""GPU parity of kvq_attn_decode_append: the decode step with the new token's
quantizing append folded into the decode kernel.

Each case builds two identical caches, runs kvq_append (one row at
ctx_len-1) + kvq_attn_decode on one and kvq_attn_decode_append on the other,
and checks that
  * the planes of both caches are equal byte for byte, and equal the oracle's
    after the same appends (the row really lands at ctx_len-1, nothing else
    changes);
  * the two outputs are equal bit for bit (same quantizer, same work split);
  * the output is within the attention tolerance of the binary64 oracle.
Position ctx_len-1 holds a different row before the call, so a write that
went missing or landed elsewhere shows.  Cases cover the 16 K/V type pairs,
head_dim 64/128/256, ctx_len = 1, tile boundaries (32, 33, 64), ragged
batches and several split counts (the wave that owns the last tile differs)."""
import itertools
import zlib

import numpy as np
import pytest

import oracle
from kvq_testutil import assert_attn_close, assert_planes_equal, bits, zero_cache

pytestmark = pytest.mark.gpu

PAIRS = list(itertools.product(["f16", "q8_0", "q4_0", "q5_0"], repeat=2))
PAIRS += [(k, "turbo3") for k in ["f16", "q8_0", "q4_0", "q5_0"]]  # turbo3 stores values only


def fused_case(kt, vt, S, Hq, Hkv, D, T, ctx, splits, seed):
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    rng = np.random.default_rng(seed)
    K = torch.from_numpy((rng.standard_t(4, (S, T, Hkv, D)) * 3).astype(np.float16)).cuda()
    V = torch.from_numpy(rng.standard_normal((S, T, Hkv, D)).astype(np.float16)).cuda()
    Kn = torch.from_numpy((rng.standard_t(4, (S, Hkv, D)) * 3).astype(np.float16)).cuda()
    Vn = torch.from_numpy(rng.standard_normal((S, Hkv, D)).astype(np.float16)).cuda()
    Q = torch.from_numpy(rng.standard_normal((S, Hq, D)).astype(np.float16)).cuda()
    scale = 1.0 / np.sqrt(D)
    pos = [c - 1 for c in ctx]

    orc = oracle.OracleLayer(kt, vt, S, Hq, Hkv, D, T)
    orc.append(bits(K), bits(V), np.zeros(S, np.int32))
    orc.append(bits(Kn)[:, None], bits(Vn)[:, None], np.array(pos, np.int32))
    ref = orc.attn_decode(bits(Q), np.array(ctx, np.int32), scale)

    for ns in splits:
        what = f"{kt}/{vt} D={D} G={Hq // Hkv} ctx={ctx} splits={ns}"
        print(what, flush=True)
        two = kvq.KVCache(1, S, Hq, Hkv, D, T, (kt, vt))
        one = kvq.KVCache(1, S, Hq, Hkv, D, T, (kt, vt))
        for c in (two, one):
            zero_cache(c)
            c.append(0, K, V, [0] * S)
        two.append(0, Kn[:, None].contiguous(), Vn[:, None].contiguous(), pos)
        o2 = two.decode(0, Q, ctx, scale, n_splits=ns)
        o1 = one.decode_append(0, Kn, Vn, Q, ctx, scale, n_splits=ns)
        torch.cuda.synchronize()
        for a, b in zip(two.plane_tensors(0), one.plane_tensors(0)):
            if a is not None:
                assert torch.equal(a, b), f"{what}: planes differ from append + decode"
        assert_planes_equal(one, 0, orc)
        assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)), f"{what}: output differs from append + decode"
        assert_attn_close(o1.cpu().numpy(), ref, what)


@pytest.mark.parametrize("kt,vt", PAIRS)
def test_decode_append_pairs(kt, vt):
    fused_case(kt, vt, S=3, Hq=16, Hkv=2, D=128, T=333, ctx=[333, 33, 1], splits=[0, 1, 3],
               seed=zlib.crc32(f"da{kt}{vt}".encode()) % 1000)


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("kt,vt", [("q8_0", "q4_0"), ("f16", "q8_0"), ("q4_0", "f16"), ("q5_0", "q5_0"), ("q8_0", "turbo3"), ("q4_0", "q4_0"), ("q8_0", "q8_0")])
def test_decode_append_head_dims(kt, vt, D):
    fused_case(kt, vt, S=2, Hq=8, Hkv=2, D=D, T=200, ctx=[64, 200], splits=[0, 2, 7], seed=D)


@pytest.mark.parametrize("ctx", [[1, 1], [32, 31], [65, 2], [256, 129]])
def test_decode_append_tile_edges(ctx):
    fused_case("q8_0", "q4_0", S=2, Hq=32, Hkv=8, D=128, T=256, ctx=ctx, splits=[0, 1, 4, 256], seed=sum(ctx))


def test_decode_append_llama3_8b_32k_full_size():
    """The benchmark's step at full size (16 sequences x 32768 positions, 32
    query / 8 kv heads, head_dim 128, K8V4, automatic split): the fused call
    writes position 32767 of every sequence; planes and outputs equal those of
    kvq_append + kvq_attn_decode on a second cache, and sampled sequences
    equal the oracle."""
    import torch

    import mixed_precision_quantized_quantize_amd as kvq
    from mixed_precision_quantized_quantize_amd import synth

    w = synth.WORKLOADS["llama3_8b_32k"]
    kt, vt = w.type_pairs[0]
    S, T = w.batch, w.ctx
    print(f"decode_append {w.name} full size", flush=True)
    caches = [kvq.KVCache(1, S, w.n_q_heads, w.n_kv_heads, w.head_dim, T, (kt, vt)) for _ in range(2)]
    for c0 in range(0, T - 1, synth.CHUNK):
        n = min(synth.CHUNK, T - 1 - c0)
        K, V = synth.kv_batch(w, 0, c0, n, device="cuda")
        for c in caches:
            c.append(0, K, V, [c0] * S)
        del K, V
    Kn, Vn = synth.kv_batch(w, 0, T - 1, 1, device="cuda", step=0)
    Q = synth.queries(w, 0, device="cuda")
    ctx, pos = [T] * S, [T - 1] * S
    caches[0].append(0, Kn, Vn, pos)
    o2 = caches[0].decode(0, Q, ctx, w.scale)
    o1 = caches[1].decode_append(0, Kn[:, 0], Vn[:, 0], Q, ctx, w.scale)
    torch.cuda.synchronize()
    for a, b in zip(caches[0].plane_tensors(0), caches[1].plane_tensors(0)):
        if a is not None:
            assert torch.equal(a, b), "planes differ from append + decode"
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)), "output differs from append + decode"
    got = o1.cpu().numpy()
    del caches
    for s in (0, 11):
        orc = oracle.OracleLayer(kt, vt, 1, w.n_q_heads, w.n_kv_heads, w.head_dim, T)
        K, V = synth.kv_batch(w, 0, 0, T - 1, device="cuda", seqs=[s])
        orc.append(bits(K), bits(V), np.zeros(1, np.int32))
        del K, V
        orc.append(bits(Kn)[s:s + 1], bits(Vn)[s:s + 1], np.array([T - 1], np.int32))
        ref = orc.attn_decode(bits(Q)[s:s + 1], np.array([T], np.int32), w.scale)
        print(assert_attn_close(got[s:s + 1], ref, f"{w.name} seq {s}"), flush=True)


def test_decode_append_and_prefill_graph_replay():
    """The fused decode step and a prefill chunk captured in one HIP graph:
    every replay (with eager work and synchronizations between replays)
    equals the eager result bit for bit, and the planes stay as the eager
    calls left them (the fused append rewrites the same row each time)."""
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    print("decode_append + prefill graph replay", flush=True)
    rng = np.random.default_rng(12)
    S, Hq, Hkv, D, T = 3, 16, 4, 128, 700
    cache = kvq.KVCache(1, S, Hq, Hkv, D, T, ("q8_0", "q4_0"))
    zero_cache(cache)
    K = torch.from_numpy((rng.standard_t(4, (S, T, Hkv, D)) * 3).astype(np.float16)).cuda()
    V = torch.from_numpy(rng.standard_normal((S, T, Hkv, D)).astype(np.float16)).cuda()
    cache.append(0, K, V, [0] * S)
    Kn = torch.from_numpy((rng.standard_t(4, (S, Hkv, D)) * 3).astype(np.float16)).cuda()
    Vn = torch.from_numpy(rng.standard_normal((S, Hkv, D)).astype(np.float16)).cuda()
    Q = torch.from_numpy(rng.standard_normal((S, Hq, D)).astype(np.float16)).cuda()
    Qp = torch.from_numpy(rng.standard_normal((S, 40, Hq, D)).astype(np.float16)).cuda()
    ctx, p0 = [700, 333, 64], [100, 0, 600]
    eager_d = cache.decode_append(0, Kn, Vn, Q, ctx, 0.0883883).clone()
    eager_p = cache.prefill(0, Qp, p0, 0.0883883).clone()
    planes = [p.clone() for p in cache.plane_tensors(0) if p is not None]
    out_d = torch.empty_like(eager_d)
    out_p = torch.empty_like(eager_p)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        cache.decode_append(0, Kn, Vn, Q, ctx, 0.0883883, out=out_d)
        cache.prefill(0, Qp, p0, 0.0883883, out=out_p)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cache.decode_append(0, Kn, Vn, Q, ctx, 0.0883883, out=out_d)
        cache.prefill(0, Qp, p0, 0.0883883, out=out_p)
    for i in range(5):
        out_d.zero_()
        out_p.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_d, eager_d), f"replay {i}: decode_append"
        assert torch.equal(out_p, eager_p), f"replay {i}: prefill"
        junk = cache.decode(0, Q, [50] * S, 0.0883883, n_splits=3)  # eager work between replays
        torch.cuda.synchronize()
        del junk
    for a, b in zip([p for p in cache.plane_tensors(0) if p is not None], planes):
        assert torch.equal(a, b)
