"""GPU parity of kvq_attn_prefill_chunk (causal flash attention of a chunk of
queries over the quantized cache) against the binary64 oracle.

Small shapes cover all 16 K/V type pairs (f16, q8_0, q5_0, q4_0), head_dim 64/128/256, GQA group
sizes 1..16 (powers of two and not), chunks from 1 query to several
workgroups with a ragged last one, ragged chunk starts across the batch
(including a chunk at position 0) and cache memory past the chunk holding
NaN bit patterns.  The long-context workload (4 x 131072 tokens, K4V4, a
512-query chunk) runs at full size and is compared on sampled outputs."""
import itertools
import zlib

import numpy as np
import pytest

import oracle
from kvq_testutil import assert_attn_close, assert_planes_equal, bits, zero_cache

pytestmark = pytest.mark.gpu

PAIRS = list(itertools.product(["f16", "q8_0", "q4_0", "q5_0"], repeat=2))
PAIRS += [(k, "turbo3") for k in ["f16", "q8_0", "q4_0", "q5_0"]]  # turbo3 stores values only


def prefill_case(kt, vt, S, Hq, Hkv, D, T, n_tok, q_pos0, seed, garbage=False, kscale=3.0, scale=None):
    """Append positions 0 .. max(q_pos0)+n_tok-1 of every sequence (the rest
    of the cache zero, or all-ones bytes with garbage=True), then run the
    chunk."""
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    rng = np.random.default_rng(seed)
    cache = kvq.KVCache(1, S, Hq, Hkv, D, T, (kt, vt))
    if garbage:
        for b in cache.buffers[0]:
            if b is not None:
                b.fill_(-1)  # binary16 NaN everywhere
    else:
        zero_cache(cache)
    orc = oracle.OracleLayer(kt, vt, S, Hq, Hkv, D, T)
    end = max(q_pos0) + n_tok
    K = torch.from_numpy((rng.standard_t(4, (S, end, Hkv, D)) * kscale).astype(np.float16)).cuda()
    V = torch.from_numpy(rng.standard_normal((S, end, Hkv, D)).astype(np.float16)).cuda()
    Q = torch.from_numpy(rng.standard_normal((S, n_tok, Hq, D)).astype(np.float16)).cuda()
    # every sequence gets max(q_pos0) + n_tok rows (one append call covers
    # the batch); past that the planes keep their initial bytes
    cache.append(0, K, V, [0] * S)
    orc.append(bits(K), bits(V), np.zeros(S, np.int32))
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    ref = orc.attn_prefill(bits(Q), np.array(q_pos0, np.int32), scale)
    out = cache.prefill(0, Q, q_pos0, scale)
    torch.cuda.synchronize()
    return assert_attn_close(out.cpu().numpy(), ref, f"prefill {kt}/{vt} D={D} G={Hq // Hkv} n_tok={n_tok} p0={q_pos0}")


@pytest.mark.parametrize("kt,vt", PAIRS)
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_pairs(kt, vt, D):
    print(f"prefill parity {kt}/{vt} D={D}", flush=True)
    prefill_case(kt, vt, S=3, Hq=16, Hkv=2, D=D, T=420, n_tok=70, q_pos0=[330, 0, 151],
                 seed=zlib.crc32(f"p{kt}{vt}{D}".encode()) % 1000)


@pytest.mark.parametrize("kt,vt", PAIRS)
def test_prefill_head_dim_256(kt, vt):
    """Every pair at head_dim 256 (eight waves of one row block per
    workgroup where a half is quantized, four of two for f16/f16): group 4
    over 2 workgroups and group 8 over 5, ragged chunk starts."""
    print(f"prefill parity {kt}/{vt} D=256", flush=True)
    prefill_case(kt, vt, S=2, Hq=8, Hkv=2, D=256, T=200, n_tok=45, q_pos0=[155, 3], seed=8)
    prefill_case(kt, vt, S=2, Hq=16, Hkv=2, D=256, T=300, n_tok=70, q_pos0=[230, 61],
                 seed=zlib.crc32(f"p256{kt}{vt}".encode()) % 1000)


@pytest.mark.parametrize("G", [1, 2, 3, 5, 16])
def test_prefill_group_sizes(G):
    print(f"prefill parity G={G}", flush=True)
    prefill_case("q8_0", "q4_0", S=2, Hq=2 * G, Hkv=2, D=128, T=300, n_tok=61, q_pos0=[239, 100], seed=20 + G)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("n_tok,q_pos0", [(1, [0, 37]), (1, [299, 5]), (33, [0, 0]), (200, [0, 100]),
                                          (32, [0, 32]), (64, [0, 64]), (65, [63, 1])])
def test_prefill_chunk_shapes(n_tok, q_pos0, D):
    """Chunks of one query up to several workgroups, starting at position 0
    or mid-cache; at head_dim 64 (two 32-key tiles per step) the last step
    may end exactly at a tile or step boundary, or hold one tile wholly
    past the chunk."""
    print(f"prefill parity n_tok={n_tok} p0={q_pos0} D={D}", flush=True)
    prefill_case("q8_0", "q4_0", S=2, Hq=32, Hkv=8, D=D, T=300, n_tok=n_tok, q_pos0=q_pos0, seed=n_tok)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kt,vt", [("q8_0", "q4_0"), ("f16", "f16"), ("q4_0", "q8_0"), ("f16", "q4_0"), ("q8_0", "q5_0"), ("q8_0", "turbo3")])
def test_prefill_ignores_garbage_past_chunk(kt, vt, D):
    """Positions after the chunk's last query were never written (all bits
    set, NaN as binary16): the diagonal tiles must keep them out (at head_dim
    64, with two 32-key tiles per step, the last workgroup of sequence 0
    ends at key 199, so its last step's second tile lies wholly past it)."""
    print(f"prefill garbage past chunk {kt}/{vt} D={D}", flush=True)
    prefill_case(kt, vt, S=2, Hq=16, Hkv=2, D=D, T=512, n_tok=50, q_pos0=[150, 131], seed=3, garbage=True)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("scale", [-0.0883883, 0.0])
def test_prefill_scale_sign(scale, D):
    """A negative scale (moved onto Q by the kernel) and scale 0 (uniform
    weights over the visible keys; masked keys must still get none)."""
    print(f"prefill scale {scale} D={D}", flush=True)
    prefill_case("q8_0", "q4_0", S=2, Hq=16, Hkv=2, D=D, T=300, n_tok=40, q_pos0=[200, 9], seed=31, scale=scale)


def test_prefill_matches_decode_for_one_query():
    """A chunk of one query at position p attends to positions 0..p, the same
    as decode with ctx_len p+1 (two entry points, one definition)."""
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    print("prefill vs decode, one query", flush=True)
    rng = np.random.default_rng(12)
    S, Hq, Hkv, D, T = 2, 32, 8, 128, 700
    cache = kvq.KVCache(1, S, Hq, Hkv, D, T, ("q8_0", "q4_0"))
    zero_cache(cache)
    K = torch.from_numpy((rng.standard_normal((S, T, Hkv, D)) * 2).astype(np.float16)).cuda()
    V = torch.from_numpy(rng.standard_normal((S, T, Hkv, D)).astype(np.float16)).cuda()
    cache.append(0, K, V, [0] * S)
    Q = torch.from_numpy(rng.standard_normal((S, 1, Hq, D)).astype(np.float16)).cuda()
    pf = cache.prefill(0, Q, [699, 411], 0.0883883)[:, 0]
    dc = cache.decode(0, Q[:, 0].contiguous(), [700, 412], 0.0883883, n_splits=1)
    torch.cuda.synchronize()
    assert_attn_close(pf.cpu().numpy(), dc.cpu().numpy().astype(np.float64), "prefill vs decode")


# ---------------------------------------------------------------- full-size workload

def test_llama3_8b_128k_prefill_full_size_sampled():
    """4 sequences x 131072 positions, 32 query / 8 kv heads, K q4_0 / V q4_0:
    the last 512-query chunk (positions 130560..131071) and a first chunk at
    position 0, in the launch configuration the benchmark times; sampled
    (query, head) outputs of one sequence against the oracle."""
    import torch

    import mixed_precision_quantized_quantize_amd as kvq
    from mixed_precision_quantized_quantize_amd import synth

    w = synth.WORKLOADS["llama3_8b_128k_prefill"]
    kt, vt = w.type_pairs[0]
    n_tok = w.prefill
    print(f"prefill parity {w.name} {kt}/{vt} n_tok={n_tok}", flush=True)
    cache = kvq.KVCache(1, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, (kt, vt))
    for t0 in range(0, w.ctx, 4096):
        K, V = synth.kv_batch(w, 0, t0, 4096, device="cuda")
        cache.append(0, K, V, [t0] * w.batch)
        del K, V
    Q = synth.queries(w, 0, n_tok=n_tok, device="cuda")
    last = cache.prefill(0, Q, [w.ctx - n_tok] * w.batch, w.scale).cpu().numpy()
    first = cache.prefill(0, Q, [0] * w.batch, w.scale).cpu().numpy()
    torch.cuda.synchronize()
    s = 2
    orc = oracle.OracleLayer(kt, vt, 1, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx)
    K, V = synth.kv_batch(w, 0, 0, w.ctx, device="cuda", seqs=[s])
    orc.append(bits(K), bits(V), np.zeros(1, np.int32))
    del K, V
    assert_planes_equal(cache, 0, orc, seq=s, n_seqs=w.batch)
    toks, heads = [0, 1, 127, 128, 300, 511], [0, 3, 4, 17, 31]
    want = np.zeros((1, n_tok, w.n_q_heads), np.uint8)
    want[np.ix_([0], toks, heads)] = 1
    Qb = bits(Q)[s:s + 1]
    for name, got, p0 in (("last chunk", last, w.ctx - n_tok), ("first chunk", first, 0)):
        ref = orc.attn_prefill(Qb, np.array([p0], np.int32), w.scale, want=want)
        print(assert_attn_close(got[s][np.ix_(toks, heads)], ref[0][np.ix_(toks, heads)], f"{w.name} {name}"),
              flush=True)


def test_prefill_head_dim_64_full_size_sampled():
    """The benchmark's head_dim-64 prefill: 4 sequences x 32768 positions, 32
    query / 4 kv heads, K8V4, the last 512-query chunk, in the launch
    configuration it times; sampled (query, head) outputs of one sequence
    against the oracle."""
    import torch

    import mixed_precision_quantized_quantize_amd as kvq
    from mixed_precision_quantized_quantize_amd import synth

    D, hq, hkv, T, S, n_tok = 64, 32, 4, 32768, 4, 512
    w = synth.Workload(f"prefill_d{D}", 1, hq, hkv, D, T, S, (("q8_0", "q4_0"),), "student_t", 6000 + D,
                       prefill=n_tok)
    kt, vt = w.type_pairs[0]
    print(f"prefill parity D={D} {kt}/{vt} {S} x {n_tok} at the end of {T}", flush=True)
    cache = kvq.KVCache(1, S, hq, hkv, D, T, (kt, vt))
    for t0 in range(0, T, 4096):
        K, V = synth.kv_batch(w, 0, t0, 4096, device="cuda")
        cache.append(0, K, V, [t0] * S)
        del K, V
    Q = synth.queries(w, 0, n_tok=n_tok, device="cuda")
    got = cache.prefill(0, Q, [T - n_tok] * S, w.scale).cpu().numpy()
    torch.cuda.synchronize()
    s = 1
    orc = oracle.OracleLayer(kt, vt, 1, hq, hkv, D, T)
    K, V = synth.kv_batch(w, 0, 0, T, device="cuda", seqs=[s])
    orc.append(bits(K), bits(V), np.zeros(1, np.int32))
    del K, V
    toks, heads = [0, 1, 63, 64, 255, 256, 511], [0, 7, 8, 21, 31]
    want = np.zeros((1, n_tok, hq), np.uint8)
    want[np.ix_([0], toks, heads)] = 1
    ref = orc.attn_prefill(bits(Q)[s:s + 1], np.array([T - n_tok], np.int32), w.scale, want=want)
    print(assert_attn_close(got[s][np.ix_(toks, heads)], ref[0][np.ix_(toks, heads)], f"prefill D={D}"), flush=True)
