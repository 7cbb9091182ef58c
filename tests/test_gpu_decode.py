"""GPU parity of kvq_attn_decode (split-K flash decode + log-sum-exp merge)
against the binary64 oracle on the same inputs.

Small shapes cover all 16 K/V type pairs (f16, q8_0, q5_0, q4_0), head_dim 64/128/256, GQA group
sizes 1..16, several tiles with a ragged tail, ragged ctx_len across the
batch, ctx_len = 1 and several split counts.  The named workloads run at
their full sizes on one layer, in the launch configuration the benchmark
times (automatic split count), and are compared on sampled outputs that the
oracle computes one sequence at a time."""
import itertools
import zlib

import numpy as np
import pytest

import oracle
from kvq_testutil import assert_attn_close, assert_planes_equal, bits, zero_cache

pytestmark = pytest.mark.gpu

PAIRS = list(itertools.product(["f16", "q8_0", "q4_0", "q5_0"], repeat=2))
PAIRS += [(k, "turbo3") for k in ["f16", "q8_0", "q4_0", "q5_0"]]  # turbo3 stores values only


def small_case(kt, vt, S, Hq, Hkv, D, T, ctx, n_splits_list, seed, kscale=3.0, scale=None, q=None):
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    rng = np.random.default_rng(seed)
    cache = kvq.KVCache(1, S, Hq, Hkv, D, T, (kt, vt))
    zero_cache(cache)
    orc = oracle.OracleLayer(kt, vt, S, Hq, Hkv, D, T)
    K = torch.from_numpy((rng.standard_t(4, (S, T, Hkv, D)) * kscale).astype(np.float16)).cuda()
    V = torch.from_numpy(rng.standard_normal((S, T, Hkv, D)).astype(np.float16)).cuda()
    Q = torch.from_numpy(rng.standard_normal((S, Hq, D)).astype(np.float16) if q is None else q).cuda()
    cache.append(0, K, V, [0] * S)
    orc.append(bits(K), bits(V), np.zeros(S, np.int32))
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    ref = orc.attn_decode(bits(Q), np.array(ctx, np.int32), scale)
    for ns in n_splits_list:
        out = cache.decode(0, Q, ctx, scale, n_splits=ns)
        torch.cuda.synchronize()
        assert_attn_close(out.cpu().numpy(), ref, f"{kt}/{vt} D={D} G={Hq // Hkv} splits={ns}")


@pytest.mark.parametrize("kt,vt", PAIRS)
@pytest.mark.parametrize("D", [64, 128])
def test_decode_pairs(kt, vt, D):
    print(f"decode parity {kt}/{vt} D={D}", flush=True)
    small_case(kt, vt, S=3, Hq=16, Hkv=2, D=D, T=333, ctx=[333, 37, 1], n_splits_list=[0, 1, 3],
               seed=zlib.crc32(f"{kt}{vt}{D}".encode()) % 1000)


@pytest.mark.parametrize("kt,vt", [("q8_0", "q4_0"), ("q4_0", "q4_0"), ("q8_0", "turbo3")])
@pytest.mark.parametrize("scale", [-0.0883883, 0.0, 0.5])
def test_decode_scale_sign(kt, vt, scale):
    """The scale is used as passed: negative (the weights favour the
    smallest scores), zero (uniform weights over the first ctx_len
    positions; the tail tile's masked positions must still get none) and
    large; ragged contexts and several split counts."""
    print(f"decode scale {scale} {kt}/{vt}", flush=True)
    small_case(kt, vt, S=3, Hq=16, Hkv=2, D=128, T=333, ctx=[333, 70, 5], n_splits_list=[0, 3, 8], seed=41,
               scale=scale)


@pytest.mark.parametrize("kt,vt", [("q8_0", "q4_0"), ("q4_0", "q4_0"), ("q4_0", "q8_0"), ("q8_0", "q8_0"), ("q5_0", "q5_0"), ("q5_0", "q4_0")])
def test_decode_query_dynamic_range(kt, vt):
    """q8_0, q4_0 and q5_0 keys enter the score product as binary16
    subnormals with the codes' offset removed through the block sum of the
    query, the high nibbles' query channels are divided by 16, and q5_0's
    fifth bits meet query channels scaled by 2^-k.  Queries whose channel
    magnitudes spread log-uniformly over 2^-24 .. 2^2 (many of them binary16
    subnormals, or subnormal once divided by 16), with a head of zeros, one
    of all-tiny and one of one-signed values (a block sum as large as it
    gets), must still match the oracle."""
    print(f"decode query range {kt}/{vt}", flush=True)
    rng = np.random.default_rng(5)
    S, Hq, Hkv, D = 2, 16, 2, 128
    mag = np.exp2(rng.uniform(-24, 2, (S, Hq, D)))
    q = mag * rng.choice([-1.0, 1.0], (S, Hq, D))
    q[0, 0] = 0.0
    q[0, 1] = np.exp2(rng.uniform(-24, -14, D))
    q[1, 2] = np.abs(q[1, 2]) + 0.5
    for D_ in (64, 128):
        qq = q[:, :, :D_].astype(np.float16)
        small_case(kt, vt, S=S, Hq=Hq, Hkv=Hkv, D=D_, T=300, ctx=[300, 45], n_splits_list=[0, 3], seed=11, q=qq)


@pytest.mark.parametrize("kt,vt", [("q8_0", "q4_0"), ("f16", "f16"), ("q4_0", "q8_0"), ("q5_0", "q5_0"), ("q8_0", "q5_0"), ("q8_0", "turbo3")])
def test_decode_head_dim_256(kt, vt):
    print(f"decode parity {kt}/{vt} D=256", flush=True)
    small_case(kt, vt, S=2, Hq=8, Hkv=2, D=256, T=200, ctx=[200, 64], n_splits_list=[0, 2], seed=7)


@pytest.mark.parametrize("G", [1, 2, 5, 16])
def test_decode_group_sizes(G):
    print(f"decode parity G={G}", flush=True)
    small_case("q8_0", "q4_0", S=2, Hq=2 * G, Hkv=2, D=128, T=260, ctx=[260, 129], n_splits_list=[0, 4], seed=G)


def test_decode_many_splits_short_context():
    print("decode parity many splits", flush=True)
    small_case("q8_0", "q4_0", S=1, Hq=8, Hkv=1, D=128, T=2000, ctx=[1999], n_splits_list=[0, 63, 256], seed=11)


@pytest.mark.parametrize("kt,vt,D,T,splits", [
    # head_dim 128: up to 256 waves = 64 workgroups (slots) per pair
    ("q8_0", "q4_0", 128, 9000, [256, 200, 5, 4]),
    ("q8_0", "turbo3", 128, 9000, [256, 6]),
    # head_dim 256: 17..32 workgroups per pair, and waves without tiles
    ("q8_0", "q4_0", 256, 4096, [65, 100, 128]),
    ("q8_0", "turbo3", 256, 4096, [100]),
])
def test_decode_merge_many_slots(kt, vt, D, T, splits):
    """Many workgroups per pair: the last one to finish combines up to 64
    slots (the turbo3 rotation back on the same path); split counts that
    are not multiples of four leave waves without tiles."""
    print(f"decode merge, many slots {kt}/{vt} D={D} splits={splits}", flush=True)
    small_case(kt, vt, S=1, Hq=4, Hkv=1, D=D, T=T, ctx=[T - 5], n_splits_list=splits, seed=D + len(splits))


# ---------------------------------------------------------------- named workloads

def workload_layer(name, layer, seqs_check, heads_check, pair=None, chunk_tokens=2048):
    """Fill one layer at full size on the GPU, decode it with the automatic
    split count, and compare sampled outputs (and the sampled sequences'
    planes, bit for bit) with the oracle."""
    import torch

    import mixed_precision_quantized_quantize_amd as kvq
    from mixed_precision_quantized_quantize_amd import synth

    w = synth.WORKLOADS[name]
    kt, vt = pair or w.type_pairs[0]
    print(f"decode parity {name} layer {layer} {kt}/{vt}", flush=True)
    cache = kvq.KVCache(1, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, (kt, vt))
    for t0 in range(0, w.ctx, chunk_tokens):
        n = min(chunk_tokens, w.ctx - t0)
        K, V = synth.kv_batch(w, layer, t0, n, device="cuda")
        cache.append(0, K, V, [t0] * w.batch)
        del K, V
    Q = synth.queries(w, layer, device="cuda")
    ctx = [w.ctx] * w.batch
    out = cache.decode(0, Q, ctx, w.scale).cpu().numpy()
    torch.cuda.synchronize()
    Qb = bits(Q)
    for s in seqs_check:
        orc = oracle.OracleLayer(kt, vt, 1, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx)
        K, V = synth.kv_batch(w, layer, 0, w.ctx, device="cuda", seqs=[s])
        orc.append(bits(K), bits(V), np.zeros(1, np.int32))
        del K, V
        assert_planes_equal(cache, 0, orc, seq=s, n_seqs=w.batch)
        want = np.zeros((1, w.n_q_heads), np.uint8)
        want[0, heads_check] = 1
        ref = orc.attn_decode(Qb[s:s + 1], np.array([w.ctx], np.int32), w.scale, want=want)
        print(assert_attn_close(out[s, heads_check], ref[0, heads_check], f"{name} seq {s}"), flush=True)


def test_single_layer_2k_all_outputs():
    workload_layer("single_layer_2k", 0, [0], list(range(32)))


@pytest.mark.parametrize("pair", [("f16", "f16"), ("q8_0", "q8_0"), ("q8_0", "q4_0"), ("q4_0", "q4_0")])
def test_tinyllama_8k(pair):
    workload_layer("tinyllama_8k", 21, [0], list(range(32)), pair=pair)


def test_llama3_8b_32k_full_size_sampled():
    workload_layer("llama3_8b_32k", 0, [0, 13], [0, 7, 8, 31])


def test_llama31_70b_32k_full_size_all_heads():
    """The one sequence of the 70B-shaped layer, every one of its 64 query
    heads (its many waves per pair exercise the merge's larger paths)."""
    workload_layer("llama31_70b_32k", 0, [0], list(range(64)))


def test_llama31_70b_32k_turbo3_full_size_all_heads():
    """The TurboQuant page's configuration: Llama-3.1-70B shape at 32K tokens,
    keys q8_0, values turbo3; all 64 query heads."""
    workload_layer("llama31_70b_32k", 0, [0], list(range(64)), pair=("q8_0", "turbo3"))


def test_llama3_8b_128k_decode_full_size_all_heads():
    """K4V4 decode at 131072 tokens: every query head of one sequence."""
    workload_layer("llama3_8b_128k_prefill", 0, [3], list(range(32)))


# ---------------------------------------------------------------- merge and graph replay

def _decode_setup(S=4, Hq=32, Hkv=8, D=128, T=4096, seed=5):
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    rng = np.random.default_rng(seed)
    cache = kvq.KVCache(1, S, Hq, Hkv, D, T, ("q8_0", "q4_0"))
    K = torch.from_numpy((rng.standard_t(4, (S, T, Hkv, D)) * 3).astype(np.float16)).cuda()
    V = torch.from_numpy(rng.standard_normal((S, T, Hkv, D)).astype(np.float16)).cuda()
    Q = torch.from_numpy(rng.standard_normal((S, Hq, D)).astype(np.float16)).cuda()
    cache.append(0, K, V, [0] * S)
    return cache, K, V, Q


def test_decode_merge_is_repeatable():
    """Waves write one partial per (sequence, kv head) they touch and the
    merge kernel combines them in a fixed order: results are bitwise equal
    across calls, also interleaved with calls that split the work
    differently."""
    import torch

    print("decode merge repeatability", flush=True)
    cache, K, V, Q = _decode_setup()
    ctx = [4096, 4000, 3001, 77]
    ref = {ns: cache.decode(0, Q, ctx, 0.0883883, n_splits=ns).clone() for ns in (32, 7, 128, 0)}
    for it in range(30):
        for ns in (32, 7, 128, 0):
            out = cache.decode(0, Q, ctx, 0.0883883, n_splits=ns)
            assert torch.equal(out, ref[ns]), f"call {it} splits {ns} differs"
    torch.cuda.synchronize()


def test_decode_graph_replay_matches_eager():
    """append + decode captured in a HIP graph: every replay (with eager work
    and synchronizations between replays) equals the eager result."""
    import torch

    print("decode graph replay", flush=True)
    cache, K, V, Q = _decode_setup(seed=6)
    ctx = [4096] * 4
    Kn, Vn = K[:, -1:].contiguous(), V[:, -1:].contiguous()
    eager = cache.decode(0, Q, ctx, 0.0883883).clone()
    out = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        cache.append(0, Kn, Vn, [4095] * 4)
        cache.decode(0, Q, ctx, 0.0883883, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cache.append(0, Kn, Vn, [4095] * 4)
        cache.decode(0, Q, ctx, 0.0883883, out=out)
    for i in range(5):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        junk = cache.decode(0, Q, [100] * 4, 0.0883883, n_splits=3)  # eager work between replays
        torch.cuda.synchronize()
        del junk


@pytest.mark.parametrize("kt,vt", [("q8_0", "q4_0"), ("f16", "f16"), ("q4_0", "q8_0"), ("q5_0", "q5_0"),
                                   ("q8_0", "turbo3")])
def test_decode_ignores_garbage_past_context(kt, vt):
    """Cache memory past ctx_len may hold any bits (here NaN patterns in codes
    and scales): the ragged tail tile must not let them into the output."""
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    print(f"decode garbage past context {kt}/{vt}", flush=True)
    rng = np.random.default_rng(9)
    S, Hq, Hkv, D, T = 2, 16, 2, 128, 256
    cache = kvq.KVCache(1, S, Hq, Hkv, D, T, (kt, vt))
    for b in cache.buffers[0]:
        if b is not None:
            b.fill_(-1)  # all bits set: binary16 NaN everywhere
    orc = oracle.OracleLayer(kt, vt, S, Hq, Hkv, D, T)
    ctx = [203, 77]
    K = torch.from_numpy((rng.standard_normal((S, 203, Hkv, D)) * 2).astype(np.float16)).cuda()
    V = torch.from_numpy(rng.standard_normal((S, 203, Hkv, D)).astype(np.float16)).cuda()
    cache.append(0, K, V, [0, 0])
    orc.append(bits(K), bits(V), np.zeros(S, np.int32))
    Q = torch.from_numpy(rng.standard_normal((S, Hq, D)).astype(np.float16)).cuda()
    ref = orc.attn_decode(bits(Q), np.array(ctx, np.int32), 0.0883883)
    for ns in (0, 1, 3):
        out = cache.decode(0, Q, ctx, 0.0883883, n_splits=ns)
        torch.cuda.synchronize()
        assert_attn_close(out.cpu().numpy(), ref, f"garbage {kt}/{vt} splits={ns}")
