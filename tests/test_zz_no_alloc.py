"""kvq_attn_decode_append_noalloc -- the decode step whose partial slots live
in the library's static per-GPU scratch array -- against
kvq_attn_decode_append with a caller-owned workspace: two identical caches,
the same call through each entry point, planes byte for byte and outputs bit
for bit.  Two calls in a row, the second with a smaller input (the scratch
then holds the first call's partials), and the first shape once more."""
import numpy as np
import pytest

import oracle
from kvq_testutil import assert_attn_close, bits

pytestmark = pytest.mark.gpu


def _twin_caches(S, Hq, Hkv, D, T, kt, vt, seed):
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    rng = np.random.default_rng(seed)
    K = torch.from_numpy((rng.standard_t(4, (S, T, Hkv, D)) * 3).astype(np.float16)).cuda()
    V = torch.from_numpy(rng.standard_normal((S, T, Hkv, D)).astype(np.float16)).cuda()
    caches = []
    for _ in range(2):
        c = kvq.KVCache(1, S, Hq, Hkv, D, T, (kt, vt))
        for b in c.buffers[0]:
            if b is not None:
                b.zero_()
        c.append(0, K, V, [0] * S)
        caches.append(c)
    Kn = torch.from_numpy(rng.standard_normal((S, Hkv, D)).astype(np.float16)).cuda()
    Vn = torch.from_numpy(rng.standard_normal((S, Hkv, D)).astype(np.float16)).cuda()
    Q = torch.from_numpy(rng.standard_normal((S, Hq, D)).astype(np.float16)).cuda()
    return caches, K, V, Kn, Vn, Q


def _compare(S, Hq, Hkv, D, T, kt, vt, ctx, n_splits, seed, with_oracle=False):
    import torch

    print(f"noalloc vs workspace: S={S} {Hq}/{Hkv} D={D} T={T} {kt}/{vt} ctx={ctx} splits={n_splits}", flush=True)
    (A, B), K, V, Kn, Vn, Q = _twin_caches(S, Hq, Hkv, D, T, kt, vt, seed)
    scale = 1.0 / np.sqrt(D)
    want = A.decode_append(0, Kn, Vn, Q, ctx, scale, n_splits=n_splits)
    got = torch.full_like(want, float("nan"))
    B.decode_append_noalloc(0, Kn, Vn, Q, ctx, scale, got, n_splits=n_splits)
    torch.cuda.synchronize()
    assert torch.equal(got, want), "outputs differ from kvq_attn_decode_append"
    for a, b in zip(A.buffers[0], B.buffers[0]):
        if a is not None:
            assert torch.equal(a, b), "planes differ from kvq_attn_decode_append's"
    if with_oracle:
        orc = oracle.OracleLayer(kt, vt, S, Hq, Hkv, D, T)
        orc.append(bits(K), bits(V), np.zeros(S, np.int32))
        orc.append(bits(Kn[:, None]), bits(Vn[:, None]), np.array([c - 1 for c in ctx], np.int32))
        ref = orc.attn_decode(bits(Q), np.array(ctx, np.int32), scale)
        print(assert_attn_close(got.cpu().numpy(), ref, "noalloc vs oracle"), flush=True)


def test_noalloc_equals_workspace_entry_point():
    # a Llama-3-8B-shaped layer at 4096 tokens, ragged contexts, automatic split
    _compare(8, 32, 8, 128, 4096, "q8_0", "q4_0", [4096, 4000, 3001, 77, 4096, 1, 2048, 999], 0, seed=1)
    # then a smaller call: fewer sequences and heads, head_dim 64, other types, fixed splits
    _compare(2, 16, 2, 64, 600, "q4_0", "turbo3", [600, 257], 5, seed=2, with_oracle=True)
    # and the first shape again, now over the smaller call's partials
    _compare(8, 32, 8, 128, 4096, "q8_0", "q4_0", [4096, 4000, 3001, 77, 4096, 1, 2048, 999], 0, seed=3)


def test_noalloc_rejects_too_many_slots():
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    # 4 sequences x 4 kv heads x 256 splits = 1024 workgroups, a slot of 16 x 260 floats each: 17 MB > 16 MiB
    S, Hq, Hkv, D, T = 4, 64, 4, 256, 8192
    c = kvq.KVCache(1, S, Hq, Hkv, D, T, ("q4_0", "q4_0"))
    Kn = torch.zeros((S, Hkv, D), dtype=torch.float16, device="cuda")
    Q = torch.zeros((S, Hq, D), dtype=torch.float16, device="cuda")
    out = torch.zeros((S, Hq, D), dtype=torch.float32, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        c.decode_append_noalloc(0, Kn, Kn, Q, [T] * S, 0.0625, out, n_splits=256)
    assert e.value.code == kvq.KVQ_E_TOO_BIG
    torch.cuda.synchronize()
    assert not out.any(), "a rejected call wrote its output"
