"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, reproduces the pages' byte totals, and rejects every invalid
argument on the host before any device work (the error convention the
llama.cpp issue asks for under "Expected behavior").  Fake but aligned device
addresses are used: a call that passed validation would touch the GPU, so
every call here is one that must fail validation."""
import ctypes
import os
import re

import pytest

import mixed_precision_quantized_quantize_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]
FAKE = 0x7F0000000000  # aligned, never dereferenced


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kvq.LIB_PATH):
        from mixed_precision_quantized_quantize_amd import build

        build.build()
    return kvq.lib()


def declared_functions():
    """Every kvq_* function declared in include/*.h."""
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(kvq.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    out = os.popen(f"nm -D --defined-only {kvq.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def test_strerror(L):
    for c in range(-7, 1):
        assert kvq.kvq_strerror(c)
    assert "unknown" in kvq.kvq_strerror(-99)


def shape(**kw):
    d = dict(n_layers=2, n_seqs=2, n_q_heads=8, n_kv_heads=2, head_dim=64, max_ctx=100)
    d.update(kw)
    return kvq.kvq_shape(*[d[k] for k, _ in kvq.kvq_shape._fields_])


def test_plane_bytes_match_printed_totals(L):
    MiB = 1 << 20
    # KVSplit page, "Vergleich der Speicherersparnis": TinyLlama at 8K tokens
    sh = shape(n_layers=22, n_seqs=1, n_q_heads=32, n_kv_heads=4, head_dim=64, max_ctx=8192)

    def total(kt, vt):
        return 22 * (sum(kvq.kvq_plane_bytes(sh, kt)) + sum(kvq.kvq_plane_bytes(sh, vt)))

    assert total("f16", "f16") == 176 * MiB
    assert total("q8_0", "q8_0") == 93.5 * MiB
    assert total("q8_0", "q4_0") == 71.5 * MiB
    assert total("q4_0", "q4_0") == 49.5 * MiB
    # llama.cpp issue, llama_kv_cache lines: 12 layers x 512-wide rows
    sh = shape(n_layers=12, n_seqs=1, n_q_heads=64, n_kv_heads=8, head_dim=64, max_ctx=131072)
    assert 12 * sum(kvq.kvq_plane_bytes(sh, "q8_0")) == 816 * MiB
    assert 12 * sum(kvq.kvq_plane_bytes(sh, "q4_0")) == 432 * MiB


def test_plane_bytes_equal_the_oracles_for_every_type(L, orc):
    """The library's and the oracle's byte counts (two independent readings
    of the layout contract), q5_0 included: 22 B per 32 elements."""
    for D in (64, 128, 256):
        sh = shape(n_layers=1, n_seqs=3, n_q_heads=8, n_kv_heads=2, head_dim=D, max_ctx=1000)
        for t in ("f16", "q8_0", "q4_0", "q5_0", "turbo3"):
            assert kvq.kvq_plane_bytes(sh, t) == orc.plane_bytes(t, 3, 2, D, 1000), (t, D)
    sh = shape(n_layers=1, n_seqs=1, n_q_heads=8, n_kv_heads=1, head_dim=128, max_ctx=1024)
    assert sum(kvq.kvq_plane_bytes(sh, "q5_0")) * 32 == 22 * 1024 * 128
    a = ctypes.c_size_t()
    assert L.kvq_plane_bytes(ctypes.byref(sh), 5, ctypes.byref(a), ctypes.byref(a)) == kvq.KVQ_E_TYPE


def make_cache(sh, kt=1, vt=2, codes=FAKE, scales=FAKE + 4096):
    n = sh.n_layers
    k = (kvq.kvq_plane * n)(*[kvq.kvq_plane(kt, codes, scales) for _ in range(n)])
    v = (kvq.kvq_plane * n)(*[kvq.kvq_plane(vt, codes, scales) for _ in range(n)])
    c = kvq.kvq_cache(sh, k, v)
    c._keep = (k, v)
    return c


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), kvq.KVQ_E_SHAPE),
    (dict(head_dim=32), kvq.KVQ_E_SHAPE),
    (dict(n_q_heads=7), kvq.KVQ_E_SHAPE),
    (dict(n_q_heads=34, n_kv_heads=2), kvq.KVQ_E_SHAPE),  # group 17 > 16
    (dict(n_seqs=257), kvq.KVQ_E_SHAPE),
    (dict(n_seqs=0), kvq.KVQ_E_SHAPE),
    (dict(max_ctx=0), kvq.KVQ_E_SHAPE),
    (dict(n_layers=0), kvq.KVQ_E_SHAPE),
    # one (sequence, kv head) range of binary16 rows must stay below 2^31 bytes
    (dict(n_seqs=1, n_q_heads=2, n_kv_heads=1, head_dim=256, max_ctx=1 << 22), kvq.KVQ_E_SHAPE),
    (dict(n_seqs=1, n_q_heads=2, n_kv_heads=1, head_dim=64, max_ctx=(1 << 24) - 31), kvq.KVQ_E_SHAPE),
    (dict(n_seqs=1, n_q_heads=2, n_kv_heads=1, head_dim=256, max_ctx=(1 << 22) - 32), kvq.KVQ_OK),
])
def test_shape_rejections(L, kw, code):
    sh = shape(**kw)
    assert kvq.kvq_cache_check(make_cache(sh) if sh.n_layers > 0 else kvq.kvq_cache(sh, None, None)) == code
    if kw.get("n_layers", 1) > 0:
        a, b = ctypes.c_size_t(), ctypes.c_size_t()
        assert L.kvq_plane_bytes(ctypes.byref(sh), 1, ctypes.byref(a), ctypes.byref(b)) == code


def test_plane_rejections(L):
    sh = shape()
    assert kvq.kvq_cache_check(make_cache(sh)) == kvq.KVQ_OK
    assert kvq.kvq_cache_check(make_cache(sh, kt=5)) == kvq.KVQ_E_TYPE
    assert kvq.kvq_cache_check(make_cache(sh, kt=4)) == kvq.KVQ_E_TYPE  # turbo3 keys: values only
    assert kvq.kvq_cache_check(make_cache(sh, kt=1, vt=4)) == kvq.KVQ_OK
    assert kvq.kvq_cache_check(make_cache(sh, codes=None)) == kvq.KVQ_E_ARG
    assert kvq.kvq_cache_check(make_cache(sh, codes=FAKE + 8)) == kvq.KVQ_E_ARG  # misaligned
    assert kvq.kvq_cache_check(make_cache(sh, scales=None)) == kvq.KVQ_E_ARG  # quantized needs scales
    assert kvq.kvq_cache_check(make_cache(sh, kt=0, vt=0, scales=None)) == kvq.KVQ_OK  # f16 needs none
    assert L.kvq_cache_check(None) == kvq.KVQ_E_ARG
    a = ctypes.c_size_t()
    assert L.kvq_plane_bytes(ctypes.byref(sh), 5, ctypes.byref(a), ctypes.byref(a)) == kvq.KVQ_E_TYPE


def test_append_rejections(L):
    sh = shape()
    c = make_cache(sh)
    ok = dict(layer=0, K=FAKE, V=FAKE, n_new=4, pos=[0, 96], kt=1, vt=2)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return kvq.kvq_append(c, a["layer"], a["K"], a["V"], a["n_new"], a["pos"], a["kt"], a["vt"], None)

    assert call(layer=2) == kvq.KVQ_E_RANGE
    assert call(layer=-1) == kvq.KVQ_E_RANGE
    assert call(K=None) == kvq.KVQ_E_ARG
    assert call(V=FAKE + 2) == kvq.KVQ_E_ARG
    assert call(kt=2) == kvq.KVQ_E_TYPE  # type differs from the plane's
    assert call(vt=9) == kvq.KVQ_E_TYPE
    assert call(n_new=0) == kvq.KVQ_E_RANGE
    assert call(pos=[0, 97]) == kvq.KVQ_E_RANGE  # 97 + 4 > max_ctx
    assert call(pos=[-1, 0]) == kvq.KVQ_E_RANGE
    assert L.kvq_append(ctypes.byref(c), 0, FAKE, FAKE, 4, None, 1, 2, None) == kvq.KVQ_E_ARG


def test_decode_rejections(L):
    sh = shape()
    c = make_cache(sh)
    need = kvq.kvq_decode_workspace_bytes(sh)
    # 2 seqs x 2 kv heads, 128 tokens of capacity (4 tiles): one counter per
    # pair (padded to 256 B), and at most one workgroup per pair (4 waves of
    # one tile), one slot each of 4 heads x (64 + 4) floats
    assert need == 256 + 4 * 4 * 68 * 4

    def call(ctx=(100, 50), ws=FAKE, wsb=need, ns=0, scale=0.125, Q=FAKE, out=FAKE, layer=0):
        return kvq.kvq_attn_decode(c, layer, Q, list(ctx), scale, out, ws, wsb, ns, None)

    assert call(ctx=(0, 5)) == kvq.KVQ_E_RANGE
    assert call(ctx=(101, 5)) == kvq.KVQ_E_RANGE
    assert call(ws=None) == kvq.KVQ_E_WORKSPACE
    assert call(wsb=16) == kvq.KVQ_E_WORKSPACE
    assert call(ns=257) == kvq.KVQ_E_RANGE
    assert call(ns=-1) == kvq.KVQ_E_RANGE
    assert call(scale=float("nan")) == kvq.KVQ_E_ARG
    assert call(Q=None) == kvq.KVQ_E_ARG
    assert call(out=FAKE + 4) == kvq.KVQ_E_ARG
    assert call(layer=5) == kvq.KVQ_E_RANGE


def test_decode_append_rejections(L):
    sh = shape()
    c = make_cache(sh)
    need = kvq.kvq_decode_workspace_bytes(sh)

    def call(K=FAKE, V=FAKE, ctx=(100, 50), ws=FAKE, wsb=need, ns=0, Q=FAKE, layer=1):
        return kvq.kvq_attn_decode_append(c, layer, K, V, Q, list(ctx), 0.125, FAKE, ws, wsb, ns, None)

    assert call(K=None) == kvq.KVQ_E_ARG
    assert call(V=None) == kvq.KVQ_E_ARG
    assert call(K=FAKE + 8) == kvq.KVQ_E_ARG
    assert call(V=FAKE + 2) == kvq.KVQ_E_ARG
    assert call(ctx=(0, 5)) == kvq.KVQ_E_RANGE  # no position ctx-1 to write
    assert call(ctx=(101, 5)) == kvq.KVQ_E_RANGE
    assert call(wsb=16) == kvq.KVQ_E_WORKSPACE
    assert call(ns=257) == kvq.KVQ_E_RANGE
    assert call(Q=None) == kvq.KVQ_E_ARG
    assert call(layer=2) == kvq.KVQ_E_RANGE


def test_decode_append_noalloc_rejections(L):
    """The no-allocation step validates like kvq_attn_decode_append, and a
    call whose partial slots exceed the static scratch is refused before any
    device work (only calls that fail validation run here)."""
    sh = shape()
    c = make_cache(sh)

    def call(c=c, K=FAKE, V=FAKE, ctx=(100, 50), ns=0, Q=FAKE, out=FAKE, layer=1):
        return kvq.kvq_attn_decode_append_noalloc(c, layer, K, V, Q, list(ctx), 0.125, out, ns, None)

    assert call(K=None) == kvq.KVQ_E_ARG
    assert call(V=FAKE + 2) == kvq.KVQ_E_ARG
    assert call(ctx=(0, 5)) == kvq.KVQ_E_RANGE
    assert call(ns=257) == kvq.KVQ_E_RANGE
    assert call(Q=None) == kvq.KVQ_E_ARG
    assert call(out=FAKE + 4) == kvq.KVQ_E_ARG
    assert call(layer=2) == kvq.KVQ_E_RANGE
    # 4 sequences x 4 kv heads x 256 splits = 1024 workgroups of four waves,
    # one slot of 16 heads x 260 floats each: 17 MB, more than the scratch
    big = make_cache(shape(n_layers=1, n_seqs=4, n_q_heads=64, n_kv_heads=4, head_dim=256, max_ctx=8192))
    assert 1024 * 16 * 260 * 4 > kvq.KVQ_NOALLOC_SCRATCH_BYTES
    assert call(c=big, ctx=(8192,) * 4, ns=256, layer=0) == kvq.KVQ_E_TOO_BIG
    assert "static scratch" in kvq.kvq_strerror(kvq.KVQ_E_TOO_BIG)


def test_prefill_rejections(L):
    sh = shape()
    c = make_cache(sh)

    def call(n_tok=10, p0=(0, 90), Q=FAKE, out=FAKE):
        return kvq.kvq_attn_prefill_chunk(c, 1, Q, n_tok, list(p0), 0.125, out, None)

    assert call(p0=(0, 91)) == kvq.KVQ_E_RANGE
    assert call(p0=(-3, 0)) == kvq.KVQ_E_RANGE
    assert call(n_tok=0) == kvq.KVQ_E_RANGE
    assert call(Q=None) == kvq.KVQ_E_ARG


def test_stream_read_rejections(L):
    """The read-bandwidth probe rejects bad arguments on the host; an empty
    read is a no-op (nothing is launched)."""
    E_ARG = -1
    assert kvq.kvq_stream_read(0, 1024, 0, FAKE, 0, 0) == E_ARG  # null source
    assert kvq.kvq_stream_read(FAKE, 1024, 0, 0, 0, 0) == E_ARG  # null sink
    assert kvq.kvq_stream_read(FAKE + 8, 1024, 0, FAKE, 0, 0) == E_ARG  # misaligned
    assert kvq.kvq_stream_read(FAKE, 1000, 0, FAKE, 0, 0) == E_ARG  # not a multiple of 16 bytes
    assert kvq.kvq_stream_read(FAKE, 1024, 0, FAKE, -1, 0) == E_ARG  # negative grid
    assert kvq.kvq_stream_read(FAKE, 0, 0, FAKE, 0, 0) == 0
