"""The Python binding rejects tensors that do not match the cache before any
call reaches the library.

The C ABI receives bare pointers and the kernels index every tensor by the
cache's shape, so a wrong shape, dtype, layout or device must raise in the
binding.  A cache whose planes are ordinary CPU tensors is enough to drive
these checks without a GPU: every call below fails validation, so nothing is
ever launched."""
import pytest
import torch

import mixed_precision_quantized_quantize_amd as kvq

S, HQ, HKV, D, T = 2, 8, 2, 64, 96


@pytest.fixture(scope="module")
def cache():
    if not __import__("os").path.exists(kvq.LIB_PATH):
        from mixed_precision_quantized_quantize_amd import build

        build.build()
    return kvq.KVCache(2, S, HQ, HKV, D, T, ("q8_0", "q4_0"), device="cpu")


def f16(*shape):
    return torch.zeros(shape, dtype=torch.float16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def test_append_rejections(cache):
    K = f16(S, 3, HKV, D)
    with pytest.raises(ValueError):
        cache.append(0, f16(S, HKV, D), f16(S, HKV, D), [0] * S)  # 3-D
    with pytest.raises(ValueError):
        cache.append(0, f16(S + 1, 3, HKV, D), f16(S + 1, 3, HKV, D), [0] * S)  # too many sequences
    with pytest.raises(ValueError):
        cache.append(0, f16(S, 3, HKV + 1, D), f16(S, 3, HKV + 1, D), [0] * S)  # kv heads
    with pytest.raises(ValueError):
        cache.append(0, f16(S, 3, HKV, D // 2), f16(S, 3, HKV, D // 2), [0] * S)  # head_dim
    with pytest.raises(ValueError):
        cache.append(0, K, f16(S, 4, HKV, D), [0] * S)  # V differs from K
    with pytest.raises(TypeError):
        cache.append(0, K.float(), f16(S, 3, HKV, D), [0] * S)
    with pytest.raises(ValueError):
        cache.append(0, f16(S, HKV, 3, D).transpose(1, 2), K, [0] * S)  # not contiguous
    with pytest.raises(ValueError):
        cache.append(0, K, K.to("meta"), [0] * S)  # another device
    with pytest.raises(ValueError):
        cache.append(0, K, K, [0] * (S + 1))
    with pytest.raises(IndexError):
        cache.append(2, K, K, [0] * S)


def test_decode_rejections(cache):
    Q = f16(S, HQ, D)
    ctx = [T] * S
    with pytest.raises(ValueError):
        cache.decode(0, f16(S, HQ + 1, D), ctx, 0.125)
    with pytest.raises(ValueError):
        cache.decode(0, f16(S + 1, HQ, D), ctx, 0.125)
    with pytest.raises(TypeError):
        cache.decode(0, Q.float(), ctx, 0.125)
    with pytest.raises(TypeError):
        cache.decode(0, Q, ctx, 0.125, out=f16(S, HQ, D))  # out must be float32
    with pytest.raises(ValueError):
        cache.decode(0, Q, ctx, 0.125, out=f32(S, HQ, D // 2))
    with pytest.raises(ValueError):
        cache.decode(0, Q, ctx, 0.125, out=f32(S, D, HQ).transpose(1, 2))
    with pytest.raises(ValueError):
        cache.decode(0, Q, ctx, 0.125, out=f32(S, HQ, D).to("meta"))
    with pytest.raises(ValueError):
        cache.decode(0, Q, [T] * (S - 1), 0.125)
    with pytest.raises(IndexError):
        cache.decode(-1, Q, ctx, 0.125)


def test_decode_append_rejections(cache):
    Q, KV = f16(S, HQ, D), f16(S, HKV, D)
    ctx = [T] * S
    with pytest.raises(ValueError):
        cache.decode_append(0, f16(S, 1, HKV, D), KV, Q, ctx, 0.125)  # rows carry no token axis
    with pytest.raises(ValueError):
        cache.decode_append(0, KV, f16(S, HKV, D + 32), Q, ctx, 0.125)
    with pytest.raises(ValueError):
        cache.decode_append(0, KV, KV, f16(S, HKV, D), ctx, 0.125)  # Q with kv heads
    with pytest.raises(TypeError):
        cache.decode_append(0, KV, KV, Q, ctx, 0.125, out=torch.zeros((S, HQ, D), dtype=torch.float64))


def test_prefill_rejections(cache):
    Q = f16(S, 5, HQ, D)
    p0 = [0] * S
    with pytest.raises(ValueError):
        cache.prefill(0, f16(S, HQ, D), p0, 0.125)  # 3-D
    with pytest.raises(ValueError):
        cache.prefill(0, f16(S, 5, HKV, D), p0, 0.125)  # kv heads instead of query heads
    with pytest.raises(ValueError):
        cache.prefill(0, f16(S - 1, 5, HQ, D), p0, 0.125)
    with pytest.raises(ValueError):
        cache.prefill(0, Q, p0, 0.125, out=f32(S, 4, HQ, D))  # out for another chunk length
    with pytest.raises(TypeError):
        cache.prefill(0, Q, p0, 0.125, out=f16(S, 5, HQ, D))
    with pytest.raises(ValueError):
        cache.prefill(0, Q, [0], 0.125)


def test_type_list_length():
    with pytest.raises(ValueError):
        kvq.KVCache(3, S, HQ, HKV, D, T, [("q8_0", "q4_0")] * 2, device="cpu")
