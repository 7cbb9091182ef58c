"""Python binding of libkvq (argument marshalling only).

Every entry point of ``include/kvq.h`` is exposed under the same name and
forwards plain pointers and sizes through ctypes; every step of the hot path
runs in the HIP kernels of ``libkvq.so``.  PyTorch is used for device memory
and streams only (``KVCache`` allocates the planes with torch).

The library must be built (``python -m mixed_precision_quantized_quantize_amd.build``);
there is no fallback of any kind: a missing library raises ``KvqLibraryMissing``.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

F16, Q8_0, Q4_0, Q5_0, TURBO3 = 0, 1, 2, 3, 4
TYPES = {"f16": F16, "q8_0": Q8_0, "q4_0": Q4_0, "q5_0": Q5_0, "turbo3": TURBO3}  # turbo3: values only
TYPE_NAMES = {v: k for k, v in TYPES.items()}

KVQ_OK, KVQ_E_ARG, KVQ_E_TYPE, KVQ_E_SHAPE, KVQ_E_RANGE, KVQ_E_WORKSPACE, KVQ_E_HIP = 0, -1, -2, -3, -4, -5, -6
KVQ_E_TOO_BIG = -7
KVQ_MAX_SEQS, KVQ_MAX_GROUP, KVQ_MAX_SPLITS = 256, 16, 256
KVQ_NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTS = ["kvq_strerror", "kvq_plane_bytes", "kvq_cache_check", "kvq_append", "kvq_decode_workspace_bytes",
           "kvq_attn_decode", "kvq_attn_decode_append", "kvq_attn_prefill_chunk", "kvq_attn_decode_append_noalloc",
           "kvq_stream_read"]


class KvqLibraryMissing(RuntimeError):
    pass


class KvqError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {kvq_strerror(code)} (code {code})")


class kvq_shape(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_seqs", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("max_ctx", ctypes.c_int32)]


class kvq_plane(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int32), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class kvq_cache(ctypes.Structure):
    _fields_ = [("shape", kvq_shape), ("k", ctypes.POINTER(kvq_plane)), ("v", ctypes.POINTER(kvq_plane))]


_lock = threading.Lock()
_lib = None


def lib():
    """The loaded libkvq.so (raises KvqLibraryMissing if it was not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise KvqLibraryMissing(f"{LIB_PATH} is not built; run "
                                        "`python -m mixed_precision_quantized_quantize_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
            P = ctypes.POINTER
            L.kvq_strerror.argtypes = [ctypes.c_int]
            L.kvq_strerror.restype = ctypes.c_char_p
            L.kvq_plane_bytes.argtypes = [P(kvq_shape), i32, P(sz), P(sz)]
            L.kvq_cache_check.argtypes = [P(kvq_cache)]
            L.kvq_append.argtypes = [P(kvq_cache), i32, vp, vp, i32, P(ctypes.c_int32), i32, i32, vp]
            L.kvq_decode_workspace_bytes.argtypes = [P(kvq_shape), P(sz)]
            L.kvq_attn_decode.argtypes = [P(kvq_cache), i32, vp, P(ctypes.c_int32), ctypes.c_float, vp, vp, sz,
                                          i32, vp]
            L.kvq_attn_decode_append.argtypes = [P(kvq_cache), i32, vp, vp, vp, P(ctypes.c_int32), ctypes.c_float,
                                                 vp, vp, sz, i32, vp]
            L.kvq_attn_prefill_chunk.argtypes = [P(kvq_cache), i32, vp, i32, P(ctypes.c_int32), ctypes.c_float,
                                                 vp, vp]
            L.kvq_attn_decode_append_noalloc.argtypes = [P(kvq_cache), i32, vp, vp, vp, P(ctypes.c_int32),
                                                         ctypes.c_float, vp, i32, vp]
            L.kvq_stream_read.argtypes = [vp, sz, ctypes.c_uint32, vp, i32, vp]
            for name in EXPORTS:
                if name != "kvq_strerror":
                    getattr(L, name).restype = ctypes.c_int
            _lib = L
    return _lib


def _i32_array(vals):
    vals = [int(v) for v in vals]
    return (ctypes.c_int32 * len(vals))(*vals)


def _check(rc: int, where: str):
    if rc != KVQ_OK:
        raise KvqError(rc, where)


def _type(t) -> int:
    return TYPES[t] if isinstance(t, str) else int(t)


# ------------------------------------------------------------------ C ABI, same names

def kvq_strerror(code: int) -> str:
    return lib().kvq_strerror(int(code)).decode()


def kvq_plane_bytes(shape: kvq_shape, type_) -> tuple[int, int]:
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().kvq_plane_bytes(ctypes.byref(shape), _type(type_), ctypes.byref(a), ctypes.byref(b)),
           "kvq_plane_bytes")
    return a.value, b.value


def kvq_cache_check(cache: kvq_cache) -> int:
    return lib().kvq_cache_check(ctypes.byref(cache))


def kvq_decode_workspace_bytes(shape: kvq_shape) -> int:
    b = ctypes.c_size_t()
    _check(lib().kvq_decode_workspace_bytes(ctypes.byref(shape), ctypes.byref(b)), "kvq_decode_workspace_bytes")
    return b.value


def kvq_append(cache: kvq_cache, layer: int, K_ptr: int, V_ptr: int, n_new: int, pos, k_type, v_type,
               stream: int) -> int:
    return lib().kvq_append(ctypes.byref(cache), int(layer), K_ptr, V_ptr, int(n_new), _i32_array(pos),
                            _type(k_type), _type(v_type), stream)


def kvq_attn_decode(cache: kvq_cache, layer: int, Q_ptr: int, ctx_len, scale: float, out_ptr: int, ws_ptr: int,
                    ws_bytes: int, n_splits: int, stream: int) -> int:
    return lib().kvq_attn_decode(ctypes.byref(cache), int(layer), Q_ptr, _i32_array(ctx_len), float(scale), out_ptr,
                                 ws_ptr, int(ws_bytes), int(n_splits), stream)


def kvq_attn_decode_append(cache: kvq_cache, layer: int, K_ptr: int, V_ptr: int, Q_ptr: int, ctx_len,
                           scale: float, out_ptr: int, ws_ptr: int, ws_bytes: int, n_splits: int, stream: int) -> int:
    return lib().kvq_attn_decode_append(ctypes.byref(cache), int(layer), K_ptr, V_ptr, Q_ptr, _i32_array(ctx_len),
                                        float(scale), out_ptr, ws_ptr, int(ws_bytes), int(n_splits), stream)


def kvq_attn_prefill_chunk(cache: kvq_cache, layer: int, Q_ptr: int, n_tok: int, q_pos0, scale: float,
                           out_ptr: int, stream: int) -> int:
    return lib().kvq_attn_prefill_chunk(ctypes.byref(cache), int(layer), Q_ptr, int(n_tok), _i32_array(q_pos0),
                                        float(scale), out_ptr, stream)


def kvq_attn_decode_append_noalloc(cache: kvq_cache, layer: int, K_ptr: int, V_ptr: int, Q_ptr: int, ctx_len,
                                   scale: float, out_ptr: int, n_splits: int, stream: int) -> int:
    return lib().kvq_attn_decode_append_noalloc(ctypes.byref(cache), int(layer), K_ptr, V_ptr, Q_ptr,
                                                _i32_array(ctx_len), float(scale), out_ptr, int(n_splits), stream)


def kvq_stream_read(src_ptr: int, nbytes: int, key: int, sink_ptr: int, blocks: int, stream: int) -> int:
    return lib().kvq_stream_read(src_ptr, int(nbytes), ctypes.c_uint32(key), sink_ptr, int(blocks), stream)


def stream_read(buf, key: int, sink, blocks: int = 0) -> None:
    """Streams the device tensor `buf` (contiguous, 16-byte aligned, size a
    multiple of 16 bytes) through the read-bandwidth probe on the current
    stream; `sink` is a device uint32 / int32 tensor of at least one element."""
    import torch

    if not (buf.is_cuda and sink.is_cuda and buf.device == sink.device and buf.is_contiguous()):
        raise ValueError("stream_read: buf and sink must be contiguous tensors on one GPU")
    if sink.numel() < 1 or sink.element_size() != 4:
        raise ValueError("stream_read: sink must hold at least one 32-bit element")
    _check(kvq_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), key, sink.data_ptr(), blocks,
                           torch.cuda.current_stream(buf.device).cuda_stream), "kvq_stream_read")


# ------------------------------------------------------------------ torch plumbing

class KVCache:
    """Cache planes in device memory (allocated with torch) plus the kvq_cache
    descriptor that points at them.  ``types`` is one (k_type, v_type) pair
    for all layers, or a list with one pair per layer."""

    def __init__(self, n_layers, n_seqs, n_q_heads, n_kv_heads, head_dim, max_ctx, types, device="cuda"):
        import torch

        self.torch = torch
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:  # compare as tensors report it
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.shape = kvq_shape(n_layers, n_seqs, n_q_heads, n_kv_heads, head_dim, max_ctx)
        if isinstance(types[0], (str, int)):
            types = [tuple(types)] * n_layers
        if len(types) != n_layers:
            raise ValueError(f"{len(types)} (k_type, v_type) pairs for {n_layers} layers")
        self.types = [(_type(k), _type(v)) for k, v in types]
        self.k_planes = (kvq_plane * n_layers)()
        self.v_planes = (kvq_plane * n_layers)()
        self.buffers = []  # (k_codes, k_scales, v_codes, v_scales) per layer
        for l, (kt, vt) in enumerate(self.types):
            bufs = []
            for t, planes in ((kt, self.k_planes), (vt, self.v_planes)):
                cb, sb = kvq_plane_bytes(self.shape, t)
                codes = torch.empty(cb, dtype=torch.uint8, device=self.device)
                scales = torch.empty(max(sb // 2, 1), dtype=torch.int16, device=self.device) if sb else None
                planes[l] = kvq_plane(t, codes.data_ptr(), scales.data_ptr() if scales is not None else None)
                bufs += [codes, scales]
            self.buffers.append(tuple(bufs))
        self.desc = kvq_cache(self.shape, self.k_planes, self.v_planes)
        _check(kvq_cache_check(self.desc), "kvq_cache_check")
        self._ws = None

    def _stream(self):
        return self.torch.cuda.current_stream(self.device).cuda_stream

    # The C ABI sees only pointers; the kernels index every tensor by the
    # cache's shape.  Each tensor is therefore checked here -- dtype, shape,
    # contiguity and device -- before anything reaches the library, so that a
    # wrong-shaped tensor raises instead of being read or written past its end.
    def _tensor(self, x, name, dtype, shape):
        t = self.torch
        if not isinstance(x, t.Tensor):
            raise TypeError(f"{name}: expected a torch.Tensor, got {type(x).__name__}")
        if x.dtype != dtype:
            raise TypeError(f"{name}: dtype {x.dtype}, expected {dtype}")
        if tuple(x.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(x.shape)}, expected {tuple(shape)}")
        if not x.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
        if x.device != self.device:
            raise ValueError(f"{name}: on {x.device}, the cache is on {self.device}")
        return x

    def _host_ints(self, vals, name):
        vals = [int(v) for v in vals]
        if len(vals) != self.shape.n_seqs:
            raise ValueError(f"{name}: {len(vals)} entries, expected n_seqs = {self.shape.n_seqs}")
        return vals

    def _layer(self, layer):
        if not 0 <= int(layer) < self.shape.n_layers:
            raise IndexError(f"layer {layer} out of range [0, {self.shape.n_layers})")
        return int(layer)

    def append(self, layer, K, V, pos):
        """K, V: binary16 device tensors [S][n_new][Hkv][D]; pos: host ints [S]."""
        sh, layer = self.shape, self._layer(layer)
        if not isinstance(K, self.torch.Tensor) or K.dim() != 4:
            raise ValueError("K: expected a 4-D tensor [n_seqs][n_new][n_kv_heads][head_dim]")
        want = (sh.n_seqs, K.shape[1], sh.n_kv_heads, sh.head_dim)
        self._tensor(K, "K", self.torch.float16, want)
        self._tensor(V, "V", self.torch.float16, want)
        pos = self._host_ints(pos, "pos")
        kt, vt = self.types[layer]
        _check(kvq_append(self.desc, layer, K.data_ptr(), V.data_ptr(), K.shape[1], pos, kt, vt, self._stream()),
               "kvq_append")

    def workspace(self):
        if self._ws is None:
            nb = kvq_decode_workspace_bytes(self.shape)
            # zero-filled once: the merge counters at its start must be zero before the first call
            self._ws = self.torch.zeros(max(nb, 16) // 4, dtype=self.torch.float32, device=self.device)
        return self._ws

    def _out(self, out, shape):
        if out is None:
            return self.torch.empty(shape, dtype=self.torch.float32, device=self.device)
        return self._tensor(out, "out", self.torch.float32, shape)

    def _decode_args(self, Q, out):
        sh = self.shape
        want = (sh.n_seqs, sh.n_q_heads, sh.head_dim)
        self._tensor(Q, "Q", self.torch.float16, want)
        return self._out(out, want), self.workspace()

    def decode(self, layer, Q, ctx_len, scale, out=None, n_splits=0):
        """Q: binary16 [S][Hq][D] -> float32 [S][Hq][D]."""
        layer = self._layer(layer)
        out, ws = self._decode_args(Q, out)
        ctx_len = self._host_ints(ctx_len, "ctx_len")
        _check(kvq_attn_decode(self.desc, layer, Q.data_ptr(), ctx_len, scale, out.data_ptr(), ws.data_ptr(),
                               ws.numel() * 4, n_splits, self._stream()), "kvq_attn_decode")
        return out

    def decode_append(self, layer, K, V, Q, ctx_len, scale, out=None, n_splits=0):
        """Writes K, V (binary16 [S][Hkv][D]) at positions ctx_len[s]-1, then
        decodes Q: binary16 [S][Hq][D] -> float32 [S][Hq][D]."""
        sh, layer = self.shape, self._layer(layer)
        for x, name in ((K, "K"), (V, "V")):
            self._tensor(x, name, self.torch.float16, (sh.n_seqs, sh.n_kv_heads, sh.head_dim))
        out, ws = self._decode_args(Q, out)
        ctx_len = self._host_ints(ctx_len, "ctx_len")
        _check(kvq_attn_decode_append(self.desc, layer, K.data_ptr(), V.data_ptr(), Q.data_ptr(), ctx_len, scale,
                                      out.data_ptr(), ws.data_ptr(), ws.numel() * 4, n_splits, self._stream()),
               "kvq_attn_decode_append")
        return out

    def decode_append_noalloc(self, layer, K, V, Q, ctx_len, scale, out, n_splits=0):
        """decode_append through kvq_attn_decode_append_noalloc: the partial
        slots live in the library's static per-GPU scratch array, and nothing
        is allocated (``out`` is required for that reason)."""
        sh, layer = self.shape, self._layer(layer)
        for x, name in ((K, "K"), (V, "V")):
            self._tensor(x, name, self.torch.float16, (sh.n_seqs, sh.n_kv_heads, sh.head_dim))
        want = (sh.n_seqs, sh.n_q_heads, sh.head_dim)
        self._tensor(Q, "Q", self.torch.float16, want)
        self._tensor(out, "out", self.torch.float32, want)
        ctx_len = self._host_ints(ctx_len, "ctx_len")
        _check(kvq_attn_decode_append_noalloc(self.desc, layer, K.data_ptr(), V.data_ptr(), Q.data_ptr(), ctx_len,
                                              scale, out.data_ptr(), n_splits, self._stream()),
               "kvq_attn_decode_append_noalloc")
        return out

    def prefill(self, layer, Q, q_pos0, scale, out=None):
        """Q: binary16 [S][n_tok][Hq][D] -> float32 [S][n_tok][Hq][D]."""
        sh, layer = self.shape, self._layer(layer)
        if not isinstance(Q, self.torch.Tensor) or Q.dim() != 4:
            raise ValueError("Q: expected a 4-D tensor [n_seqs][n_tok][n_q_heads][head_dim]")
        want = (sh.n_seqs, Q.shape[1], sh.n_q_heads, sh.head_dim)
        self._tensor(Q, "Q", self.torch.float16, want)
        out = self._out(out, want)
        q_pos0 = self._host_ints(q_pos0, "q_pos0")
        _check(kvq_attn_prefill_chunk(self.desc, layer, Q.data_ptr(), Q.shape[1], q_pos0, scale, out.data_ptr(),
                                      self._stream()), "kvq_attn_prefill_chunk")
        return out

    def plane_tensors(self, layer):
        """(k_codes, k_scales, v_codes, v_scales) device tensors of a layer."""
        return self.buffers[layer]
