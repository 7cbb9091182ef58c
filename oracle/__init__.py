"""CPU oracle for the mixed-precision quantized KV cache: Python side.

TEST INFRASTRUCTURE ONLY.  The tests, the package's ``smoke()`` check and the
benchmark's CPU-baseline leg are the only callers allowed; the product path
never imports this package.

The arithmetic lives in ``kvq_oracle.c`` (plain C, binary64 attention),
compiled here with gcc into ``libkvq_oracle.so`` and reached through ctypes.
This module only marshals numpy arrays.  Each function's docstring names the
page passage it follows; the C file's header lists the readings taken where
the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "libkvq_oracle.so")

F16, Q8_0, Q4_0, Q5_0, TURBO3 = 0, 1, 2, 3, 4
TYPES = {"f16": F16, "q8_0": Q8_0, "q4_0": Q4_0, "q5_0": Q5_0, "turbo3": TURBO3}
ROLE_K, ROLE_V = 0, 1
# q5_0 blocks: 16 nibble bytes, then the 32 high bits as 4 little-endian bytes;
# turbo3: 8 bytes of 2-bit planes, then the 32 third bits
BLOCK_CODE_BYTES = {F16: 64, Q8_0: 32, Q4_0: 16, Q5_0: 20, TURBO3: 12}

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class Plane(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int32), ("role", ctypes.c_int32),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class Shape(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_ctx", ctypes.c_int32)]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB)
            vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
            L.kvqo_f32_to_f16.argtypes = [ctypes.c_float]
            L.kvqo_f32_to_f16.restype = ctypes.c_uint16
            L.kvqo_f16_to_f32.argtypes = [ctypes.c_uint16]
            L.kvqo_f16_to_f32.restype = ctypes.c_float
            L.kvqo_f32_to_f16_n.argtypes = [vp, vp, i64]
            L.kvqo_f16_to_f32_n.argtypes = [vp, vp, i64]
            L.kvqo_quantize_blocks.argtypes = [i32, vp, i64, vp, vp]
            L.kvqo_dequantize_blocks.argtypes = [i32, vp, vp, i64, vp]
            L.kvqo_wht32.argtypes = [vp, vp]
            L.kvqo_capacity.argtypes = [i64]
            L.kvqo_capacity.restype = i64
            L.kvqo_row_code_bytes.argtypes = [i32, i64]
            L.kvqo_row_code_bytes.restype = i64
            L.kvqo_plane_bytes.argtypes = [i32, i64, i64, i64, i64, vp, vp]
            L.kvqo_append.argtypes = [vp, vp, vp, i32, vp]
            L.kvqo_read_rows.argtypes = [vp, vp, i32, i32, i64, i64, vp]
            L.kvqo_attn_decode.argtypes = [vp, vp, vp, vp, vp, ctypes.c_double, vp, vp]
            L.kvqo_attn_prefill.argtypes = [vp, vp, vp, vp, i32, vp, ctypes.c_double, vp, vp]
            L.kvqo_max_threads.restype = i32
            _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _type_id(t) -> int:
    return TYPES[t] if isinstance(t, str) else int(t)


# ---------------------------------------------------------------- binary16

def f32_to_f16_bits(x) -> np.ndarray:
    """IEEE 754 binary32 -> binary16 bits, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    lib().kvqo_f32_to_f16_n(_ptr(x), _ptr(y), x.size)
    return y


def f16_bits_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    y = np.empty(h.shape, dtype=np.float32)
    lib().kvqo_f16_to_f32_n(_ptr(h), _ptr(y), h.size)
    return y


# ---------------------------------------------------------------- blocks

def quantize_blocks(t, x_bits) -> tuple[np.ndarray, np.ndarray]:
    """Quantize blocks x [n, 32] (binary16 bits) -> (scale bits [n], codes [n, cb]).

    q8_0 / q4_0 as llama.cpp's 32-element block formats named on the llama.cpp
    optimization page ("KV-Cache-Praezision"); q5_0, the 5-bit block named in
    the llama.cpp issue's comment thread; the formulas and op order are the
    readings listed in kvq_oracle.c.
    """
    t = _type_id(t)
    x = np.ascontiguousarray(x_bits, dtype=np.uint16).reshape(-1, 32)
    n = x.shape[0]
    d = np.zeros(n, dtype=np.uint16)
    codes = np.zeros((n, BLOCK_CODE_BYTES[t]), dtype=np.uint8)
    lib().kvqo_quantize_blocks(t, _ptr(x), n, _ptr(d), _ptr(codes))
    return d, codes


def wht32(x) -> np.ndarray:
    """H x for the 32-point Sylvester Hadamard matrix (turbo3's rotation), binary64."""
    x = np.ascontiguousarray(x, dtype=np.float64).reshape(32)
    y = np.empty(32, dtype=np.float64)
    lib().kvqo_wht32(_ptr(x), _ptr(y))
    return y


def dequantize_blocks(t, d_bits, codes) -> np.ndarray:
    """Dequantized values [n, 32] in float64: d*q (q8_0), d*(c-8) (q4_0),
    d*(c-16) (q5_0); turbo3 undoes the rotation of d*L[c]."""
    t = _type_id(t)
    d = np.ascontiguousarray(d_bits, dtype=np.uint16).reshape(-1)
    c = np.ascontiguousarray(codes, dtype=np.uint8).reshape(d.size, BLOCK_CODE_BYTES[t])
    out = np.empty((d.size, 32), dtype=np.float64)
    lib().kvqo_dequantize_blocks(t, _ptr(d), _ptr(c), d.size, _ptr(out))
    return out


# ---------------------------------------------------------------- planes

def capacity(max_ctx: int) -> int:
    return int(lib().kvqo_capacity(int(max_ctx)))


def plane_bytes(t, n_seqs, n_kv_heads, head_dim, max_ctx) -> tuple[int, int]:
    """(codes bytes, scale bytes) of one plane: 34 B / 18 B per 32 elements for
    q8_0 / q4_0 and 2 B per element for f16 (KVSplit page, "Vergleich der
    Speicherersparnis"; llama.cpp issue, llama_kv_cache size lines); 22 B for
    q5_0 (its block layout, not printed on the pages)."""
    a, b = ctypes.c_int64(), ctypes.c_int64()
    lib().kvqo_plane_bytes(_type_id(t), n_seqs, n_kv_heads, head_dim, max_ctx,
                           ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


class OracleLayer:
    """Host copies of one layer's K plane (token-major) and V plane
    (8-token interleaved), written by the oracle's own quantizer."""

    def __init__(self, k_type, v_type, n_seqs, n_q_heads, n_kv_heads, head_dim, max_ctx):
        self.k_type, self.v_type = _type_id(k_type), _type_id(v_type)
        assert self.k_type != TURBO3, "turbo3 is a values-only type"
        self.shape = Shape(n_seqs, n_q_heads, n_kv_heads, head_dim, max_ctx)
        kc, ks = plane_bytes(self.k_type, n_seqs, n_kv_heads, head_dim, max_ctx)
        vc, vs = plane_bytes(self.v_type, n_seqs, n_kv_heads, head_dim, max_ctx)
        self.k_codes = np.zeros(kc, dtype=np.uint8)
        self.k_scales = np.zeros(ks // 2, dtype=np.uint16)
        self.v_codes = np.zeros(vc, dtype=np.uint8)
        self.v_scales = np.zeros(vs // 2, dtype=np.uint16)
        self.kp = Plane(self.k_type, ROLE_K, self.k_codes.ctypes.data,
                        self.k_scales.ctypes.data if ks else None)
        self.vp = Plane(self.v_type, ROLE_V, self.v_codes.ctypes.data,
                        self.v_scales.ctypes.data if vs else None)

    def append(self, K_bits, V_bits, pos):
        """Quantize new rows K, V [S][n_new][Hkv][D] (binary16 bits) into
        positions pos[s] .. pos[s]+n_new-1."""
        S, H, D = self.shape.n_seqs, self.shape.n_kv_heads, self.shape.head_dim
        K = np.ascontiguousarray(K_bits, dtype=np.uint16)
        V = np.ascontiguousarray(V_bits, dtype=np.uint16)
        n_new = K.size // (S * H * D)
        assert K.shape == V.shape and K.size == S * n_new * H * D
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        assert pos.shape == (S,) and (pos >= 0).all() and (pos + n_new <= self.shape.max_ctx).all()
        L = lib()
        L.kvqo_append(ctypes.byref(self.kp), ctypes.byref(self.shape), _ptr(K), n_new, _ptr(pos))
        L.kvqo_append(ctypes.byref(self.vp), ctypes.byref(self.shape), _ptr(V), n_new, _ptr(pos))

    def read_rows(self, role, s, h, t0, n) -> np.ndarray:
        out = np.empty((n, self.shape.head_dim), dtype=np.float64)
        p = self.kp if role == ROLE_K else self.vp
        lib().kvqo_read_rows(ctypes.byref(p), ctypes.byref(self.shape), s, h, t0, n, _ptr(out))
        return out

    def attn_decode(self, Q_bits, ctx_len, scale, want=None) -> np.ndarray:
        """Decode attention, binary64: textbook softmax attention over the
        dequantized cache (llama.cpp optimization page, "Flash Attention":
        flash attention is exactly standard attention).  Q [S][Hq][D]."""
        sh = self.shape
        Q = np.ascontiguousarray(Q_bits, dtype=np.uint16)
        assert Q.size == sh.n_seqs * sh.n_q_heads * sh.head_dim
        ctx = np.ascontiguousarray(ctx_len, dtype=np.int32)
        assert ctx.shape == (sh.n_seqs,) and (ctx >= 1).all() and (ctx <= sh.max_ctx).all()
        w = None if want is None else np.ascontiguousarray(want, dtype=np.uint8)
        out = np.full((sh.n_seqs, sh.n_q_heads, sh.head_dim), np.nan, dtype=np.float64)
        lib().kvqo_attn_decode(ctypes.byref(self.kp), ctypes.byref(self.vp), ctypes.byref(sh),
                               _ptr(Q), _ptr(ctx), float(scale), _ptr(w), _ptr(out))
        return out

    def attn_prefill(self, Q_bits, q_pos0, scale, want=None) -> np.ndarray:
        """Causal chunked prefill, binary64 (llama.cpp optimization page,
        "Batch-Groessen-Abstimmung"): Q [S][n_tok][Hq][D]; query i sits at
        q_pos0[s]+i and sees positions 0..q_pos0[s]+i."""
        sh = self.shape
        Q = np.ascontiguousarray(Q_bits, dtype=np.uint16)
        n_tok = Q.size // (sh.n_seqs * sh.n_q_heads * sh.head_dim)
        p0 = np.ascontiguousarray(q_pos0, dtype=np.int32)
        assert p0.shape == (sh.n_seqs,) and (p0 >= 0).all() and (p0 + n_tok <= sh.max_ctx).all()
        w = None if want is None else np.ascontiguousarray(want, dtype=np.uint8)
        out = np.full((sh.n_seqs, n_tok, sh.n_q_heads, sh.head_dim), np.nan, dtype=np.float64)
        lib().kvqo_attn_prefill(ctypes.byref(self.kp), ctypes.byref(self.vp), ctypes.byref(sh),
                                _ptr(Q), n_tok, _ptr(p0), float(scale), _ptr(w), _ptr(out))
        return out


def max_threads() -> int:
    return int(lib().kvqo_max_threads())
