"""Seeded synthetic inputs (binary16 K, V, Q) shared by the tests, the smoke
check and the benchmark.

This module holds no quantization or attention arithmetic: it only draws
random numbers with torch generators and names the workload shapes.  The
pages measure real models on real text (TinyLlama, Llama-3.x, Gemma,
perplexity corpora, needle-in-a-haystack); none of those is available, so
these seeded draws with the same shapes stand in for them.

Distributions:
  normal   : N(0, 1)
  outlier  : N(0, 1) with 4 channels per (layer, kv head) multiplied by 8
  student_t: Student-t with 4 degrees of freedom, built from normals as
             Z / sqrt((Z1^2 + Z2^2 + Z3^2 + Z4^2) / 4), times a per
             (layer, kv head, channel) scale drawn from U(0.5, 8)
Keys use the config's key distribution; values and queries are N(0, 1).

Every draw is keyed by (config seed, layer, sequence, 2048-token chunk), so a
single sequence or token range can be regenerated without the rest.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

CHUNK = 2048


@dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx: int
    batch: int
    type_pairs: tuple  # ((k_type, v_type), ...)
    key_dist: str
    seed: int
    prefill: int = 0  # queries per causal chunk (0 = none)
    notes: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / float(self.head_dim) ** 0.5


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_layer_2k", 1, 32, 4, 64, 2048, 1, (("q8_0", "q4_0"),), "normal", 1000,
                 notes="one layer, GQA 8, also appends all 2048 rows"),
        Workload("tinyllama_8k", 22, 32, 4, 64, 8192, 1,
                 (("f16", "f16"), ("q8_0", "q8_0"), ("q8_0", "q4_0"), ("q4_0", "q4_0")), "outlier", 2000,
                 notes="TinyLlama-shaped cache, 22 layers x 256-wide KV"),
        Workload("llama3_8b_32k", 32, 32, 8, 128, 32768, 16, (("q8_0", "q4_0"),), "student_t", 3000,
                 notes="Llama-3-8B-shaped decode, K8V4"),
        Workload("llama31_70b_32k", 80, 64, 8, 128, 32768, 1, (("q8_0", "q4_0"), ("q8_0", "turbo3")), "student_t",
                 4000, notes="Llama-3.1-70B-shaped decode, K8V4; also K q8_0 / V turbo3 (the TurboQuant page's setup)"),
        Workload("llama3_8b_128k_prefill", 32, 32, 8, 128, 131072, 4, (("q4_0", "q4_0"),), "student_t", 5000,
                 prefill=512, notes="long context, K4V4 decode plus a 512-query causal chunk"),
    ]
}


def _gen(device, *key) -> torch.Generator:
    seed = 0
    for k in key:
        seed = (seed * 1000003 + int(k) + 1) % (2**62)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _channel_scales(w: Workload, layer: int, device) -> torch.Tensor:
    """Per (kv head, channel) multipliers of the key distribution, float32."""
    H, D = w.n_kv_heads, w.head_dim
    if w.key_dist == "student_t":
        g = _gen(device, w.seed, layer, 7)
        return torch.rand((H, D), generator=g, device=device) * 7.5 + 0.5
    s = torch.ones((H, D), device=device)
    if w.key_dist == "outlier":
        for h in range(H):
            g = _gen("cpu", w.seed, layer, 11, h)
            idx = torch.randperm(D, generator=g)[:4]
            s[h, idx.to(device)] = 8.0
    return s


def _draw(dist: str, shape, g: torch.Generator, device) -> torch.Tensor:
    if dist == "student_t":
        z = torch.randn(shape, generator=g, device=device)
        chi = torch.randn((4,) + tuple(shape), generator=g, device=device)
        return z / torch.sqrt((chi * chi).sum(0) / 4.0)
    return torch.randn(shape, generator=g, device=device)


def kv_rows(w: Workload, layer: int, seq: int, t0: int, n: int, device="cpu", step: int = -1):
    """K, V binary16 rows for positions t0..t0+n-1 of one sequence: [n][Hkv][D].

    step >= 0 selects the fresh decode-step rows instead of the cache rows."""
    H, D = w.n_kv_heads, w.head_dim
    scales = _channel_scales(w, layer, device)
    Ks, Vs = [], []
    t = t0
    while t < t0 + n:
        c = t // CHUNK
        lo, hi = c * CHUNK, (c + 1) * CHUNK
        take_lo, take_hi = t, min(t0 + n, hi)
        gk = _gen(device, w.seed, layer, seq, c, 1, step + 1)
        gv = _gen(device, w.seed, layer, seq, c, 2, step + 1)
        k = _draw(w.key_dist if w.key_dist == "student_t" else "normal", (CHUNK, H, D), gk, device) * scales
        v = torch.randn((CHUNK, H, D), generator=gv, device=device)
        Ks.append(k[take_lo - lo:take_hi - lo].to(torch.float16))
        Vs.append(v[take_lo - lo:take_hi - lo].to(torch.float16))
        t = take_hi
    return torch.cat(Ks), torch.cat(Vs)


def kv_batch(w: Workload, layer: int, t0: int, n: int, device="cpu", seqs=None, step: int = -1):
    """K, V binary16 [S][n][Hkv][D] for the listed sequences (default all)."""
    seqs = range(w.batch) if seqs is None else seqs
    Ks, Vs = zip(*(kv_rows(w, layer, s, t0, n, device, step) for s in seqs))
    return torch.stack(Ks).contiguous(), torch.stack(Vs).contiguous()


def queries(w: Workload, layer: int, n_tok: int = 0, device="cpu", step: int = 0):
    """Q binary16: [S][Hq][D] for decode (n_tok == 0), else [S][n_tok][Hq][D]."""
    g = _gen(device, w.seed, layer, 3, step, n_tok)
    shape = (w.batch, w.n_q_heads, w.head_dim) if n_tok == 0 else (w.batch, n_tok, w.n_q_heads, w.head_dim)
    return torch.randn(shape, generator=g, device=device).to(torch.float16).contiguous()


def as_bits(t: torch.Tensor):
    """binary16 tensor -> numpy uint16 bit patterns (host)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")
