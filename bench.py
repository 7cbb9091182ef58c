#!/usr/bin/env python3
"""Decode-attention benchmark over the mixed-precision quantized KV cache.

A decode step = for every layer: quantize the new token's K/V row of every
sequence into the cache and flash-decode every sequence's query over the
whole cache, both in one kvq_attn_decode_append call (--unfused:
kvq_append, then kvq_attn_decode).  Inputs are seeded synthetic tensors,
resident in HBM before any timed region starts.

The printed JSON line is the Llama-3-8B-shaped decode (32 layers, 32 query /
8 kv heads, head_dim 128, 32768-token context, batch 16, K q8_0 / V q4_0):
`value` = algorithmic KV bytes per step / step time (GB/s); `roofline`
covers one layer's call (one decode_kernel launch) timed with HIP
events on the stream it runs on; `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload on this host.  The same line carries:
  configs   every other workload, each with its own step time, roofline
            and oracle baseline:
              single_layer_2k  one layer, 2048 tokens: append all rows, then
                               decode (K8V4)
              tinyllama_8k     22 layers x 8192 tokens, f16/f16, q8_0/q8_0,
                               K8V4, K4V4, with the cache byte totals checked
              llama31_70b_32k  80 layers, batch 1, K8V4 and q8_0/turbo3
              llama3_8b_128k   32 layers, 131072 tokens, batch 4, K4V4
            The two small workloads fit in the last-level cache: their main
            figures are taken with the cache flushed before every step (a
            1 GiB write), and the back-to-back figure is reported beside it,
            labelled cache-resident.
  prefill   the causal chunked prefill (512 queries per sequence at the end
            of a 131072-token K4V4 cache, one layer) against the dense
            binary16 matrix-core peak.
  pairs     one layer of the headline shape for each of the 20 K/V type
            pairs (all caches resident, rounds interleaved), per-call time
            and the fraction of 8 TB/s for each pair's own bytes.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--only NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn KV GB/s (% HBM peak) + tok/s, K8V4 Llama-3-8B shape, 32K ctx"
HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense binary16 matrix peak
MALL_FLUSH_BYTES = 1 << 30     # a write of this size between steps evicts the last-level cache
PREWARM_S = 0.2               # untimed warm-up of the measurements other than the headline (see prewarm)

ONLY = ("llama3_8b_32k", "single_layer_2k", "tinyllama_8k", "llama31_70b_32k", "llama3_8b_128k", "prefill")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--only", choices=ONLY, default=None,
                   help="measure one workload only and print its object (profiling runs)")
    p.add_argument("--pair", default=None, help="with --only: one K/V type pair, e.g. q8_0/turbo3")
    p.add_argument("--splits", type=int, default=0, help="decode splits per (seq, kv head); 0 = automatic")
    p.add_argument("--graph", action="store_true", help="replay each step from a captured HIP graph")
    p.add_argument("--unfused", action="store_true",
                   help="append with kvq_append, then decode with kvq_attn_decode (two calls per layer)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    p.add_argument("--no-configs", action="store_true", help="headline workload (and prefill) only")
    p.add_argument("--no-pairs", action="store_true", help="skip the one-layer sweeps (decode and prefill) over all 20 type pairs")
    p.add_argument("--no-stream-ceiling", action="store_true", help="skip the streaming-read ceiling measurement")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget of the headline workload")
    p.add_argument("--cpu-seconds-other", type=float, default=3.0, help="oracle time budget of each other workload")
    p.add_argument("--calib-copy", action="store_true",
                   help="after timing, run three plain 1 GiB device-to-device copies (a reference for "
                        "hardware byte counters)")
    return p.parse_args()


# ---------------------------------------------------------------- byte accounting

def plane_bytes(w, t, n_seqs=None, ctx=None):
    import mixed_precision_quantized_quantize_amd as kvq

    sh = kvq.kvq_shape(1, n_seqs or w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, ctx or w.ctx)
    return sum(kvq.kvq_plane_bytes(sh, t))


def kv_bytes_per_layer(w, kt, vt):
    return plane_bytes(w, kt) + plane_bytes(w, vt)


def row_bytes(w, t):
    """Bytes of one cached row (one position, one kv head) of type t: codes,
    scales and bit words."""
    return plane_bytes(w, t, n_seqs=1, ctx=32) // (32 * w.n_kv_heads)


def launch_bytes(w, kt, vt, fused=True):
    """Algorithmic HBM bytes of one decode launch over one layer: the layer's
    K and V planes read once, the binary16 queries read, the float32 outputs
    written and, when the append is fused, the new f16 K/V rows read and their
    quantized rows written."""
    S = w.batch
    q_bytes = S * w.n_q_heads * w.head_dim * 2
    o_bytes = S * w.n_q_heads * w.head_dim * 4
    new_bytes = (S * w.n_kv_heads * w.head_dim * 2 * 2 +
                 S * w.n_kv_heads * (row_bytes(w, kt) + row_bytes(w, vt))) if fused else 0
    return kv_bytes_per_layer(w, kt, vt) + q_bytes + o_bytes + new_bytes


DECODE_SOURCES = ("kvq_decode.hip", "kvq_device.h", "kvq_quant.h", "kvq_internal.h")
PREFILL_SOURCES = ("kvq_prefill.hip", "kvq_device.h", "kvq_internal.h")


def sources_hash(names) -> str:
    """sha256 over the kernel sources `names` (in that order); the profile
    summaries record the same hash."""
    h = hashlib.sha256()
    for name in names:
        h.update(open(os.path.join(ROOT, "mixed_precision_quantized_quantize_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def profile_name(workload, kt, vt, first_pair):
    return f"decode_kernel_{workload}" + ("" if first_pair else f"_{kt}_{vt}") + ".txt"


def traffic_from_profile(kernel, name):
    """Measured HBM bytes per launch of `kernel` ("decode_kernel" or
    "prefill_kernel") from a committed counter summary (FETCH_SIZE and
    WRITE_SIZE scaled by a plain copy of known size), or None when there is
    none or the kernel's sources changed since the counters were taken."""
    srcs = {"decode_kernel": DECODE_SOURCES, "prefill_kernel": PREFILL_SOURCES}[kernel]
    rec = {}
    try:
        for line in open(os.path.join(ROOT, "profiles", name)):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.split("#")[0].strip()
    except OSError:
        return None
    if rec.get(f"{kernel}_sources_sha256") != sources_hash(srcs) or "hbm_bytes_per_launch" not in rec:
        return None
    return int(rec["hbm_bytes_per_launch"])


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------- timing helpers

def events(n):
    import torch

    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def prewarm(run, seconds):
    """Untimed calls of run() until `seconds` of wall-clock time have passed
    (checked every four calls).  Right after a cache is filled, the first few
    tens of milliseconds of calls run slower (up to 2.7x on the first ones)
    before they settle; the headline workload keeps exactly its W warmup
    steps, the other measurements warm up for a fixed time instead.  Returns
    the number of calls."""
    import torch

    t0, n = time.perf_counter(), 0
    while seconds > 0:
        for _ in range(4):
            run()
        n += 4
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break
    return n


def time_steps(run, steps, warmup, stream, flush=None, run_all=None, prewarm_s=0.0):
    """Back-to-back steps bracketed by one pair of events (the timed region
    holds the steps and nothing else; run_all, if given, runs all `steps` of
    them at once, e.g. one graph of them all), then a second pass with events
    around each step for the median and spread; with `flush`, a third pass
    that runs flush() before each step and times the step alone.  Before the
    `warmup` steps, `prewarm_s` seconds of untimed steps."""
    import torch

    n_pre = prewarm(run, prewarm_s)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    (e0, e1), = events(1)
    e0.record(stream)
    if run_all is not None:
        run_all()
    else:
        for _ in range(steps):
            run()
    e1.record(stream)
    torch.cuda.synchronize()
    res = {"ms_per_step": e0.elapsed_time(e1) / steps, "prewarm_steps": n_pre}
    ev = events(steps)
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    res.update(ms_median=median(per), ms_min=min(per), ms_max=max(per))
    if flush is not None:
        ev = events(steps)
        for a, b in ev:
            flush()
            a.record(stream)
            run()
            b.record(stream)
        torch.cuda.synchronize()
        res["ms_flushed"] = [a.elapsed_time(b) for a, b in ev]
    return res


def graph_of(fn, times=1):
    """A HIP graph of `times` consecutive calls of fn (captured after one
    eager call)."""
    import torch

    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(times):
            fn()
    torch.cuda.synchronize()
    return g


def mall_flusher(dev):
    """A 1 GiB buffer whose plain overwrite evicts every cache level."""
    import torch

    buf = torch.empty(MALL_FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    state = [0]

    def flush():
        state[0] += 1
        buf.fill_(state[0])

    return buf, flush


def stream_ceiling(dev, nbytes: int, achieved: float) -> dict:
    """The practical read-bandwidth ceiling: kvq_stream_read over a buffer of
    one decode call's KV size, outside the timed region."""
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    n = nbytes // 16 * 16
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(3):
        kvq.stream_read(buf, 0x7FFFFFFF, sink)
    torch.cuda.synchronize()
    reps = 20
    (e0, e1), = events(1)
    e0.record()
    for _ in range(reps):
        kvq.stream_read(buf, 0x7FFFFFFF, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = n / (ms * 1e-3) / 1e9
    del buf
    return {"value": round(gbs, 1), "unit": "GB/s", "bytes_per_launch": n, "us_per_launch": round(ms * 1e3, 2),
            "kernel": "kvq_stream_read: non-temporal 16-byte loads, 8 in flight per lane, 8 workgroups of 256 per CU",
            "frac_of_peak": round(gbs / HBM_PEAK_GBPS, 4), "decode_frac_of_ceiling": round(achieved / gbs, 4)}


# ---------------------------------------------------------------- decode workloads

def fill_cache(w, kt, vt, dev, n_fill, keep_layers=(), keep_seqs=None):
    """A cache of the workload's shape whose first n_fill positions hold the
    seeded rows; returns it and host copies of the rows of `keep_layers`
    (sequences keep_seqs, default all) for the oracle."""
    import torch

    import mixed_precision_quantized_quantize_amd as kvq
    from mixed_precision_quantized_quantize_amd import synth

    cache = kvq.KVCache(w.n_layers, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, (kt, vt), device=dev)
    kept = {l: ([], []) for l in keep_layers}
    sel = None if keep_seqs is None else torch.tensor(keep_seqs, device=dev)
    for l in range(w.n_layers):
        for c0 in range(0, n_fill, synth.CHUNK):
            n = min(synth.CHUNK, n_fill - c0)
            K, V = synth.kv_batch(w, l, c0, n, device=dev)
            cache.append(l, K, V, [c0] * w.batch)
            if l in kept:
                kept[l][0].append((K if sel is None else K[sel]).cpu())
                kept[l][1].append((V if sel is None else V[sel]).cpu())
            del K, V
    torch.cuda.synchronize()
    return cache, {l: (torch.cat(a, dim=1), torch.cat(b, dim=1)) for l, (a, b) in kept.items()}


def oracle_decode_baseline(w, kt, vt, layers, kept, new_rows, queries, seqs, seconds, sample):
    """The oracle, as it stands, on a bounded sample of a decode step: for
    each listed layer, append the new row and decode every query head of the
    listed sequences (binary64), repeated for about `seconds`.  Returns the
    oracle's KV GB/s over the sample and the extrapolated full step."""
    import numpy as np

    import oracle
    from mixed_precision_quantized_quantize_amd.synth import as_bits

    S = len(seqs)
    orcs = []
    for l in layers:
        K0, V0 = kept[l]
        orc = oracle.OracleLayer(kt, vt, S, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx)
        orc.append(as_bits(K0), as_bits(V0), np.zeros(S, np.int32))
        Kn, Vn = new_rows[l]
        orcs.append((orc, as_bits(Kn[seqs][:, None]), as_bits(Vn[seqs][:, None]), as_bits(queries[l][seqs])))
    ctx = np.full(S, w.ctx, np.int32)
    pos = np.full(S, w.ctx - 1, np.int32)
    reps, t0 = 0, time.perf_counter()
    while True:
        for orc, kn, vn, q in orcs:
            orc.append(kn, vn, pos)
            orc.attn_decode(q, ctx, w.scale)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    kvb = len(layers) * kv_bytes_per_layer(w, kt, vt) * S // w.batch
    full = dt * (w.n_layers / len(layers)) * (w.batch / S)
    return {
        "value": round(kvb / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.max_threads(), "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{sample}: append 1 row + decode all {w.n_q_heads} query heads over {w.ctx} tokens, binary64, "
                  f"{reps} repetition(s), {dt:.3f} s each (full {w.n_layers}-layer step of {w.batch} sequence(s) "
                  f"extrapolates to {full:.2f} s, {w.batch / full:.4f} tok/s)",
    }


def decode_workload(w, kt, vt, dev, args, first_pair=True, flush_mall=False, oracle_layers=(0,),
                    oracle_seqs=None, cpu_seconds=3.0, headline=False, use_graph=None):
    """One decode workload: a full step over all layers, timed, with its
    roofline and the oracle baseline.  use_graph: replay the step from a
    captured HIP graph (default: --graph).  Returns the result object."""
    import torch

    from mixed_precision_quantized_quantize_amd import synth

    L, S, T = w.n_layers, w.batch, w.ctx
    cpu = not args.no_cpu_baseline
    oracle_seqs = list(range(S)) if oracle_seqs is None else oracle_seqs
    log(f"{w.name} {kt}/{vt}: {L} layers, {S} seqs, {w.n_q_heads}/{w.n_kv_heads} heads, D {w.head_dim}, ctx {T}")
    t0 = time.perf_counter()
    cache, kept = fill_cache(w, kt, vt, dev, T - 1, keep_layers=oracle_layers if cpu else (),
                             keep_seqs=None if oracle_seqs == list(range(S)) else oracle_seqs)
    kv_layer = kv_bytes_per_layer(w, kt, vt)
    log(f"  cache filled: {L} layers x {kv_layer / 2**20:.2f} MiB in {time.perf_counter() - t0:.1f} s")
    new_rows, Qs = {}, {}
    for l in range(L):
        K, V = synth.kv_batch(w, l, T - 1, 1, device=dev, step=0)
        new_rows[l] = (K[:, 0].contiguous(), V[:, 0].contiguous())
        Qs[l] = synth.queries(w, l, device=dev)
    out = torch.empty((L, S, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    cache.workspace()
    pos, ctx = [T - 1] * S, [T] * S
    stream = torch.cuda.current_stream(dev)

    def step():
        for l in range(L):
            Kn, Vn = new_rows[l]
            if args.unfused:
                cache.append(l, Kn[:, None], Vn[:, None], pos)
                cache.decode(l, Qs[l], ctx, w.scale, out=out[l], n_splits=args.splits)
            else:
                cache.decode_append(l, Kn, Vn, Qs[l], ctx, w.scale, out=out[l], n_splits=args.splits)

    graph = graph_all = None
    if args.graph if use_graph is None else use_graph:
        graph = graph_of(step)
        graph_all = graph_of(step, args.steps)  # back-to-back steps without per-replay host overhead
    run = graph.replay if graph is not None else step
    flush_buf, flush = mall_flusher(dev) if flush_mall else (None, None)
    tm = time_steps(run, args.steps, args.warmup, stream, flush=flush,
                    run_all=graph_all.replay if graph_all is not None else None,
                    prewarm_s=0.0 if headline else PREWARM_S)
    del flush_buf, graph_all

    if args.unfused:
        # the step also holds append launches: bracket each decode call with
        # events in one extra step after the timed regions
        ev = events(L)
        for l in range(L):
            Kn, Vn = new_rows[l]
            cache.append(l, Kn[:, None], Vn[:, None], pos)
            ev[l][0].record(stream)
            cache.decode(l, Qs[l], ctx, w.scale, out=out[l], n_splits=args.splits)
            ev[l][1].record(stream)
        torch.cuda.synchronize()
        call_ms = sum(a.elapsed_time(b) for a, b in ev) / L
        call_timing = "HIP events around each kvq_attn_decode call of one extra step (events add a few us)"
    else:
        # a step is exactly L back-to-back kvq_attn_decode_append calls on
        # `stream`: the timed region's events give their average duration
        # (gaps between calls included)
        call_ms = tm["ms_per_step"] / L
        call_timing = "HIP events around the timed region / (steps x layers); gaps between calls included"

    alg_launch = launch_bytes(w, kt, vt, fused=not args.unfused)
    kv_step = kv_layer * L
    ms_main = median(tm["ms_flushed"]) if flush_mall else tm["ms_per_step"]
    call_main = ms_main / L if flush_mall else call_ms
    traffic = None if args.unfused else traffic_from_profile("decode_kernel", profile_name(w.name, kt, vt, first_pair))
    value = kv_step / (ms_main * 1e-3) / 1e9
    achieved = alg_launch / (call_main * 1e-3) / 1e9
    res = {
        "config": {"workload": w.name, "layers": L, "batch": S, "ctx": T, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "k_type": kt, "v_type": vt,
                   "splits": args.splits or "auto", "graph": graph is not None,
                   "append": "separate kvq_append" if args.unfused else "fused into the decode call"},
        "value": round(value, 2), "unit": "GB/s",
        "ms_per_step": round(ms_main, 4),
        "untimed_prewarm_steps": tm["prewarm_steps"],
        "ms_per_step_median": round(median(tm["ms_flushed"]) if flush_mall else tm["ms_median"], 4),
        "ms_per_step_min_max": [round(min(tm["ms_flushed"]), 4), round(max(tm["ms_flushed"]), 4)] if flush_mall
        else [round(tm["ms_min"], 4), round(tm["ms_max"], 4)],
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "tok_per_s": round(S / (ms_main * 1e-3), 1),
        "tok_per_s_note": "attention-only: append + decode of all layers, no projections or MLP",
        "kv_bytes_per_step": kv_step,
        "roofline": {
            "bound": "hbm",
            "kernel": ("kvq_attn_decode call (decode_kernel: streaming the tiles and the split merge), one layer"
                       if args.unfused else
                       "kvq_attn_decode_append call (decode_kernel: row append, streaming the tiles and the "
                       "split merge), one layer"),
            "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_GB_per_s": None if traffic is None else round(traffic / (call_main * 1e-3) / 1e9, 2),
            "traffic_note": "HBM bytes per launch from the committed counter summary (FETCH_SIZE + WRITE_SIZE, "
                            "copy-calibrated) whose kernel sources match; the rate divides them by avg_launch_ms",
            "alg_bytes_per_launch": alg_launch,
            "avg_launch_ms": round(call_main, 5),
            "avg_launch_timing": ("median flushed step / layers: each step timed alone after a 1 GiB write"
                                  if flush_mall else call_timing),
        },
        "cpu_baseline": None,
    }
    if flush_mall:
        res["timing"] = ("each step timed alone with HIP events after a 1 GiB device write that evicts the "
                         "last-level cache (median of the steps)")
        res["cache_resident"] = {
            "ms_per_step": round(tm["ms_per_step"], 4),
            "value": round(kv_step / (tm["ms_per_step"] * 1e-3) / 1e9, 2), "unit": "GB/s",
            "roofline_frac": round(alg_launch / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "note": "cache-resident: steps back to back (one graph of all timed steps when the step is a graph), "
                    "the whole cache fits in the last-level cache",
        }
    if headline:
        res["_alg_bytes_launch"] = alg_launch
        res["_achieved"] = achieved
    log(f"  step {ms_main:.4f} ms, {value:.1f} GB/s ({100 * value / HBM_PEAK_GBPS:.1f}% of peak), "
        f"call {call_main * 1e3:.1f} us -> {achieved:.1f} GB/s"
        + (f"; cache-resident step {tm['ms_per_step']:.4f} ms" if flush_mall else ""))
    del cache, out
    torch.cuda.empty_cache()
    if cpu:
        what = (f"layer{'s' if len(oracle_layers) > 1 else ''} "
                f"{'0..%d' % (len(oracle_layers) - 1) if len(oracle_layers) > 1 else oracle_layers[0]}, "
                f"sequence{'s' if len(oracle_seqs) > 1 else ''} "
                f"{'all %d' % S if len(oracle_seqs) == S else ','.join(map(str, oracle_seqs))} of {w.name} "
                f"({kt}/{vt})")
        res["cpu_baseline"] = oracle_decode_baseline(w, kt, vt, list(oracle_layers), kept,
                                                     {l: tuple(x.cpu() for x in new_rows[l]) for l in oracle_layers},
                                                     {l: Qs[l].cpu() for l in oracle_layers}, oracle_seqs,
                                                     cpu_seconds, what)
    return res


def single_layer_2k(dev, args):
    """One layer, 2048 tokens, batch 1, K8V4: quantize-append all 2048 rows
    (one kvq_append call) and decode one query per sequence over them (one
    kvq_attn_decode call); each step timed alone after a 1 GiB write, plus
    the back-to-back (cache-resident) figure."""
    import numpy as np
    import torch

    import mixed_precision_quantized_quantize_amd as kvq
    from mixed_precision_quantized_quantize_amd import synth

    import_oracle = not args.no_cpu_baseline
    w = synth.WORKLOADS["single_layer_2k"]
    kt, vt = w.type_pairs[0]
    S, T = w.batch, w.ctx
    log(f"{w.name} {kt}/{vt}: append {T} rows + decode")
    cache = kvq.KVCache(1, S, w.n_q_heads, w.n_kv_heads, w.head_dim, T, (kt, vt), device=dev)
    K, V = synth.kv_batch(w, 0, 0, T, device=dev)
    Q = synth.queries(w, 0, device=dev)
    out = torch.empty((S, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    cache.workspace()
    stream = torch.cuda.current_stream(dev)
    ev_parts = [events(args.steps), events(args.steps)]
    state = {"i": -1}

    def step():
        cache.append(0, K, V, [0] * S)
        cache.decode(0, Q, [T] * S, w.scale, out=out, n_splits=args.splits)

    def step_parts():  # the same step with events around each call
        i = state["i"] = (state["i"] + 1) % args.steps
        ev_parts[0][i][0].record(stream)
        cache.append(0, K, V, [0] * S)
        ev_parts[0][i][1].record(stream)
        ev_parts[1][i][0].record(stream)
        cache.decode(0, Q, [T] * S, w.scale, out=out, n_splits=args.splits)
        ev_parts[1][i][1].record(stream)

    # the step replayed from a HIP graph (three launches of a few us: eager
    # steps back to back would be bounded by the host's launch rate); the
    # back-to-back figure replays one graph of all the timed steps
    graph, graph_all = graph_of(step), graph_of(step, args.steps)
    flush_buf, flush = mall_flusher(dev)
    tm = time_steps(graph.replay, args.steps, args.warmup, stream, flush=flush, run_all=graph_all.replay,
                    prewarm_s=PREWARM_S)
    del graph_all
    # per-call durations of flushed steps (events inside the step)
    for _ in range(args.steps):
        flush()
        step_parts()
    torch.cuda.synchronize()
    app_ms = median([a.elapsed_time(b) for a, b in ev_parts[0]])
    dec_ms = median([a.elapsed_time(b) for a, b in ev_parts[1]])
    del flush_buf
    kv = kv_bytes_per_layer(w, kt, vt)
    src = S * T * w.n_kv_heads * w.head_dim * 2 * 2
    qo = S * w.n_q_heads * w.head_dim * (2 + 4)
    ms = median(tm["ms_flushed"])
    res = {
        "config": {"workload": w.name, "layers": 1, "batch": S, "ctx": T, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "k_type": kt, "v_type": vt,
                   "step": f"kvq_append of all {T} rows, then kvq_attn_decode over them", "graph": True},
        "value": round(kv / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
        "ms_per_step": round(ms, 4),
        "untimed_prewarm_steps": tm["prewarm_steps"],
        "ms_per_step_min_max": [round(min(tm["ms_flushed"]), 4), round(max(tm["ms_flushed"]), 4)],
        "timing": ("each step timed alone with HIP events after a 1 GiB device write that evicts the last-level "
                   "cache (median of the steps)"),
        "pct_hbm_peak": round(100 * kv / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "tok_per_s": round(S / (ms * 1e-3), 1),
        "kv_bytes_per_step": kv,
        "append": {"us_per_call": round(app_ms * 1e3, 2), "bytes": src + kv,
                   "GB_per_s": round((src + kv) / (app_ms * 1e-3) / 1e9, 1),
                   "note": f"binary16 rows read ({src} B) + codes and scales written ({kv} B), flushed steps"},
        "roofline": {
            "bound": "hbm", "kernel": "kvq_attn_decode call (one decode_kernel launch), one layer; latency-bound "
                                      "at this size (one small wave of work per launch)",
            "achieved": round((kv + qo) / (dec_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round((kv + qo) / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None,
            "alg_bytes_per_launch": kv + qo, "avg_launch_ms": round(dec_ms, 5),
            "avg_launch_timing": "median of HIP events around the decode call in flushed steps",
        },
        "cache_resident": {"ms_per_step": round(tm["ms_per_step"], 4),
                           "value": round(kv / (tm["ms_per_step"] * 1e-3) / 1e9, 2), "unit": "GB/s",
                           "note": "cache-resident: all timed steps back to back in one graph; cache and inputs "
                                   "stay in the caches"},
        "cpu_baseline": None,
    }
    log(f"  flushed step {ms * 1e3:.1f} us (append {app_ms * 1e3:.1f} us, decode {dec_ms * 1e3:.1f} us); "
        f"cache-resident step {tm['ms_per_step'] * 1e3:.1f} us")
    if import_oracle:
        import oracle

        Kb, Vb, Qb = synth.as_bits(K), synth.as_bits(V), synth.as_bits(Q)
        reps, t0 = 0, time.perf_counter()
        while True:
            orc = oracle.OracleLayer(kt, vt, S, w.n_q_heads, w.n_kv_heads, w.head_dim, T)
            orc.append(Kb, Vb, np.zeros(S, np.int32))
            orc.attn_decode(Qb, np.full(S, T, np.int32), w.scale)
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds_other:
                break
        dt = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {
            "value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": oracle.max_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"the whole step of {w.name}: quantize-append all {T} rows and decode all {w.n_q_heads} "
                      f"query heads, binary64, {reps} repetition(s), {dt * 1e3:.1f} ms each"}
    del cache, K, V, out
    torch.cuda.empty_cache()
    return res


def tinyllama_bytes_check(w, pairs):
    """The KVSplit page's cache sizes at TinyLlama's shape and 8K tokens
    ("Vergleich der Speicherersparnis"): 176 / 93.5 / 71.5 / 49.5 MiB."""
    printed = {("f16", "f16"): 176.0, ("q8_0", "q8_0"): 93.5, ("q8_0", "q4_0"): 71.5, ("q4_0", "q4_0"): 49.5}
    out = {}
    for kt, vt in pairs:
        mib = w.n_layers * kv_bytes_per_layer(w, kt, vt) / 2**20
        out[f"{kt}/{vt}"] = {"mib": mib, "printed_mib": printed[(kt, vt)], "equal": mib == printed[(kt, vt)]}
    return out


# ---------------------------------------------------------------- prefill

def prefill_measure(dev, calls=5, cpu=False, pair=None):
    """Causal chunked prefill on one layer of the long-context workload: the
    last 512-query chunk of each of 4 sequences over 131072 K4V4 positions
    (or the K/V type pair `pair`).
    Algorithmic flop = 4 * head_dim * n_q_heads * (visible keys summed over
    the chunk's queries) per sequence (Q.K and P.V, multiply-add = 2)."""
    import torch

    import mixed_precision_quantized_quantize_amd as kvq
    from mixed_precision_quantized_quantize_amd import synth

    w = synth.WORKLOADS["llama3_8b_128k_prefill"]
    kt, vt = pair or w.type_pairs[0]
    n_tok, T, S = w.prefill, w.ctx, w.batch
    log(f"prefill {w.name} {kt}/{vt}: {S} x {n_tok} queries at the end of {T} tokens")
    cache = kvq.KVCache(1, S, w.n_q_heads, w.n_kv_heads, w.head_dim, T, (kt, vt), device=dev)
    for c0 in range(0, T, synth.CHUNK):
        K, V = synth.kv_batch(w, 0, c0, min(synth.CHUNK, T - c0), device=dev)
        cache.append(0, K, V, [c0] * S)
        del K, V
    Q = synth.queries(w, 0, n_tok=n_tok, device=dev)
    out = torch.empty(tuple(Q.shape), dtype=torch.float32, device=dev)
    p0 = [T - n_tok] * S
    stream = torch.cuda.current_stream(dev)
    prewarm(lambda: cache.prefill(0, Q, p0, w.scale, out=out), PREWARM_S)
    (e0, e1), = events(1)
    e0.record(stream)
    for _ in range(calls):
        cache.prefill(0, Q, p0, w.scale, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    keys = sum(T - n_tok + i + 1 for i in range(n_tok))
    flop = 4.0 * w.head_dim * w.n_q_heads * keys * S
    tflops = flop / (ms * 1e-3) / 1e12
    del cache, out
    torch.cuda.empty_cache()
    log(f"  {ms:.3f} ms per call, {tflops:.1f} TFLOP/s ({100 * tflops / MFMA_F16_PEAK_TFLOPS:.1f}% of peak)")
    traffic = (traffic_from_profile("prefill_kernel", f"prefill_kernel_{w.name}.txt")
               if (kt, vt) == w.type_pairs[0] else None)
    res = {
        "workload": w.name, "layer": 0, "batch": S, "n_tok": n_tok, "q_pos0": T - n_tok, "ctx": T,
        "k_type": kt, "v_type": vt, "ms_per_call": round(ms, 4), "alg_flop_per_call": flop,
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel, one layer", "achieved": round(tflops, 1),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "traffic_unit": "bytes per launch (HBM, counters)",
                     "traffic_GB_per_s": None if traffic is None else round(traffic / (ms * 1e-3) / 1e9, 2),
                     "avg_launch_ms": round(ms, 5)},
        "cpu_baseline": None,
    }
    if cpu:
        res["cpu_baseline"] = prefill_cpu_baseline(w, Q, (kt, vt))
    return res


def prefill_pairs(dev):
    """The causal prefill of `prefill_measure` (one layer, 4 x 512 queries at
    the end of 131072 positions) for every K/V type pair, one after another
    on fresh caches: ms per call and TFLOP/s of the same algorithmic flop."""
    rows = []
    for kt, vt in PAIRS_ALL:
        r = prefill_measure(dev, pair=(kt, vt))
        rows.append({"k_type": kt, "v_type": vt, "ms_per_call": r["ms_per_call"],
                     "TFLOP_per_s": r["roofline"]["achieved"], "frac": r["roofline"]["frac"]})
    return rows


def prefill_head_dims(dev, calls=3, rounds=5):
    """The causal prefill at the other head dims: head_dim 64 (32 query / 4 kv
    heads) and 256 (16 / 8), 4 sequences, the last 512-query chunk of 32768
    positions, one layer; K8V4 and f16/f16.  Seeded Student-t keys as in the
    long-context workload.  ms per call: median over `rounds` groups of
    `calls` calls, after a timed warm-up."""
    import torch

    import mixed_precision_quantized_quantize_amd as kvq
    from mixed_precision_quantized_quantize_amd import synth

    out_list = []
    for D, hq, hkv in ((64, 32, 4), (256, 16, 8)):
        w = synth.Workload(f"prefill_d{D}", 1, hq, hkv, D, 32768, 4, (("q8_0", "q4_0"), ("f16", "f16")),
                           "student_t", 6000 + D, prefill=512)
        n_tok, T, S = w.prefill, w.ctx, w.batch
        Q = synth.queries(w, 0, n_tok=n_tok, device=dev)
        for kt, vt in w.type_pairs:
            cache = kvq.KVCache(1, S, hq, hkv, D, T, (kt, vt), device=dev)
            for c0 in range(0, T, synth.CHUNK):
                K, V = synth.kv_batch(w, 0, c0, min(synth.CHUNK, T - c0), device=dev)
                cache.append(0, K, V, [c0] * S)
                del K, V
            out = torch.empty(tuple(Q.shape), dtype=torch.float32, device=dev)
            p0 = [T - n_tok] * S
            stream = torch.cuda.current_stream(dev)
            prewarm(lambda: cache.prefill(0, Q, p0, w.scale, out=out), PREWARM_S)
            group_ms = []
            for (e0, e1) in events(rounds):
                e0.record(stream)
                for _ in range(calls):
                    cache.prefill(0, Q, p0, w.scale, out=out)
                e1.record(stream)
                torch.cuda.synchronize()
                group_ms.append(e0.elapsed_time(e1) / calls)
            ms = median(group_ms)
            flop = 4.0 * D * hq * sum(T - n_tok + i + 1 for i in range(n_tok)) * S
            tf = flop / (ms * 1e-3) / 1e12
            log(f"  prefill D={D} {hq}/{hkv} {kt}/{vt}: {ms:.3f} ms, {tf:.1f} TFLOP/s "
                f"({100 * tf / MFMA_F16_PEAK_TFLOPS:.1f}% of peak)")
            out_list.append({"head_dim": D, "q_heads": hq, "kv_heads": hkv, "k_type": kt, "v_type": vt,
                             "batch": S, "n_tok": n_tok, "ctx": T, "ms_per_call": round(ms, 4),
                             "TFLOP_per_s": round(tf, 1), "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)})
            del cache, out
            torch.cuda.empty_cache()
    return out_list


def prefill_cpu_baseline(w, Q, pair, n_q=64):
    """The oracle's causal prefill on a bounded sample of the same call:
    sequence 0, the first and the last n_q queries of the chunk, all heads."""
    import numpy as np

    import oracle
    from mixed_precision_quantized_quantize_amd import synth

    kt, vt = pair
    n_tok, T = w.prefill, w.ctx
    orc = oracle.OracleLayer(kt, vt, 1, w.n_q_heads, w.n_kv_heads, w.head_dim, T)
    for c0 in range(0, T, synth.CHUNK):
        K, V = synth.kv_batch(w, 0, c0, min(synth.CHUNK, T - c0), device=Q.device, seqs=[0])
        orc.append(synth.as_bits(K), synth.as_bits(V), np.array([c0], np.int32))
        del K, V
    qb = synth.as_bits(Q[:1])
    flop, dt = 0.0, 0.0
    for first in (0, n_tok - n_q):
        p0 = T - n_tok + first
        t0 = time.perf_counter()
        orc.attn_prefill(qb[:, first:first + n_q], np.array([p0], np.int32), w.scale)
        dt += time.perf_counter() - t0
        flop += 4.0 * w.head_dim * w.n_q_heads * sum(p0 + i + 1 for i in range(n_q))
    return {"value": round(flop / dt / 1e12, 5), "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"layer 0, sequence 0 of {w.name}: the first and the last {n_q} queries of the "
                      f"{n_tok}-query chunk, all {w.n_q_heads} query heads, binary64 ({dt:.2f} s)"}


# ---------------------------------------------------------------- the run

def other_configs(dev, args, only=None, pair=None):
    """Every workload other than the headline, as result objects."""
    from mixed_precision_quantized_quantize_amd import synth

    W = synth.WORKLOADS
    cs = args.cpu_seconds_other
    out = []

    def pairs_of(w):
        ps = list(w.type_pairs)
        return [tuple(pair.split("/"))] if pair else ps

    if only in (None, "single_layer_2k"):
        out.append(single_layer_2k(dev, args))
    if only in (None, "tinyllama_8k"):
        w = W["tinyllama_8k"]
        check = tinyllama_bytes_check(w, w.type_pairs)
        for i, (kt, vt) in enumerate(pairs_of(w)):
            # 22 launch-bound layer calls of ~10 us: the step is replayed from a
            # HIP graph, so that back-to-back steps are not bounded by the
            # host's launch rate
            r = decode_workload(w, kt, vt, dev, args, first_pair=(kt, vt) == w.type_pairs[0], flush_mall=True,
                                oracle_layers=tuple(range(w.n_layers)), cpu_seconds=cs, use_graph=True)
            r["cache_bytes_check"] = check.get(f"{kt}/{vt}")
            out.append(r)
    if only in (None, "llama31_70b_32k"):
        w = W["llama31_70b_32k"]
        for kt, vt in pairs_of(w):
            out.append(decode_workload(w, kt, vt, dev, args, first_pair=(kt, vt) == w.type_pairs[0],
                                       cpu_seconds=cs))
    if only in (None, "llama3_8b_128k"):
        w = W["llama3_8b_128k_prefill"]
        for kt, vt in pairs_of(w):
            out.append(decode_workload(w, kt, vt, dev, args, first_pair=(kt, vt) == w.type_pairs[0],
                                       oracle_seqs=[0], cpu_seconds=cs))
    return out


PAIRS_ALL = [(k, v) for k in ("f16", "q8_0", "q4_0", "q5_0") for v in ("f16", "q8_0", "q4_0", "q5_0", "turbo3")]


def pairs_sweep(dev, rounds=5, calls=10):
    """One layer of the Llama-3-8B-shaped decode step (16 sequences x 32768
    tokens, 32/8 heads, head_dim 128; kvq_attn_decode_append, automatic
    split) for each of the 20 K/V type pairs.  Every pair's cache is resident
    at once, holding the same seeded rows; the rounds are interleaved over
    the pairs (a cache timed right after it was filled runs slower while the
    fill's dirty lines leave the last-level cache).  Per pair: the median
    per-call time and the GB/s of that pair's own algorithmic bytes."""
    import torch

    import mixed_precision_quantized_quantize_amd as kvq
    from mixed_precision_quantized_quantize_amd import synth

    w = synth.WORKLOADS["llama3_8b_32k"]
    S, T = w.batch, w.ctx
    log(f"pairs: one layer of {w.name}, {len(PAIRS_ALL)} type pairs, interleaved")
    caches = {p: kvq.KVCache(1, S, w.n_q_heads, w.n_kv_heads, w.head_dim, T, p, device=dev) for p in PAIRS_ALL}
    for c0 in range(0, T - 1, synth.CHUNK):
        K, V = synth.kv_batch(w, 0, c0, min(synth.CHUNK, T - 1 - c0), device=dev)
        for c in caches.values():
            c.append(0, K, V, [c0] * S)
        del K, V
    Kn, Vn = synth.kv_batch(w, 0, T - 1, 1, device=dev, step=0)
    Kn, Vn = Kn[:, 0].contiguous(), Vn[:, 0].contiguous()
    Q = synth.queries(w, 0, device=dev)
    out = torch.empty((S, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ctx = [T] * S
    times = {p: [] for p in PAIRS_ALL}
    for _ in range(rounds):
        for p in PAIRS_ALL:
            c = caches[p]
            for _ in range(2):
                c.decode_append(0, Kn, Vn, Q, ctx, w.scale, out=out)
            (e0, e1), = events(1)
            e0.record(stream)
            for _ in range(calls):
                c.decode_append(0, Kn, Vn, Q, ctx, w.scale, out=out)
            e1.record(stream)
            torch.cuda.synchronize()
            times[p].append(e0.elapsed_time(e1) / calls)
    res = []
    for kt, vt in PAIRS_ALL:
        alg = launch_bytes(w, kt, vt)
        ms = median(times[(kt, vt)])
        gbs = alg / (ms * 1e-3) / 1e9
        res.append({"k_type": kt, "v_type": vt, "us_per_call": round(ms * 1e3, 2), "alg_bytes_per_call": alg,
                    "GB_per_s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBPS, 4)})
        log(f"  {kt}/{vt}: {ms * 1e3:.1f} us, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBPS:.0f}%)")
    del caches, out
    torch.cuda.empty_cache()
    return {"workload": w.name, "layers": 1, "timing": f"median of {rounds} interleaved rounds of {calls} calls",
            "pairs": res}


def calib_copy(dev):
    """Three plain 1 GiB device-to-device copies: the reference that scales
    hardware byte counters (FETCH_SIZE, WRITE_SIZE) to bytes."""
    import torch

    x = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    del x, y


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the library runs on one GPU; there is no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixed_precision_quantized_quantize_amd as kvq
    from mixed_precision_quantized_quantize_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    kvq.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")

    if args.only == "prefill":
        res = prefill_measure(dev, cpu=not args.no_cpu_baseline,
                              pair=tuple(args.pair.split("/")) if args.pair else None)
        if args.calib_copy:
            calib_copy(dev)
        print(json.dumps({"prefill": res}), flush=True)
        return
    if args.only not in (None, "llama3_8b_32k"):
        res = other_configs(dev, args, only=args.only, pair=args.pair)
        if args.calib_copy:
            calib_copy(dev)
        print(json.dumps({"configs": res}), flush=True)
        return

    w = synth.WORKLOADS["llama3_8b_32k"]
    kt, vt = tuple(args.pair.split("/")) if args.pair else w.type_pairs[0]
    head = decode_workload(w, kt, vt, dev, args, first_pair=(kt, vt) == w.type_pairs[0], headline=True,
                           cpu_seconds=args.cpu_seconds)
    alg_launch, achieved = head.pop("_alg_bytes_launch"), head.pop("_achieved")
    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "ms_per_step_median": head["ms_per_step_median"],
        "ms_per_step_min_max": head["ms_per_step_min_max"],
        "ms_per_step_median_note": "a second pass of the same number of steps, each bracketed by events",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "dtype_note": "binary16 MFMA inputs with float32 accumulation and softmax; the cache stores q8_0 keys and "
                      "q4_0 values",
        "data": "synthetic (seeded: K Student-t nu=4 x per-channel U(0.5,8), V and Q N(0,1), binary16)",
        "config": head["config"],
        "pct_hbm_peak": head["pct_hbm_peak"],
        "tok_per_s": head["tok_per_s"],
        "tok_per_s_note": head["tok_per_s_note"],
        "kv_bytes_per_step": head["kv_bytes_per_step"],
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "prefill": None,
        "configs": [],
    }
    if not args.no_stream_ceiling:
        result["stream_read_ceiling"] = stream_ceiling(dev, kv_bytes_per_layer(w, kt, vt), achieved)
        log(f"streaming-read ceiling {result['stream_read_ceiling']['value']:.1f} GB/s")
    if args.calib_copy:
        calib_copy(dev)
    torch.cuda.empty_cache()
    if not args.no_prefill and args.only is None:
        result["prefill"] = prefill_measure(dev, cpu=not args.no_cpu_baseline)
        result["prefill"]["other_head_dims"] = prefill_head_dims(dev)
    if not args.no_configs and args.only is None:
        result["configs"] = other_configs(dev, args)
    if not args.no_pairs and args.only is None:
        result["pairs"] = pairs_sweep(dev)
        if result["prefill"] is not None:
            result["prefill"]["pairs"] = prefill_pairs(dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
