#!/usr/bin/env python3
"""Decode-attention benchmark over the mixed-precision quantized KV cache.

One step = for every layer: quantize the new token's K/V row of every
sequence into the cache and flash-decode every sequence's query over the
whole cache, both in one kvq_attn_decode_append call (--unfused: kvq_append
then kvq_attn_decode, the same work in two calls).  Default workload: the Llama-3-8B-shaped
decode -- 32 layers, 32 query / 8 kv heads, head_dim 128, 32768-token
context, batch 16, K q8_0 / V q4_0 -- on seeded synthetic inputs that are
resident in HBM before the timed region starts.

Prints ONE JSON line.  `value` = algorithmic KV bytes per step / step time
(GB/s); `roofline` covers the decode call (streaming kernel + merge kernel),
(kvq_attn_decode_append: append + streaming kernel, then merge kernel)
timed with HIP events on the stream it runs on; `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload on this host; `prefill`
times the causal chunked prefill (512 queries per sequence at the end of a
131072-token K4V4 cache, one layer) against the dense binary16 MFMA peak.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
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

HBM_PEAK_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="llama3_8b_32k")
    p.add_argument("--splits", type=int, default=0, help="decode splits per (seq, kv head); 0 = automatic")
    p.add_argument("--graph", action="store_true", help="replay each step from a captured HIP graph")
    p.add_argument("--unfused", action="store_true",
                   help="append with kvq_append, then decode with kvq_attn_decode (two calls per layer)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true", help="skip the prefill measurement")
    p.add_argument("--no-stream-ceiling", action="store_true", help="skip the streaming-read ceiling measurement")
    p.add_argument("--prefill-only", action="store_true",
                   help="measure only the chunked prefill (prints a JSON line with the `prefill` object)")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--calib-copy", action="store_true",
                   help="after timing, run three plain 1 GiB device-to-device copies (a reference for "
                        "hardware byte counters)")
    return p.parse_args()


def kv_bytes_per_layer(w, kt, vt):
    import mixed_precision_quantized_quantize_amd as kvq

    sh = kvq.kvq_shape(1, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx)
    return sum(kvq.kvq_plane_bytes(sh, kt)) + sum(kvq.kvq_plane_bytes(sh, vt))


def row_bytes(w, t):
    """Bytes of one cached row (one position, one kv head) of type t."""
    return {"f16": 2 * w.head_dim, "q8_0": w.head_dim + w.head_dim // 16,
            "q4_0": w.head_dim // 2 + w.head_dim // 16}[t]


DECODE_SOURCES = ("kvq_decode.hip", "kvq_device.h", "kvq_quant.h", "kvq_internal.h")


def decode_sources_hash() -> str:
    """sha256 over the sources the decode and merge kernels are built from,
    in a fixed order (the profile summary records the same hash)."""
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        h.update(open(os.path.join(ROOT, "mixed_precision_quantized_quantize_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def traffic_from_profile(src_hash, workload):
    """Measured HBM bytes per decode call (both kernels) from the committed
    counter summary (FETCH_SIZE and WRITE_SIZE scaled by a plain copy of known
    size), or None when the decode source changed since the counters were
    taken."""
    path = os.path.join(ROOT, "profiles", f"decode_merge_kernels_{workload}.txt")
    rec = {}
    try:
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.split("#")[0].strip()
    except OSError:
        return None
    if rec.get("decode_kernel_sources_sha256") != src_hash or "hbm_bytes_per_launch" not in rec:
        return None
    return int(rec["hbm_bytes_per_launch"])


MFMA_F16_PEAK_TFLOPS = 2500.0  # dense binary16 matrix peak


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
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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


def prefill_measure(dev, calls=5, cpu=False):
    """Causal chunked prefill on one layer of the long-context workload: the
    last 512-query chunk of each of 4 sequences over 131072 K4V4 positions.
    Algorithmic flop = 4 * head_dim * n_q_heads * (visible keys summed over
    the chunk's queries) per sequence (Q.K and P.V, multiply-add = 2)."""
    import torch

    import mixed_precision_quantized_quantize_amd as kvq
    from mixed_precision_quantized_quantize_amd import synth

    w = synth.WORKLOADS["llama3_8b_128k_prefill"]
    kt, vt = w.type_pairs[0]
    n_tok, T, S = w.prefill, w.ctx, w.batch
    cache = kvq.KVCache(1, S, w.n_q_heads, w.n_kv_heads, w.head_dim, T, (kt, vt), device=dev)
    for c0 in range(0, T, synth.CHUNK):
        K, V = synth.kv_batch(w, 0, c0, min(synth.CHUNK, T - c0), device=dev)
        cache.append(0, K, V, [c0] * S)
        del K, V
    Q = synth.queries(w, 0, n_tok=n_tok, device=dev)
    out = torch.empty(tuple(Q.shape), dtype=torch.float32, device=dev)
    p0 = [T - n_tok] * S
    stream = torch.cuda.current_stream(dev)
    for _ in range(2):
        cache.prefill(0, Q, p0, w.scale, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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
    res = {
        "workload": w.name, "layer": 0, "batch": S, "n_tok": n_tok, "q_pos0": T - n_tok, "ctx": T,
        "k_type": kt, "v_type": vt, "ms_per_call": round(ms, 4), "alg_flop_per_call": flop,
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel, one layer", "achieved": round(tflops, 1),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)},
        "cpu_baseline": None,
    }
    if cpu:
        res["cpu_baseline"] = prefill_cpu_baseline(w, Q)
    return res


def prefill_cpu_baseline(w, Q, n_q=64):
    """The oracle's causal prefill on a bounded sample of the same call:
    sequence 0, the first and the last n_q queries of the chunk, all heads."""
    import numpy as np

    import oracle
    from mixed_precision_quantized_quantize_amd import synth

    kt, vt = w.type_pairs[0]
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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, kt, vt, layer_kv, q_bits, seconds):
    """The oracle, as it stands, on layer 0 of the workload: append the new
    row and decode all query heads of every sequence, repeated for about
    `seconds`.  Returns the oracle's KV GB/s."""
    import numpy as np

    import oracle

    K_bits, V_bits, Kn_bits, Vn_bits = layer_kv
    S = w.batch
    orc = oracle.OracleLayer(kt, vt, S, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx)
    orc.append(K_bits, V_bits, np.zeros(S, np.int32))
    threads = oracle.max_threads()
    ctx = np.full(S, w.ctx, np.int32)
    pos = np.full(S, w.ctx - 1, np.int32)
    reps, t0 = 0, time.perf_counter()
    while True:
        orc.append(Kn_bits, Vn_bits, pos)
        orc.attn_decode(q_bits, ctx, w.scale)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    kvb = kv_bytes_per_layer(w, kt, vt)
    return {
        "value": round(kvb / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"layer 0 of {w.name}: append 1 row + decode all {S} sequences x {w.n_q_heads} query heads "
                  f"over {w.ctx} tokens, binary64, {reps} repetition(s), {dt:.3f} s each "
                  f"(full {w.n_layers}-layer step extrapolates to {dt * w.n_layers:.1f} s, "
                  f"{S / (dt * w.n_layers):.3f} tok/s)",
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the library runs on one GPU; there is no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixed_precision_quantized_quantize_amd as kvq
    from mixed_precision_quantized_quantize_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    kvq.lib()  # fail loudly if the HIP library is missing
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_measure(torch.device("cuda:0"))}), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    kt, vt = w.type_pairs[0]
    L, S, T = w.n_layers, w.batch, w.ctx
    dev = torch.device("cuda:0")
    log(f"workload {w.name}: {L} layers, {S} seqs, {w.n_q_heads}/{w.n_kv_heads} heads, D {w.head_dim}, "
        f"ctx {T}, K {kt} / V {vt}")

    # ------------------------------------------------------------ resident cache
    t0 = time.perf_counter()
    cache = kvq.KVCache(L, S, w.n_q_heads, w.n_kv_heads, w.head_dim, T, (kt, vt), device=dev)
    layer0 = None
    for l in range(L):
        for c0 in range(0, T - 1, synth.CHUNK):
            n = min(synth.CHUNK, T - 1 - c0)
            K, V = synth.kv_batch(w, l, c0, n, device=dev)
            cache.append(l, K, V, [c0] * S)
            if l == 0 and not args.no_cpu_baseline:
                layer0 = layer0 or ([], [])
                layer0[0].append(K.cpu())
                layer0[1].append(V.cpu())
            del K, V
    torch.cuda.synchronize()
    log(f"cache filled: {L} layers x {kv_bytes_per_layer(w, kt, vt) / 2**20:.1f} MiB in {time.perf_counter() - t0:.1f} s")

    Knew, Vnew, Qs = [], [], []  # new rows [S][1][Hkv][D]
    for l in range(L):
        K, V = synth.kv_batch(w, l, T - 1, 1, device=dev, step=0)
        Knew.append(K)
        Vnew.append(V)
        Qs.append(synth.queries(w, l, device=dev))
    out = torch.empty((L, S, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    cache.workspace()
    pos, ctx = [T - 1] * S, [T] * S
    stream = torch.cuda.current_stream(dev)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]

    def step(timed):
        for l in range(L):
            if args.unfused:
                cache.append(l, Knew[l], Vnew[l], pos)
            if timed:
                ev[l][0].record(stream)
            if args.unfused:
                cache.decode(l, Qs[l], ctx, w.scale, out=out[l], n_splits=args.splits)
            else:
                cache.decode_append(l, Knew[l][:, 0], Vnew[l][:, 0], Qs[l], ctx, w.scale, out=out[l],
                                    n_splits=args.splits)
            if timed:
                ev[l][1].record(stream)

    graph = None
    if args.graph:
        step(False)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(False)
        torch.cuda.synchronize()

    def run():
        if graph is not None:
            graph.replay()
        else:
            step(False)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    # The timed region holds the K steps and nothing else: timing events
    # between the layers' calls would cost several microseconds each.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        run()
    end.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps

    # per-step durations in a second pass after the timed region (events
    # between steps only), for the median and spread
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for e0, e1 in step_ev:
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize()
    per_step = sorted(e0.elapsed_time(e1) for e0, e1 in step_ev)
    ms_median = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])

    if args.unfused:
        # the step also holds append launches: bracket each decode call with
        # events in one extra step after the timed region
        step(True)
        torch.cuda.synchronize()
        dec_avg_ms = sum(ev[l][0].elapsed_time(ev[l][1]) for l in range(L)) / L
        call_timing = "HIP events around each kvq_attn_decode call of one extra step (events add a few us)"
    else:
        # a step is exactly L back-to-back kvq_attn_decode_append calls on
        # `stream`: the timed region's events give their average duration
        # (gaps between calls included)
        dec_avg_ms = ms_step / L
        call_timing = "HIP events around the timed region / (steps x layers); gaps between calls included"

    kv_layer = kv_bytes_per_layer(w, kt, vt)
    q_bytes = S * w.n_q_heads * w.head_dim * 2
    o_bytes = S * w.n_q_heads * w.head_dim * 4
    # the fused call also reads the new binary16 rows and writes their codes
    new_bytes = 0 if args.unfused else (S * w.n_kv_heads * w.head_dim * 2 * 2 +
                                        S * w.n_kv_heads * (row_bytes(w, kt) + row_bytes(w, vt)))
    alg_bytes_launch = kv_layer + q_bytes + o_bytes + new_bytes
    kv_step = kv_layer * L
    value = kv_step / (ms_step * 1e-3) / 1e9
    achieved = alg_bytes_launch / (dec_avg_ms * 1e-3) / 1e9
    traffic = traffic_from_profile(decode_sources_hash(), w.name)

    result = {
        "metric": "decode-attn KV GB/s (% HBM peak) + tok/s, K8V4 Llama-3-8B shape, 32K ctx",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(ms_median, 4),
        "ms_per_step_min_max": [round(per_step[0], 4), round(per_step[-1], 4)],
        "ms_per_step_median_note": "a second pass of the same number of steps, each bracketed by events",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "dtype_note": "binary16 MFMA inputs with float32 accumulation and softmax; the cache stores q8_0 keys and q4_0 values",
        "data": "synthetic (seeded: K Student-t nu=4 x per-channel U(0.5,8), V and Q N(0,1), binary16)",
        "config": {"workload": w.name, "layers": L, "batch": S, "ctx": T, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "k_type": kt, "v_type": vt,
                   "splits": args.splits or "auto", "graph": bool(graph is not None),
                   "append": "separate kvq_append" if args.unfused else "fused into the decode call"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "tok_per_s": round(S / (ms_step * 1e-3), 1),
        "tok_per_s_note": "attention-only: append + decode of all layers, no projections or MLP",
        "kv_bytes_per_step": kv_step,
        "roofline": {
            "bound": "hbm",
            "kernel": ("kvq_attn_decode call (decode_kernel streaming the tiles + merge_kernel), one layer"
                       if args.unfused else
                       "kvq_attn_decode_append call (decode_kernel: row append + streaming the tiles; "
                       "merge_kernel), one layer"),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": alg_bytes_launch,
            "avg_launch_ms": round(dec_avg_ms, 5),
            "avg_launch_timing": call_timing,
        },
        "cpu_baseline": None,
        "prefill": None,
    }
    log(f"step {ms_step:.3f} ms, {value:.1f} GB/s ({100 * value / HBM_PEAK_GBPS:.1f}% of peak), "
        f"decode call {dec_avg_ms * 1e3:.1f} us -> {achieved:.1f} GB/s")

    if not args.no_stream_ceiling:
        result["stream_read_ceiling"] = stream_ceiling(dev, kv_layer, achieved)
        log(f"streaming-read ceiling {result['stream_read_ceiling']['value']:.1f} GB/s")

    if args.calib_copy:
        x = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        del x, y

    if not args.no_cpu_baseline or not args.no_prefill:
        del cache
        torch.cuda.empty_cache()
    if not args.no_prefill:
        log("timing the chunked prefill ...")
        result["prefill"] = prefill_measure(dev, cpu=not args.no_cpu_baseline)
    if not args.no_cpu_baseline and layer0 is not None:
        from mixed_precision_quantized_quantize_amd.synth import as_bits

        K0 = as_bits(torch.cat(layer0[0], dim=1))
        V0 = as_bits(torch.cat(layer0[1], dim=1))
        kv = (K0, V0, as_bits(Knew[0]), as_bits(Vnew[0]))
        log("timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(w, kt, vt, kv, as_bits(Qs[0]), args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
