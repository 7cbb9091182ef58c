"""Key-versus-value sensitivity computed from the HIP decode outputs.

The KVSplit page ("Wissenschaftliche Einsichten und Versuchsergebnisse")
finds keys more sensitive to quantization than values, so spending the bits
on K (K8V4) beats the reverse (K4V8).  Without model weights this is
reproduced in direction only: for every K/V type pair the GPU decodes the
same seeded cache, and the relative RMS error of its output against
unquantized attention (the binary64 oracle over the binary16 inputs, i.e.
the f16/f16 cache) is tabulated.  Each pair's GPU output is also held to the
parity tolerance against the oracle over the same quantized cache, and the
orderings that tests/test_sensitivity.py asserts on the oracle are asserted
here on the GPU's numbers.  Run with -s to see the table."""
import itertools

import numpy as np
import pytest

import oracle
from kvq_testutil import assert_attn_close, bits
from mixed_precision_quantized_quantize_amd import synth

pytestmark = pytest.mark.gpu

TYPES = ["f16", "q8_0", "q5_0", "q4_0"]
V_TYPES = TYPES + ["turbo3"]


def gpu_rel_errors(wname, n_tok, n_seqs):
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    w = synth.WORKLOADS[wname]
    K, V = synth.kv_batch(w, 0, 0, n_tok, device="cuda", seqs=range(n_seqs))
    Q = synth.queries(w, 0, device="cuda")[:n_seqs].contiguous()
    Kb, Vb, Qb = bits(K), bits(V), bits(Q)
    ctx = np.full(n_seqs, n_tok, np.int32)
    unq = oracle.OracleLayer("f16", "f16", n_seqs, w.n_q_heads, w.n_kv_heads, w.head_dim, n_tok)
    unq.append(Kb, Vb, np.zeros(n_seqs, np.int32))
    ref = unq.attn_decode(Qb, ctx, w.scale)
    err = {}
    for kt, vt in itertools.product(TYPES, V_TYPES):
        cache = kvq.KVCache(1, n_seqs, w.n_q_heads, w.n_kv_heads, w.head_dim, n_tok, (kt, vt))
        cache.append(0, K, V, [0] * n_seqs)
        out = cache.decode(0, Q, ctx.tolist(), w.scale).cpu().numpy().astype(np.float64)
        torch.cuda.synchronize()
        orc = oracle.OracleLayer(kt, vt, n_seqs, w.n_q_heads, w.n_kv_heads, w.head_dim, n_tok)
        orc.append(Kb, Vb, np.zeros(n_seqs, np.int32))
        assert_attn_close(out, orc.attn_decode(Qb, ctx, w.scale), f"{wname} {kt}/{vt}")
        err[(kt, vt)] = float(np.linalg.norm(out - ref) / np.linalg.norm(ref))
        del cache
    return err


def check_ordering(err, what):
    head = "K \\ V   " + "".join(f"{v:>9s}" for v in V_TYPES)
    rows = "\n".join(f"{k:7s} " + "".join(f"{err[(k, v)]:9.4f}" for v in V_TYPES) for k in TYPES)
    print(f"\n{what}: relative RMS error of the GPU output vs unquantized binary64 attention\n{head}\n{rows}",
          flush=True)
    # the GPU's f16/f16 differs from unquantized attention by its rounding only
    assert err[("f16", "f16")] < 2e-3, what
    # keys are the sensitive half: the same bits spent on K lose less
    assert err[("q8_0", "q4_0")] < err[("q4_0", "q8_0")], what
    assert err[("f16", "q4_0")] < err[("q4_0", "f16")], what
    assert err[("f16", "q8_0")] < err[("q8_0", "f16")], what
    # more bits on either side lose less
    assert err[("q8_0", "q8_0")] < err[("q8_0", "q4_0")] < err[("q4_0", "q4_0")], what
    assert err[("q8_0", "q8_0")] < err[("q4_0", "q8_0")], what
    # q5_0 between q8_0 and q4_0
    assert err[("q8_0", "q8_0")] < err[("q5_0", "q5_0")] < err[("q4_0", "q4_0")], what
    assert err[("q8_0", "q4_0")] < err[("q5_0", "q4_0")] < err[("q4_0", "q4_0")], what
    # turbo3 values lose more than q4_0 values, yet K8 + turbo3 V beats K4 + V8
    assert err[("q8_0", "q4_0")] < err[("q8_0", "turbo3")] < err[("q4_0", "q8_0")], what


def test_gpu_keys_more_sensitive_outlier_channels():
    print("sensitivity (GPU) tinyllama_8k", flush=True)
    check_ordering(gpu_rel_errors("tinyllama_8k", 2048, 1), "tinyllama_8k inputs, 2048 tokens")


def test_gpu_keys_more_sensitive_student_t_keys():
    print("sensitivity (GPU) llama3_8b_32k", flush=True)
    check_ordering(gpu_rel_errors("llama3_8b_32k", 2048, 2), "llama3_8b_32k inputs, 2048 tokens, 2 sequences")
