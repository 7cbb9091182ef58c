"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_driver.c compiles oracle/kvq_oracle.c into one program
with gcc -fsanitize=address,undefined (no OpenMP, so the loops run serially)
and calls every exported function on tiny shapes of every cache type and
type pair: quantizers on random, all-zero and negative-zero blocks, the
binary16 conversions over all 65536 patterns, the Walsh-Hadamard transform,
ragged appends into planes allocated at exactly the oracle's own byte count,
decode with ragged contexts and an output mask, a causal prefill chunk, and
reading every row back.  Any out-of-bounds access, use after free, signed
overflow or other undefined behaviour aborts the program."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(HERE, "oracle_sanitize_driver.c"), "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed:\n{r.stderr}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"sanitized oracle run failed (rc {r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "ok" in r.stdout
