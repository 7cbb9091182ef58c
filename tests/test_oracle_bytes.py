"""Pins the oracle's byte accounting to the totals the pages print
(tests/golden/byte_counts.txt, each line cited there)."""
import os

import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "byte_counts.txt")
MiB = 1 << 20


def golden_rows(kind):
    rows = []
    for line in open(GOLDEN):
        f = line.split()
        if f and not line.startswith("#") and f[0] == kind:
            rows.append(f)
    return rows


def cache_bytes(orc, k_type, v_type, layers, heads, hd, tokens):
    kc, ks = orc.plane_bytes(k_type, 1, heads, hd, tokens)
    vc, vs = orc.plane_bytes(v_type, 1, heads, hd, tokens)
    return layers * (kc + ks), layers * (vc + vs)


@pytest.mark.parametrize("row", golden_rows("kvsplit") + golden_rows("issue"), ids=lambda r: r[0] + "-" + r[1])
def test_printed_cache_sizes(orc, row):
    _, _, kt, vt, layers, heads, hd, tokens, k_mib, v_mib, total = row
    k, v = cache_bytes(orc, kt, vt, int(layers), int(heads), int(hd), int(tokens))
    assert k + v == float(total) * MiB  # exact, not approximate
    if k_mib != "-":
        assert k == float(k_mib) * MiB and v == float(v_mib) * MiB


def test_issue_ratio_is_34_to_18(orc):
    # independent of the row width: K q8_0 816 MiB vs V q4_0 432 MiB
    kc, ks = orc.plane_bytes("q8_0", 1, 1, 32, 32)
    vc, vs = orc.plane_bytes("q4_0", 1, 1, 32, 32)
    assert (kc + ks, vc + vs) == (32 * 34, 32 * 18)
    assert 816 * 18 == 432 * 34


@pytest.mark.parametrize("row", golden_rows("saving"), ids=lambda r: r[1])
def test_printed_savings(orc, row):
    _, label, kt, vt, pct = row
    base = sum(cache_bytes(orc, "f16", "f16", 22, 4, 64, 8192))
    q = sum(cache_bytes(orc, kt, vt, 22, 4, 64, 8192))
    assert round(100 * (1 - q / base)) == int(pct)


def test_capacity_rounds_to_tiles(orc):
    assert orc.capacity(1) == 32 and orc.capacity(32) == 32 and orc.capacity(33) == 64
    kc, ks = orc.plane_bytes("q4_0", 2, 3, 64, 33)
    assert kc == 2 * 3 * 64 * 32 and ks == 2 * 3 * 64 * 2 * 2


def test_q5_0_plane_bytes(orc):
    """q5_0 (no byte totals on the pages): 16 nibble bytes + 4 high-bit bytes in
    the code stream and a 2-byte scale per 32 elements = 22 B, between q4_0's
    18 and q8_0's 34."""
    S, H, D, T = 2, 8, 128, 4096
    c, s = orc.plane_bytes("q5_0", S, H, D, T)
    elems = S * H * D * T
    assert c == elems // 32 * 20 and s == elems // 32 * 2
    c4, s4 = orc.plane_bytes("q4_0", S, H, D, T)
    c8, s8 = orc.plane_bytes("q8_0", S, H, D, T)
    assert (c4 + s4) < (c + s) < (c8 + s8)
    assert (c + s) * 32 == 22 * elems
