"""GPU check of the read-bandwidth probe (kvq_stream_read): it must visit
every 16-byte element once, including the elements of the unrolled part and
of the ragged tail.  A zero buffer with one marked element: exactly the lane
that reads it folds to the mark's value, so the sink is written iff the
element was read."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16,blocks", [(1, 1), (1000, 3), (1 << 20, 0), ((1 << 20) + 77, 0), (5000, 2)])
def test_stream_read_visits_every_element(n16, blocks):
    import torch

    import mixed_precision_quantized_quantize_amd as kvq

    print(f"stream_read n16={n16} blocks={blocks}", flush=True)
    buf = torch.zeros(n16 * 4, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(n16)
    for idx in sorted({0, n16 - 1, int(rng.integers(n16)), n16 // 2}):
        buf.zero_()
        buf[4 * idx] = 0x5A5A1234  # x ^ y ^ z ^ w of the marked element
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        kvq.stream_read(buf, 0x5A5A1234, sink, blocks)
        torch.cuda.synchronize()
        assert sink.item() == 0x5A5A1234, f"element {idx} of {n16} not read"
        # a key no lane folds to leaves the sink alone
        sink.zero_()
        kvq.stream_read(buf, 0x11111111, sink, blocks)
        torch.cuda.synchronize()
        assert sink.item() == 0
