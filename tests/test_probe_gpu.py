"""The read-floor helper (a measurement aid, not part of the method): it runs
through the C ABI for every load shape the bench sweeps, reads only what it
is given, and leaves its sink untouched for data that cannot produce the
sentinel (every 32-bit word of a buffer of ones is 0x01010101)."""
import pytest
import torch

import bit_quantized_linear_int8_amd as qa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wgs", [1, 256, 2048])
@pytest.mark.parametrize("lane_bytes", [4, 8, 16])
@pytest.mark.parametrize("unroll", [1, 4, 8])
def test_stream_read_runs_and_leaves_sink(wgs, lane_bytes, unroll):
    nbytes = 16924672
    src = torch.ones(nbytes + 4096, dtype=torch.uint8, device="cuda")
    sink = torch.full((2048 * 512,), 7, dtype=torch.int32, device="cuda")
    for nb in (nbytes, 1000, 0):
        qa.qa_probe_stream_read(src, nb, wgs, lane_bytes, unroll, sink=sink)
    torch.cuda.synchronize()
    assert bool((sink == 7).all())
