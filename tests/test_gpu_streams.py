"""streams.side_streams: the streams the ring driver runs its copies and second compute
stream on are distinct, kept for the process, and run beside the calling stream and each
other (spin kernels on all three at once take about the time of one)."""

import time

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _wall(streams, cycles):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in streams:
        with torch.cuda.stream(s):
            torch.cuda._sleep(cycles)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def test_side_streams_overlap_the_calling_stream():
    import context_attention_lse_amd as ca
    ca._lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    a, b = ca.streams.side_streams(2, dev)
    assert a is not b and a.cuda_stream != b.cuda_stream
    assert ca.streams.side_streams(2, dev)[0] is a    # kept for the process
    cur = torch.cuda.current_stream(dev)
    cycles = 8_000_000
    one = min(_wall([cur], cycles) for _ in range(3))
    three = min(_wall([cur, a, b], cycles) for _ in range(3))
    say(f"one spin {one * 1e3:.2f} ms, three streams at once {three * 1e3:.2f} ms")
    assert three < 1.6 * one
