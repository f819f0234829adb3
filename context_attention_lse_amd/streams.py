"""Side streams that run beside the calling stream.

HIP places a stream on one of a few hardware queues (GPU_MAX_HW_QUEUES, 4 by default) when
the stream is first used, and shares the queues once they are all taken; two streams on one
queue run their work one after the other. A ring pass needs its copy stream and its second
compute stream to overlap the calling stream and each other, so it takes them from here:
fresh streams whose first use is a short spin kernel beside one on each stream already
chosen (and on the calling stream), kept only when the spins overlapped. The chosen streams
are kept per device for the life of the process; ring passes share them, since a pass joins
its side streams back into the calling stream before it returns.
"""

import time

import torch

_CHOSEN = {}
_SPIN_CYCLES = 4_000_000   # a few milliseconds of spinning at the shader clock
_TRIES = 12


def _spin_time(streams):
    """Wall time of one spin kernel on each stream, all issued before any is waited for."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in streams:
        with torch.cuda.stream(s):
            torch.cuda._sleep(_SPIN_CYCLES)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def side_streams(n, device=None):
    """``n`` streams that each overlap the current stream and one another (best effort: after
    a dozen candidates that all share a queue with a chosen stream, the last one is kept)."""
    dev = torch.device("cuda", torch.cuda.current_device() if device is None else torch.device(device).index)
    chosen = _CHOSEN.setdefault(dev.index, [])
    if len(chosen) >= n:
        return chosen[:n]
    with torch.cuda.device(dev):
        cur = torch.cuda.current_stream(dev)
        _spin_time([cur])
        one = min(_spin_time([cur]) for _ in range(2))
        while len(chosen) < n:
            for k in range(_TRIES):
                s = torch.cuda.Stream(device=dev)
                # every chosen stream and the candidate spin at once with the current stream
                if _spin_time([cur, *chosen, s]) < 1.5 * one or k == _TRIES - 1:
                    chosen.append(s)
                    break
    return chosen[:n]
