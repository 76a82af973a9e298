"""The entry points under HIP graph capture.

The library's host code makes no allocation, memset or synchronisation
call, so a caller can capture its launches in a graph (through torch's
graph capture, which makes the capture stream the current one).  Every
entry point's calls are captured into one graph; the graph is replayed
three times, with eager work (the outputs refilled with NaN) and a
synchronisation between replays, and every replay is checked bitwise
against the eager results.
"""

import numpy as np
import pytest

from gpu_util import host, log, need_gpu
from test_gpu_streams import _calls

pytestmark = pytest.mark.gpu


def test_captured_calls_replay_bitwise():
    torch = need_gpu()
    calls = _calls(torch, seed=200)
    for _, outs, launch in calls:
        launch()
    torch.cuda.synchronize()
    ref = [[host(x).copy() for x in outs] for _, outs, _ in calls]
    # warm-up on a side stream, as for any capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _, _, launch in calls:
            launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, _, launch in calls:
            launch()
    torch.cuda.synchronize()
    for rep in range(3):
        for _, outs, _ in calls:
            for x in outs:
                x.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (name, outs, _), r in zip(calls, ref):
            for i, (x, want) in enumerate(zip(outs, r)):
                assert np.array_equal(host(x), want, equal_nan=True), f"replay {rep}: {name} output {i}"
        log(f"replay {rep} ok")
