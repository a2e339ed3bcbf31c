"""Several host threads drive the library at once, each on a stream of its own with its
own inputs, metadata and workspaces, as a serving process would: every result equals,
bit for bit, that of the same calls made one after the other on the default stream.
The library keeps no state shared between calls apart from the kernel-timing hook,
which these calls leave unset; the cases use the three tile families (256x256,
128x128 and the 32-row tiles of few rows per expert)."""
import threading

import numpy as np
import pytest

import synth
from _util import Gpu

pytestmark = pytest.mark.gpu

CASES = [
    dict(N=3000, H=256, I=256, E=8, K=4, seed=21),  # 256x256 tiles
    dict(N=1500, H=384, I=128, E=5, K=3, seed=22),  # 128x128 tiles (H not a multiple of 256)
    dict(N=64, H=256, I=128, E=32, K=2, seed=23),  # 32-row tiles (<= 16 rows per expert)
    dict(N=2000, H=256, I=256, E=6, K=2, seed=24),
]
KEYS = ("out", "h", "dx", "dw_up", "dw_down", "dtw")


def run_all(g):
    g.build()
    g.forward()
    g.backward()


def outputs(g):
    return {k: getattr(g, k).float().cpu().numpy() for k in KEYS}


def test_threads_on_own_streams_match_serial():
    import torch

    ds = [synth.case(**c) for c in CASES]
    serial = []
    for d in ds:
        g = Gpu(d)
        run_all(g)
        torch.cuda.synchronize()
        serial.append(outputs(g))

    gs = [Gpu(d) for d in ds]
    torch.cuda.synchronize()  # inputs were copied on the default stream
    streams = [torch.cuda.Stream() for _ in gs]
    start = threading.Barrier(len(gs))
    errors = []

    def work(i):
        try:
            with torch.cuda.stream(streams[i]):
                start.wait(timeout=60)
                for _ in range(3):
                    run_all(gs[i])
            streams[i].synchronize()
        except BaseException as ex:  # reported by the main thread
            errors.append((i, ex))

    print(f"threads: {len(gs)} cases, 3 rounds each", flush=True)
    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(gs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for i, g in enumerate(gs):
        got = outputs(g)
        for k in KEYS:
            assert np.array_equal(got[k], serial[i][k]), f"case {i}: {k} differs from the serial run"
