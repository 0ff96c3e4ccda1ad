"""Two problems on two streams, issued from two host threads at once.

The library keeps no per-call state between calls except the plan staging slots (shared under a
lock), so calls on distinct saved / workspace buffers may run concurrently. Each of two threads
runs forward and backward of its own problem on its own stream, several times; every result must
equal, bit for bit, that problem's result computed alone.
"""
import threading

import pytest

from rnnt_inputs import make_inputs
from test_gpu_parity import say

pytestmark = pytest.mark.gpu

GRADS = ("dhA", "dhL", "dWA", "dWL", "dbZ", "dWO", "dbO")


def test_two_streams_two_threads(gpu_lib):
    import torch

    rl = gpu_lib
    probs = [
        rl.Problem(make_inputs(4, 120, 30, 1000, 256, 192, 640, dtype="bf16", seed=501, t_range=(60, 120),
                               u_range=(0, 30), bias_std=0.1), tile=(32, 16), tiles_per_wave=6),
        rl.Problem(make_inputs(3, 90, 40, 700, 128, 64, 512, dtype="bf16", seed=502, t_range=(30, 90),
                               u_range=(5, 40), bias_std=0.1), mode="untiled"),
    ]
    refs = []
    for p in probs:
        p.forward()
        p.backward()
        torch.cuda.synchronize()
        refs.append((p.costs.clone(), {k: p.grads[k].clone() for k in GRADS}))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []
    say("two problems on two streams from two threads")

    def worker(i):
        try:
            p, s = probs[i], streams[i]
            with torch.cuda.stream(s):
                for _ in range(4):
                    p.costs.fill_(float("nan"))
                    p.forward()
                    p.backward()
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for p, (c, g) in zip(probs, refs):
        assert torch.equal(p.costs.view(torch.int32), c.view(torch.int32))
        for k in GRADS:
            assert torch.equal(p.grads[k].view(torch.int32), g[k].view(torch.int32)), k
