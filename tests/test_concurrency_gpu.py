"""Two host threads, each launching on a stream of its own at the same time,
get the results of sequential calls (the library keeps no state between
calls apart from a per-device compute-unit count and the per-thread error
message)."""
import threading

import numpy as np
import pytest
import torch

import activation_epilogue_amd as fl
from activation_epilogue_amd import synth
from gpu_util import say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a device"
    fl.load_library()


def test_two_threads_two_streams():
    jobs = [("f16", "glu", (300, 520, 200), 81), ("bf16", "gelu_tanh", (513, 264, 1000), 82)]
    data, refs = [], []
    for dt, act, (M, N, K), seed in jobs:
        d = synth.draw(M, N, K, dt, act, seed=seed)
        dev = {k: to_dev(d[k], dt) for k in ("A", "B", "bias", "Y")}
        ref = fl.fused_linear(dev["A"], dev["B"], dev["bias"], dev["Y"], act=act)
        torch.cuda.synchronize()
        data.append(dev)
        refs.append(to_host(ref, dt))
    outs = [[None] * 20 for _ in jobs]
    errors = []
    start = threading.Barrier(len(jobs))

    def worker(i):
        try:
            dt, act, (M, N, K), _ = jobs[i]
            dev = data[i]
            stream = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(stream):
                for r in range(20):
                    outs[i][r] = fl.fused_linear(dev["A"], dev["B"], dev["bias"], dev["Y"], act=act)
            stream.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    say("two threads, two streams")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (dt, _, _, _) in enumerate(jobs):
        for r, o in enumerate(outs[i]):
            assert np.array_equal(to_host(o, dt).view(np.uint16), refs[i].view(np.uint16)), f"job {i} call {r}"
