"""Re-entrancy of the C ABI: several host threads, each with its own stream
and its own buffers, call the layer and the dense projection at the same time
(the binding's ctypes calls release the interpreter lock, so the library runs
concurrently, including its first-use device queries); every thread's results
equal the single-threaded ones bit for bit."""
import threading

import numpy as np
import pytest
import torch

import fp4_routed_expert_amd as moe
import synth
from gpu_cases import get_case, to_dev

pytestmark = pytest.mark.gpu

THREADS = 4


def test_concurrent_threads_match_sequential(dev):
    c = get_case("c0", dev)
    sh = c.sh
    d = synth.make_dense_inputs("d0", T=150, K=384, N=288)
    dw = moe.dense_prepack(to_dev(d.wq, dev), to_dev(d.ws, dev))
    dx = to_dev(d.x.view(np.int16), dev).view(torch.bfloat16)
    flags = [0, moe.MOE_FLAG_FORCE_DECODE, moe.MOE_FLAG_FORCE_PREFILL]
    torch.cuda.synchronize()

    # the threads run first, so in a fresh process their calls are also the
    # library's first ones on the device; the single-threaded results after
    out = [None] * THREADS
    errors = []
    start = threading.Barrier(THREADS)

    def work(i):
        try:
            s = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(s):
                start.wait()
                ys = []
                for rep in range(3):
                    f = flags[(i + rep) % len(flags)]
                    ys.append((f, moe.layer_forward(c.pw, c.x, c.logits, sh.k, f)))
                yd = moe.dense_layer(dw, dx)
            s.synchronize()
            out[i] = (ys, yd)
        except Exception as e:  # reported below, on the test's thread
            errors.append(repr(e))

    th = [threading.Thread(target=work, args=(i,)) for i in range(THREADS)]
    for t in th:
        t.start()
    for t in th:
        t.join(timeout=120)
    assert not errors, errors
    ref_y = {f: moe.layer_forward(c.pw, c.x, c.logits, sh.k, f) for f in flags}
    ref_d = moe.dense_layer(dw, dx)
    torch.cuda.synchronize()
    for i in range(THREADS):
        ys, yd = out[i]
        for f, y in ys:
            assert torch.equal(y, ref_y[f]), f"thread {i} flags {f}"
        assert torch.equal(yd.view(torch.int16), ref_d.view(torch.int16)), f"thread {i} dense"
