"""Host threads sharing the library: two threads enqueue split-k calls on one
stream at the same moment while the stream's workspace grows (a fresh stream
per round, so every round starts with an empty workspace).  The library keeps
a stream's workspace locked from its lookup until the call's launches are
enqueued, so the growing call can only free the old buffer once the other
call's kernels are on the stream ahead of it.  Both results are checked
against the oracle every round.  (ctypes releases the GIL during the calls,
so the two threads do run the library concurrently.)"""
import threading

import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
import workloads
from gpu_util import have_gpu, to_device

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]


@pytest.mark.parametrize("kernel", ["splitk", "splitk_ordered"])
def test_two_threads_one_stream_while_the_workspace_grows(kernel):
    xa, xsa = to_device(workloads.argmax_moved_normal(4, 1 << 17, 901), "f16")
    xb, xsb = to_device(workloads.argmax_moved_normal(32, 1 << 19, 902), "f16")
    ref_a = oracle.safe_softmax(xsa)
    ref_b = oracle.safe_softmax(xsb)
    for rnd in range(12):
        s = torch.cuda.Stream()
        ya, yb = torch.empty_like(xa), torch.empty_like(xb)
        torch.cuda.synchronize()  # inputs were written on the default stream
        barrier = threading.Barrier(2)
        errors = []

        def call(x, y):
            try:
                barrier.wait()
                rws.softmax(x, out=y, kernel=kernel, stream=s)
            except Exception as e:  # reported below
                errors.append(e)

        order = [(xa, ya), (xb, yb)] if rnd % 2 == 0 else [(xb, yb), (xa, ya)]
        threads = [threading.Thread(target=call, args=a) for a in order]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        s.synchronize()
        assert not errors, errors
        for y, ref, name in ((ya, ref_a, "small"), (yb, ref_b, "large")):
            err = np.abs(y.to(torch.float64).cpu().numpy() - ref).max()
            assert err <= 1e-3, f"round {rnd} {name}: max abs error {err:.3e}"
