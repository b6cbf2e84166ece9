"""Fused single-launch split-k (each workgroup keeps its chunk in registers
and waits for its row's partials): epochs across many calls, streams and
shapes, grids larger than the device holds at once (rows then follow in
dispatch order), the refusal of a row whose workgroups cannot all be
resident, the dispatcher's choice of it, and the workspace
allocation-failure path (forced from the host)."""
import os

import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
from gpu_util import FreshStream, have_gpu, to_device
from tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]


def _x(rows, cols, seed, dtype="f16", offset=0):
    x64 = np.random.Generator(np.random.PCG64(seed)).normal(0.0, 3.0, (rows, cols))
    return to_device(x64, dtype, offset=offset)


def test_many_calls_varying_shapes_one_stream():
    shapes = [(8, 300000), (5, 70001), (16, 1 << 20), (1, 4096 * 8 + 3), (8, 300000), (3, 9999)]
    cases = []
    for i, (r, c) in enumerate(shapes):
        x, stored = _x(r, c, seed=i, offset=i % 2)
        cases.append((x, stored, torch.empty_like(x)))
    torch.cuda.synchronize()
    # enqueue everything back to back (counters and epochs must carry over)
    for rep in range(3):
        for x, _, y in cases:
            rws.softmax(x, out=y, kernel="splitk_fused")
    torch.cuda.synchronize()
    for (x, stored, y), (r, c) in zip(cases, shapes):
        check(y.double().cpu().numpy(), oracle.safe_softmax(stored), "f16", f"fused {r}x{c}")


def test_two_streams_interleaved():
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    xa, sa = _x(16, 200000, seed=10)
    xb, sb = _x(9, 150001, seed=11, dtype="bf16")
    ya, yb = torch.empty_like(xa), torch.empty_like(xb)
    torch.cuda.synchronize()
    for _ in range(5):
        with torch.cuda.stream(s1):
            rws.softmax(xa, out=ya, kernel="splitk_fused")
        with torch.cuda.stream(s2):
            rws.softmax(xb, out=yb, kernel="splitk_fused")
    torch.cuda.synchronize()
    check(ya.double().cpu().numpy(), oracle.safe_softmax(sa), "f16", "stream 1")
    check(yb.double().cpu().numpy(), oracle.safe_softmax(sb), "bf16", "stream 2")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_fused_matches_two_launch(dtype):
    x, stored = _x(6, 500001, seed=12, dtype=dtype, offset=1)
    a = rws.softmax(x, kernel="splitk_fused")
    b = rws.softmax(x, kernel="splitk")
    torch.cuda.synchronize()
    ref = oracle.safe_softmax(stored)
    check(a.double().cpu().numpy(), ref, dtype, "fused")
    check(b.double().cpu().numpy(), ref, dtype, "two-launch")


def test_refuses_row_that_cannot_be_co_resident():
    # fp32 rows of 20M elements: 5M granules a row, more than any variant's
    # resident workgroups hold at once (at most 4M granules); refused before
    # any launch
    x = torch.zeros(1, 20 << 20, dtype=torch.float32, device="cuda")
    with pytest.raises(rws.SoftmaxError) as e:
        rws.softmax(x, kernel="splitk_fused")
    assert e.value.status == rws.RWS_ERR_UNSUPPORTED_SHAPE
    # the dispatcher takes the two launches for such a row
    assert rws.softmax_kernel_name(
        rws.softmax_select_kernel(1, 20 << 20, rws.RWS_F32, x.data_ptr(), x.data_ptr())) \
        == "splitk"


def test_grid_larger_than_the_device_runs_row_by_row():
    # 48 rows of 1M fp16 (96 MiB): 1536 workgroups of 64 KiB, more than the
    # 1024 the device holds at once; later rows start as earlier rows finish
    rows, cols = 48, 1 << 20
    x, stored = _x(rows, cols, seed=14)
    desc = rws.softmax_describe_launch(rows, cols, rws.RWS_F16, x.data_ptr(), x.data_ptr(),
                                       rws.KERNEL_IDS["splitk_fused"])
    print(f"\n{desc}", flush=True)
    assert "grid=1536 " in desc, desc
    y = torch.empty_like(x)
    with FreshStream() as s:
        with torch.cuda.stream(s):
            rws.softmax(x, out=y, kernel="splitk_fused")
            rws.stream_status()
    check(y.double().cpu().numpy(), oracle.safe_softmax(stored), "f16", "fused, two passes")


@pytest.mark.parametrize("rows,cols,family", [
    (4, 1 << 23, "splitk_fused"),      # 64 MiB: the whole grid fits at once
    (32, 1 << 20, "splitk_fused"),     # 64 MiB
    (4, 1 << 20, "splitk_fused"),      # at most four rows
    (16, 1 << 20, "splitk_ordered"),   # 32 MiB, sixteen rows
    (4, 1 << 25, "splitk"),            # 256 MiB: more than the device holds
])
def test_dispatcher_choice_on_the_device(rows, cols, family):
    # the occupancy the device reports, not the compiled lower bound
    kid = rws.softmax_select_kernel(rows, cols, rws.RWS_F16, 256, 512)
    assert rws.softmax_kernel_name(kid) == family


def test_workspace_allocation_failure_is_reported():
    s = torch.cuda.Stream()  # a stream with no workspace yet
    x, stored = _x(4, 400000, seed=13)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    os.environ["RWS_TEST_FAIL_ALLOC"] = "1"
    try:
        st = rws.softmax_fwd_kernel(x.data_ptr(), y.data_ptr(), 4, 400000, rws.RWS_F16,
                                    int(s.cuda_stream), rws.KERNEL_IDS["splitk"])
        assert st == rws.RWS_ERR_HIP
        assert "workspace" in rws.softmax_last_error()
    finally:
        del os.environ["RWS_TEST_FAIL_ALLOC"]
    with torch.cuda.stream(s):
        rws.softmax(x, out=y, kernel="splitk")
    s.synchronize()
    check(y.double().cpu().numpy(), oracle.safe_softmax(stored), "f16", "after failure")
