"""Ordered single-launch split-k: epoch-tagged partials across many calls,
shapes, streams and launch batches, the 32-bit epoch wrap (started near it
through a host-side test hook), in-place calls, agreement with the two-launch
form, and the workspace allocation-failure path (forced from the host).
Every result is checked against the CPU oracle."""
import os

import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
import workloads
from gpu_util import FreshStream, have_gpu, to_device
from tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]


def _x(rows, cols, seed, dtype="f16", offset=0):
    x64 = np.random.Generator(np.random.PCG64(seed)).normal(0.0, 3.0, (rows, cols))
    return to_device(x64, dtype, offset=offset)


def _describe(x, kernel="splitk_ordered"):
    return rws.softmax_describe_launch(x.shape[0], x.shape[1], rws.dtype_code(x.dtype),
                                       x.data_ptr(), x.data_ptr(), rws.KERNEL_IDS[kernel])


def test_workload_uses_ordered_form():
    w = workloads.WORKLOADS["fp16_16x1M"]
    desc = rws.softmax_describe_launch(w.rows, w.cols, rws.RWS_F16, 256, 256)
    assert desc.startswith("splitk_ordered"), desc


def test_many_calls_varying_shapes_one_stream():
    # back-to-back calls of different shapes and chunk counts reuse the same
    # tag words: only the epoch tells one call's partials from another's
    shapes = [(8, 300000), (5, 70001), (16, 1 << 20), (1, 4096 * 8 + 3), (8, 300000), (3, 9999),
              (40, 50000)]
    cases = []
    for i, (r, c) in enumerate(shapes):
        x, stored = _x(r, c, seed=100 + i, offset=i % 2)
        cases.append((x, stored, torch.empty_like(x)))
    torch.cuda.synchronize()
    for _ in range(3):
        for x, _, y in cases:
            rws.softmax(x, out=y, kernel="splitk_ordered")
    torch.cuda.synchronize()
    for (x, stored, y), (r, c) in zip(cases, shapes):
        check(y.double().cpu().numpy(), oracle.safe_softmax(stored), "f16",
              f"ordered {r}x{c}: {_describe(x)}")


def test_two_streams_interleaved():
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    xa, sa = _x(16, 200000, seed=110)
    xb, sb = _x(9, 150001, seed=111, dtype="bf16")
    ya, yb = torch.empty_like(xa), torch.empty_like(xb)
    torch.cuda.synchronize()
    for _ in range(5):
        with torch.cuda.stream(s1):
            rws.softmax(xa, out=ya, kernel="splitk_ordered")
        with torch.cuda.stream(s2):
            rws.softmax(xb, out=yb, kernel="splitk_ordered")
    torch.cuda.synchronize()
    check(ya.double().cpu().numpy(), oracle.safe_softmax(sa), "f16", "stream 1")
    check(yb.double().cpu().numpy(), oracle.safe_softmax(sb), "bf16", "stream 2")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_matches_two_launch(dtype):
    # unaligned rows (offset 1): partial granules at every chunk edge
    x, stored = _x(6, 500001, seed=112, dtype=dtype, offset=1)
    a = rws.softmax(x, kernel="splitk_ordered")
    b = rws.softmax(x, kernel="splitk")
    torch.cuda.synchronize()
    ref = oracle.safe_softmax(stored)
    check(a.double().cpu().numpy(), ref, dtype, "ordered")
    check(b.double().cpu().numpy(), ref, dtype, "two-launch")


def test_in_place():
    x, stored = _x(16, 1 << 20, seed=113)
    rws.softmax(x, out=x, kernel="splitk_ordered")
    torch.cuda.synchronize()
    check(x.double().cpu().numpy(), oracle.safe_softmax(stored), "f16", "in place")


def test_several_launches_in_one_call():
    # one granule per row: P = 1, so a launch takes 2^22 rows (2^23
    # workgroups over both stages); 2^22 + 3 rows need two launches, which
    # reuse the tag words under two epochs
    rows = (1 << 22) + 3
    x, stored = _x(rows, 8, seed=114)
    d = _describe(x)
    assert "P=1 " in d, d
    y = rws.softmax(x, kernel="splitk_ordered")
    torch.cuda.synchronize()
    err = np.abs(y.double().cpu().numpy() - oracle.safe_softmax(stored)).max()
    assert err <= 1e-3, f"max abs error {err:.3e}"


def test_epoch_wrap():
    # A fresh stream gets a fresh tag buffer whose host epochs start 5 below
    # the end of their range [1, 2^31) (test hook read at allocation); 12
    # calls cross the end, where the library zeroes the words and restarts at
    # epoch 1.
    shapes = [(16, 65536 + 7), (4, 200000), (16, 65536 + 7)]
    cases = []
    for i, (r, c) in enumerate(shapes):
        x, stored = _x(r, c, seed=120 + i)
        cases.append((x, stored, oracle.safe_softmax(stored)))
    torch.cuda.synchronize()
    os.environ["RWS_TEST_TAG_EPOCH"] = str(0x7FFFFFFF - 5)
    try:
        with FreshStream() as s:
            for k in range(12):
                x, _, ref = cases[k % len(cases)]
                y = torch.empty_like(x)
                with torch.cuda.stream(s):
                    rws.softmax(x, out=y, kernel="splitk_ordered")
                s.synchronize()
                check(y.double().cpu().numpy(), ref, "f16", f"call {k} across the epoch wrap")
    finally:
        del os.environ["RWS_TEST_TAG_EPOCH"]


def test_workspace_allocation_failure_is_reported():
    x, stored = _x(4, 400000, seed=130)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    with FreshStream() as s:  # a stream with no workspace yet
        os.environ["RWS_TEST_FAIL_ALLOC"] = "1"
        try:
            st = rws.softmax_fwd_kernel(x.data_ptr(), y.data_ptr(), 4, 400000, rws.RWS_F16,
                                        int(s.cuda_stream), rws.KERNEL_IDS["splitk_ordered"])
            assert st == rws.RWS_ERR_HIP
            assert "workspace" in rws.softmax_last_error()
        finally:
            del os.environ["RWS_TEST_FAIL_ALLOC"]
        with torch.cuda.stream(s):
            rws.softmax(x, out=y, kernel="splitk_ordered")
        s.synchronize()
        check(y.double().cpu().numpy(), oracle.safe_softmax(stored), "f16", "after failure")


def test_ordered_only_up_to_its_limits():
    # the ordered form from eight rows while the input fits 32 MiB and a row
    # needs at most 512 chunks; past that, the fused single launch while its
    # whole grid fits the device at once, else the two launches
    def family(rows, cols):
        return rws.softmax_describe_launch(rows, cols, rws.RWS_F16, 256, 256).split("<")[0]
    assert family(16, 1 << 20) == "splitk_ordered"
    assert family(8, 1 << 21) == "splitk_ordered"    # 32 MiB, P = 256
    assert family(2, 1 << 23) == "splitk_fused"      # P = 1024
    assert family(16, 1 << 21) == "splitk_fused"     # 64 MiB
    assert family(2, 1 << 25) == "splitk"            # 128 MiB
    assert family(1, 1 << 28) == "splitk"            # 512 MiB
