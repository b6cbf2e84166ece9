"""softmax_fwd_noalloc, the forward entry point that allocates no device
memory, against the entry point whose kernels it shares.

Shapes that the dispatcher sends to split-k run the two-launch split-k on
partials held in the library's file-scope scratch array; the existing entry
point runs the same kernels (softmax_fwd_kernel with RWS_KERNEL_SPLITK) on
its own workspace, so the two outputs must be bit-identical, and both are
within the oracle's tolerance.  Calls follow one another on one stream, the
second with a smaller input than the first (the array keeps the last call's
contents); a shape whose partials exceed the array runs in row batches; a
row needing more than the whole array is rejected before any launch; a
shape outside split-k takes the plain forward path.
"""
import numpy as np
import pytest
import torch

import oracle
import row_wise_safe_amd as rws
from gpu_util import have_gpu, to_device
from tolerance import check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")]

SCRATCH_PAIRS = (512 << 10) // 8  # (m, d) pairs the scratch holds


@pytest.fixture(scope="module", autouse=True)
def _lib():
    rws.load_library()
    yield


def _noalloc(x, out):
    st = rws.softmax_fwd_noalloc(x.data_ptr(), out.data_ptr(), x.shape[0], x.shape[1],
                                 rws.dtype_code(x.dtype), torch.cuda.current_stream().cuda_stream)
    assert st == rws.RWS_OK, rws.softmax_last_error()
    return out


def _existing(x, kernel):
    out = torch.empty_like(x)
    st = rws.softmax_fwd_kernel(x.data_ptr(), out.data_ptr(), x.shape[0], x.shape[1],
                                rws.dtype_code(x.dtype), torch.cuda.current_stream().cuda_stream,
                                rws.KERNEL_IDS[kernel])
    assert st == rws.RWS_OK, rws.softmax_last_error()
    return out


def _pairs(rows, cols, x):
    desc = rws.softmax_describe_launch(rows, cols, rws.dtype_code(x.dtype), x.data_ptr(),
                                       x.data_ptr(), rws.KERNEL_IDS["splitk"])
    return rows * int(desc.split(" P=")[1].split()[0])


def test_two_calls_in_a_row_second_smaller():
    cases = [((16, 1 << 20), "f16", 3.0), ((4, 300001), "f32", 2.0), ((64, 5000), "bf16", 4.0)]
    for i, ((rows, cols), dtype, sigma) in enumerate(cases):
        print(f"noalloc call {i}: {dtype} [{rows},{cols}]", flush=True)
        x64 = np.random.Generator(np.random.PCG64(900 + i)).normal(0.0, sigma, (rows, cols))
        x, xs = to_device(x64, dtype, offset=i)  # the second call's rows are unaligned
        auto = rws.softmax_select_kernel(rows, cols, rws.dtype_code(x.dtype), x.data_ptr(),
                                         x.data_ptr())
        split = rws.softmax_kernel_name(auto).startswith("splitk")
        out = torch.full_like(x, float("nan"))
        _noalloc(x, out)
        ref_out = _existing(x, "splitk" if split else "auto")
        torch.cuda.synchronize()
        iv = torch.int16 if out.element_size() == 2 else torch.int32
        assert torch.equal(out.view(iv), ref_out.view(iv))
        check(out.double().cpu().numpy(), oracle.safe_softmax(xs), dtype,
              f"noalloc {dtype} [{rows},{cols}]")
        if i < 2:
            assert split, "the first two calls take the split-k path"


def test_rows_in_batches_that_fit_the_scratch():
    # 300 rows of 4M bf16 columns: 256 chunks per row, 76800 partials, more
    # than the scratch holds -> two batches; seeded on the device
    rows, cols = 300, 1 << 22
    g = torch.Generator(device="cuda")
    g.manual_seed(20260905)
    x = torch.randn(rows, cols, generator=g, device="cuda", dtype=torch.float32).mul_(3.0)
    x = x.to(torch.bfloat16)
    assert _pairs(rows, cols, x) > SCRATCH_PAIRS
    print(f"noalloc batches: bf16 [{rows},{cols}]", flush=True)
    out = torch.full_like(x, float("nan"))
    _noalloc(x, out)
    ref_out = _existing(x, "splitk")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    for r in (0, 1, 255, 256, 257, 299):  # both sides of the batch boundary
        xs = x[r:r + 1].double().cpu().numpy()
        check(out[r:r + 1].double().cpu().numpy(), oracle.safe_softmax(xs), "bf16", f"row {r}")
    del x, out, ref_out
    torch.cuda.empty_cache()


def test_plain_forward_shapes_match_softmax_fwd():
    # a line-aligned shape (wave_row) and one of short unaligned rows (tile_rows)
    for seed, (rows, cols) in ((910, (4096, 512)), (911, (1000, 250))):
        x, xs = to_device(np.random.Generator(np.random.PCG64(seed)).normal(0, 8, (rows, cols)),
                          "f16")
        out = _noalloc(x, torch.empty_like(x))
        ref_out = _existing(x, "auto")
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        check(out.double().cpu().numpy(), oracle.safe_softmax(xs), "f16",
              f"noalloc [{rows},{cols}]")


def test_rows_longer_than_the_scratch_are_rejected():
    # fp32 rows of 2^30 columns: 131072 chunks of 2048 granules per row, 1 MiB
    # of partials per row; rejected before any launch (the tensor is real,
    # so a launch could not fault even if the check were missing)
    x = torch.empty(1, 1 << 30, dtype=torch.float32, device="cuda")
    st = rws.softmax_fwd_noalloc(x.data_ptr(), x.data_ptr(), 1, 1 << 30, rws.RWS_F32,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == rws.RWS_ERR_UNSUPPORTED_SHAPE
    assert "scratch" in rws.softmax_last_error()
    torch.cuda.synchronize()
    del x
    torch.cuda.empty_cache()
